// Row kernels between token order and expert-grouped order (HBM-bound copies and reductions).
//
//   permute      xg[pos[t,k]] = x[t]   -- TeraMoE README, dispatch worker (writes the expert
//                inputs); MoonEP FAQ (tokens written straight into expert-grouped positions).
//                Token-major: each token row is read once and written K times.
//   combine      out[t] = bf16(sum_k w_k * y[pos[t,k]]), k ascending, fp32, no atomics --
//                TeraMoE combine worker (weighted accumulation) and gather worker (several
//                results of one token reduced locally). With unit weights it is the dX reduction.
//   combine_bwd  dy[pos[t,k]] = bf16(s[t,k] * dout[t]) and dscores[t,k] = <dout[t], y[pos[t,k]]>
//                -- the transpose of combine and the derivative with respect to the scores.
//                dout[t] is read once per group of 8 slots.
//
// One wavefront per token; every lane moves 16-byte chunks (8 bf16), so one wavefront instruction
// touches 1 KiB of a row. The K slots of a token are the same for every lane of its wavefront, so
// a dropped slot (pos < 0) skips its work for the whole wavefront. For K in {1, 2, 4, 6, 8} the
// combine kernels are compiled for that K and issue the row loads of all slots of a chunk
// together; other K take the slots one at a time.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kRowWaves = 4;  // tokens per 256-thread workgroup

__device__ __forceinline__ void unpack8(const uint4& v, float* f) {
  f[0] = bf16_to_f32(v.x & 0xffffu); f[1] = bf16_to_f32(v.x >> 16);
  f[2] = bf16_to_f32(v.y & 0xffffu); f[3] = bf16_to_f32(v.y >> 16);
  f[4] = bf16_to_f32(v.z & 0xffffu); f[5] = bf16_to_f32(v.z >> 16);
  f[6] = bf16_to_f32(v.w & 0xffffu); f[7] = bf16_to_f32(v.w >> 16);
}

// 16-byte load with the non-temporal hint, for the rows the combines gather and read exactly once
// (on MI355X it lifts the combine from about 62% to about 71% of the HBM peak; the permute, whose
// token rows are read once too, is about 5% slower with it and reads plainly)
__device__ __forceinline__ uint4 load_once(const uint4* p) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 v = __builtin_nontemporal_load((const u32x4*)p);
  return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ uint4 pack8(const float* f) {
  return make_uint4(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]),
                    pack_bf16x2(f[6], f[7]));
}

__global__ __launch_bounds__(256) void moe_permute(const uint4* __restrict__ x,
                                                 const int32_t* __restrict__ pos,
                                                 uint4* __restrict__ xg, int T, int K, int nch) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * kRowWaves + (threadIdx.x >> 6);
  if (t >= T) return;
  const uint4* xr = x + (int64_t)t * nch;
  const int32_t* pt = pos + (int64_t)t * K;
  int c = lane;
  for (; c + 192 < nch; c += 256) {
    const uint4 v0 = xr[c], v1 = xr[c + 64], v2 = xr[c + 128], v3 = xr[c + 192];
    for (int k = 0; k < K; ++k) {
      const int p = pt[k];
      if (p < 0 || !MOE_CHECK(p < T * K)) continue;
      uint4* dst = xg + (int64_t)p * nch + c;
      dst[0] = v0; dst[64] = v1; dst[128] = v2; dst[192] = v3;
    }
  }
  for (; c < nch; c += 64) {
    const uint4 v = xr[c];
    for (int k = 0; k < K; ++k) {
      const int p = pt[k];
      if (p >= 0 && MOE_CHECK(p < T * K)) xg[(int64_t)p * nch + c] = v;
    }
  }
}

// KT > 0: K == KT at compile time, so the loads of all K slots of a chunk are issued together
// (a dropped slot loads row 0 and is skipped in the sum); KT == 0: any K, one slot at a time.
template <bool WEIGHTED, int KT>
__global__ __launch_bounds__(256) void moe_combine(const uint4* __restrict__ rows,
                                                 const int32_t* __restrict__ pos,
                                                 const float* __restrict__ scores,
                                                 uint4* __restrict__ out, int T, int K_, int nch) {
  const int K = KT > 0 ? KT : K_;
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * kRowWaves + (threadIdx.x >> 6);
  if (t >= T) return;
  const int32_t* pt = pos + (int64_t)t * K;
  const float* st = WEIGHTED ? scores + (int64_t)t * K : nullptr;
  int c = lane;
  if constexpr (KT > 0) {
    int pk[KT];
    float wk[KT];
#pragma unroll
    for (int k = 0; k < KT; ++k) {
      pk[k] = pt[k];
      if (pk[k] >= 0 && !MOE_CHECK(pk[k] < T * K)) pk[k] = -1;
      wk[k] = WEIGHTED ? st[k] : 1.0f;
    }
    for (; c + 64 < nch; c += 128) {
      uint4 v0[KT], v1[KT];
#pragma unroll
      for (int k = 0; k < KT; ++k) {
        const uint4* r = rows + (int64_t)(pk[k] < 0 ? 0 : pk[k]) * nch + c;
        v0[k] = load_once(r);
        v1[k] = load_once(r + 64);
      }
      float a0[8] = {0, 0, 0, 0, 0, 0, 0, 0}, a1[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
      for (int k = 0; k < KT; ++k) {
        if (pk[k] < 0) continue;
        float f0[8], f1[8];
        unpack8(v0[k], f0);
        unpack8(v1[k], f1);
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          a0[q] += wk[k] * f0[q];
          a1[q] += wk[k] * f1[q];
        }
      }
      out[(int64_t)t * nch + c] = pack8(a0);
      out[(int64_t)t * nch + c + 64] = pack8(a1);
    }
  } else {
    for (; c + 64 < nch; c += 128) {
      float a0[8] = {0, 0, 0, 0, 0, 0, 0, 0}, a1[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      for (int k = 0; k < K; ++k) {
        const int p = pt[k];
        if (p < 0 || !MOE_CHECK(p < T * K)) continue;
        const float w = WEIGHTED ? st[k] : 1.0f;
        const uint4* r = rows + (int64_t)p * nch + c;
        const uint4 v0 = load_once(r), v1 = load_once(r + 64);
        float f0[8], f1[8];
        unpack8(v0, f0);
        unpack8(v1, f1);
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          a0[q] += w * f0[q];
          a1[q] += w * f1[q];
        }
      }
      out[(int64_t)t * nch + c] = pack8(a0);
      out[(int64_t)t * nch + c + 64] = pack8(a1);
    }
  }
  for (; c < nch; c += 64) {
    float a0[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int k = 0; k < K; ++k) {
      const int p = pt[k];
      if (p < 0 || !MOE_CHECK(p < T * K)) continue;
      const float w = WEIGHTED ? st[k] : 1.0f;
      float f0[8];
      unpack8(load_once(rows + (int64_t)p * nch + c), f0);
#pragma unroll
      for (int q = 0; q < 8; ++q) a0[q] += w * f0[q];
    }
    out[(int64_t)t * nch + c] = pack8(a0);
  }
}

// One wavefront per token; the K slots are taken in groups of up to 8 (KG) so that each chunk of
// dout[t] is read once per group (once in all for K <= 8) while the slots' y rows stream past it.
// Per slot the dot product accumulates lane-wise over ascending chunks, then across the wavefront.
// KT > 0: K == KT <= KG at compile time, and the y loads of all slots of a chunk are issued
// together (a dropped slot loads row 0 and neither stores nor sums).
template <int KT>
__global__ __launch_bounds__(256) void moe_combine_bwd_dscores(const uint4* __restrict__ dout,
                                                     const uint4* __restrict__ y,
                                                     const int32_t* __restrict__ pos,
                                                     const float* __restrict__ scores,
                                                     uint4* __restrict__ dy,
                                                     float* __restrict__ dscores, int T, int K_,
                                                     int nch) {
  constexpr int KG = 8;
  static_assert(KT <= KG, "one group");
  const int K = KT > 0 ? KT : K_;
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * kRowWaves + (threadIdx.x >> 6);
  if (t >= T) return;
  const uint4* dr = dout + (int64_t)t * nch;
  if constexpr (KT > 0) {
    int pk[KT];
    float sk[KT], part[KT];
#pragma unroll
    for (int j = 0; j < KT; ++j) {
      pk[j] = pos[(int64_t)t * KT + j];
      if (pk[j] >= 0 && !MOE_CHECK(pk[j] < T * K)) pk[j] = -1;
      sk[j] = scores[(int64_t)t * KT + j];
      part[j] = 0.0f;
    }
    for (int c = lane; c < nch; c += 64) {
      uint4 vy[KT];
#pragma unroll
      for (int j = 0; j < KT; ++j) vy[j] = load_once(y + (int64_t)(pk[j] < 0 ? 0 : pk[j]) * nch + c);
      float fd[8];
      unpack8(load_once(dr + c), fd);
#pragma unroll
      for (int j = 0; j < KT; ++j) {
        if (pk[j] < 0) continue;
        float fy[8], o[8];
        unpack8(vy[j], fy);
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          part[j] += fd[q] * fy[q];
          o[q] = sk[j] * fd[q];
        }
        dy[(int64_t)pk[j] * nch + c] = pack8(o);
      }
    }
#pragma unroll
    for (int j = 0; j < KT; ++j) {
      float v = part[j];
      for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
      if (lane == 0) dscores[(int64_t)t * KT + j] = pk[j] < 0 ? 0.0f : v;
    }
    return;
  }
  for (int k0 = 0; k0 < K; k0 += KG) {
    const int kn = K - k0 < KG ? K - k0 : KG;
    int pk[KG];
    float sk[KG], part[KG];
#pragma unroll
    for (int j = 0; j < KG; ++j) {
      pk[j] = j < kn ? pos[(int64_t)t * K + k0 + j] : -1;
      if (pk[j] >= 0 && !MOE_CHECK(pk[j] < T * K)) pk[j] = -1;
      sk[j] = j < kn ? scores[(int64_t)t * K + k0 + j] : 0.0f;
      part[j] = 0.0f;
    }
    for (int c = lane; c < nch; c += 64) {
      float fd[8];
      unpack8(dr[c], fd);
#pragma unroll
      for (int j = 0; j < KG; ++j) {
        if (pk[j] < 0) continue;  // wave-uniform
        float fy[8], o[8];
        unpack8(load_once(y + (int64_t)pk[j] * nch + c), fy);
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          part[j] += fd[q] * fy[q];
          o[q] = sk[j] * fd[q];
        }
        dy[(int64_t)pk[j] * nch + c] = pack8(o);
      }
    }
#pragma unroll
    for (int j = 0; j < KG; ++j) {
      if (j >= kn) break;
      float v = part[j];
      for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
      if (lane == 0) dscores[(int64_t)t * K + k0 + j] = pk[j] < 0 ? 0.0f : v;
    }
  }
}

}  // namespace

hipError_t launch_permute(const moe_shape& s, const int32_t* pos, const uint16_t* x, uint16_t* xg,
                          hipStream_t st) {
  const int T = (int)s.T;
  hipLaunchKernelGGL(moe_permute, dim3((T + kRowWaves - 1) / kRowWaves), dim3(256), 0, st,
                     (const uint4*)x, pos, (uint4*)xg, T, (int)s.K, (int)(s.D / 8));
  return hipGetLastError();
}

template <bool WEIGHTED>
void combine_k(const moe_shape& s, const int32_t* pos, const uint16_t* rows, const float* scores,
               uint16_t* out, hipStream_t st) {
  const int T = (int)s.T, K = (int)s.K, nch = (int)(s.D / 8);
  const dim3 grid((T + kRowWaves - 1) / kRowWaves), block(256);
  const uint4* r = (const uint4*)rows;
  uint4* o = (uint4*)out;
  switch (K) {
    case 1: hipLaunchKernelGGL((moe_combine<WEIGHTED, 1>), grid, block, 0, st, r, pos, scores, o, T, K, nch); break;
    case 2: hipLaunchKernelGGL((moe_combine<WEIGHTED, 2>), grid, block, 0, st, r, pos, scores, o, T, K, nch); break;
    case 4: hipLaunchKernelGGL((moe_combine<WEIGHTED, 4>), grid, block, 0, st, r, pos, scores, o, T, K, nch); break;
    case 6: hipLaunchKernelGGL((moe_combine<WEIGHTED, 6>), grid, block, 0, st, r, pos, scores, o, T, K, nch); break;
    case 8: hipLaunchKernelGGL((moe_combine<WEIGHTED, 8>), grid, block, 0, st, r, pos, scores, o, T, K, nch); break;
    default: hipLaunchKernelGGL((moe_combine<WEIGHTED, 0>), grid, block, 0, st, r, pos, scores, o, T, K, nch); break;
  }
}

hipError_t launch_combine(const moe_shape& s, const int32_t* pos, const uint16_t* rows,
                          const float* scores, uint16_t* out, hipStream_t st) {
  if (scores)
    combine_k<true>(s, pos, rows, scores, out, st);
  else
    combine_k<false>(s, pos, rows, scores, out, st);
  return hipGetLastError();
}

hipError_t launch_combine_bwd(const moe_shape& s, const int32_t* pos, const uint16_t* dout,
                              const uint16_t* y, const float* scores, uint16_t* dy,
                              float* dscores, hipStream_t st) {
  const int T = (int)s.T, K = (int)s.K, nch = (int)(s.D / 8);
  const dim3 grid((T + kRowWaves - 1) / kRowWaves), block(256);
  const uint4 *d = (const uint4*)dout, *yy = (const uint4*)y;
  uint4* o = (uint4*)dy;
  switch (K) {
    case 1: hipLaunchKernelGGL(moe_combine_bwd_dscores<1>, grid, block, 0, st, d, yy, pos, scores, o, dscores, T, K, nch); break;
    case 2: hipLaunchKernelGGL(moe_combine_bwd_dscores<2>, grid, block, 0, st, d, yy, pos, scores, o, dscores, T, K, nch); break;
    case 4: hipLaunchKernelGGL(moe_combine_bwd_dscores<4>, grid, block, 0, st, d, yy, pos, scores, o, dscores, T, K, nch); break;
    case 6: hipLaunchKernelGGL(moe_combine_bwd_dscores<6>, grid, block, 0, st, d, yy, pos, scores, o, dscores, T, K, nch); break;
    case 8: hipLaunchKernelGGL(moe_combine_bwd_dscores<8>, grid, block, 0, st, d, yy, pos, scores, o, dscores, T, K, nch); break;
    default: hipLaunchKernelGGL(moe_combine_bwd_dscores<0>, grid, block, 0, st, d, yy, pos, scores, o, dscores, T, K, nch); break;
  }
  return hipGetLastError();
}

#ifdef MOE_CHECKED
hipError_t oob_counter_rowops(unsigned int** p) { return oob_counter_address(p); }
#endif

}  // namespace moe
