// Router: per-token expert scores and (group-limited) top-k on the GPU.
//
// MegaMoE (ROCm Primus technical guide), introduction: the routed-expert path starts from a
// router made of a score function and a group-limited top-k. Primus, "Router force load
// balancing", `uniform`: benchmark routing draws random logits and routes them. Readings (the
// pages give no formulas):
//   * score: softmax over the token's E logits, or the logistic sigmoid of each logit. Both grow
//     with the expert's own logit, so the K best-scored experts are the K largest logits: the
//     selection compares logits, never rounded scores (ties go to the lower expert id; NaN ranks
//     below every number);
//   * group limit: experts form n_group equal groups of consecutive ids, a group ranks by its
//     largest logit (ties: lower group), the topk_group best groups stay, and the K experts are
//     chosen among their experts;
//   * weights: the chosen experts' scores (softmax over all E, or sigmoid), optionally divided by
//     their sum over the K chosen; ids and weights come out in selection order.
//
// One wavefront per token; lane l holds the logits of experts l, l+64, ... (NV per lane: the
// kernel is compiled for NV = 1, 2, 4, 8, 16, i.e. E up to 64, 128, 256, 512, 1024, so that its
// registers, and with them the number of tokens in flight, follow E). Every candidate is a 64-bit
// key, (order-preserving image of the logit) << 32 | (~expert id), so "larger key" is exactly
// "ranks first" and one wavefront max per pick selects the next expert; candidates outside the
// kept groups or already chosen have key 0. The group ranking goes through LDS (dynamic, only
// when there are groups).
#include <type_traits>

#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kRouteWaves = 4;  // tokens per 256-thread workgroup

// order-preserving map of a float to 32 bits: larger float -> larger key, equal floats (+0 and
// -0 included) -> equal keys; NaN -> 0 (below all)
__device__ __forceinline__ uint32_t order_key(float v) {
  const uint32_t u = __float_as_uint(v);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0u;
  if ((u & 0x7fffffffu) == 0u) return 0x80000000u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)v, off);
    const uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(v >> 32), off);
    const uint64_t o = ((uint64_t)hi << 32) | lo;
    v = o > v ? o : v;
  }
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

__device__ __forceinline__ float wave_max_f(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  return v;
}

template <typename IdT, int NV>
__global__ __launch_bounds__(256) void moe_route_topk(const float* __restrict__ logits, int T,
                                                    int E, int K, int score_fn, int renorm,
                                                    int n_group, int topk_group,
                                                    IdT* __restrict__ ids,
                                                    float* __restrict__ weights) {
  extern __shared__ uint64_t skeys_all[];  // [kRouteWaves][NV * 64] when n_group > 1
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int t = blockIdx.x * kRouteWaves + w;
  if (t >= T) return;
  const float* lt = logits + (int64_t)t * E;
  const int nv = (E + 63) / 64;
  uint64_t* skeys = skeys_all + w * (NV * 64);

  uint64_t key[NV];
  float val[NV];
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int e = j * 64 + lane;
    val[j] = 0.0f;
    key[j] = 0;
    if (j < nv && e < E) {
      val[j] = lt[e];
      key[j] = ((uint64_t)order_key(val[j]) << 32) | (uint32_t)(0xffffffffu - (uint32_t)e);
    }
  }

  if (n_group > 1) {
    // group ranking through LDS: lane g < n_group scans its group's keys
    const int gs = E / n_group;
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int e = j * 64 + lane;
      if (j < nv && e < E) skeys[e] = key[j];
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    uint64_t gk = 0;
    if (lane < n_group) {
      uint64_t best = 0;
      for (int e = lane * gs; e < (lane + 1) * gs; ++e) best = skeys[e] > best ? skeys[e] : best;
      // a group ranks by its best logit (high half of its best key), then by the lower group id
      gk = (best & 0xffffffff00000000ull) | (uint32_t)(0xffffffffu - (uint32_t)lane);
    }
    uint64_t kept = 0;  // bit g: group g kept
    for (int r = 0; r < topk_group; ++r) {
      const uint64_t m = wave_max_u64(gk);
      const int g = (int)(0xffffffffu - (uint32_t)m);
      kept |= 1ull << g;
      if (lane == g) gk = 0;
    }
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int e = j * 64 + lane;
      if (j < nv && e < E && !((kept >> (e / gs)) & 1ull)) key[j] = 0;
    }
  }

  // K picks; lane k remembers pick k
  int my_id = 0;
  for (int k = 0; k < K; ++k) {
    uint64_t best = 0;
#pragma unroll
    for (int j = 0; j < NV; ++j) best = key[j] > best ? key[j] : best;
    const uint64_t m = wave_max_u64(best);
    const int e = (int)(0xffffffffu - (uint32_t)m);
    if (lane == k) my_id = e;
#pragma unroll
    for (int j = 0; j < NV; ++j)  // the owner drops it
      if (j == (e >> 6) && (e & 63) == lane) key[j] = 0;
  }

  // weights
  const bool mine = lane < K;
  const float lk = mine ? lt[my_id] : 0.0f;
  float wk;
  if (score_fn == MOE_SCORE_SOFTMAX) {
    float m, z;
    if (renorm) {
      m = wave_max_f(mine ? lk : -INFINITY);
      z = wave_sum(mine ? expf(lk - m) : 0.0f);
    } else {
      float lm = -INFINITY;
#pragma unroll
      for (int j = 0; j < NV; ++j)
        if (j < nv && j * 64 + lane < E) lm = fmaxf(lm, val[j]);
      m = wave_max_f(lm);
      float ls = 0.0f;
#pragma unroll
      for (int j = 0; j < NV; ++j)
        if (j < nv && j * 64 + lane < E) ls += expf(val[j] - m);
      z = wave_sum(ls);
    }
    wk = expf(lk - m) / z;
  } else {
    const float s = 1.0f / (1.0f + expf(-lk));
    if (renorm) {
      const float z = wave_sum(mine ? s : 0.0f);
      wk = s / z;
    } else {
      wk = s;
    }
  }
  if (mine) {
    ids[(int64_t)t * K + lane] = (IdT)my_id;
    weights[(int64_t)t * K + lane] = wk;
  }
}

}  // namespace

hipError_t launch_route(const moe_shape& s, const moe_router& r, const float* logits, void* ids,
                        float* weights, hipStream_t st) {
  const int T = (int)s.T;
  const dim3 grid((T + kRouteWaves - 1) / kRouteWaves);
  const int ng = r.n_group > 1 ? r.n_group : 1;
  const int tg = r.n_group > 1 ? r.topk_group : 1;
  const int E = (int)s.E, nv = (E + 63) / 64;
  const int NV = nv <= 1 ? 1 : nv <= 2 ? 2 : nv <= 4 ? 4 : nv <= 8 ? 8 : 16;  // E <= 1024
  const size_t lds = ng > 1 ? sizeof(uint64_t) * kRouteWaves * NV * 64 : 0;
  auto go = [&](auto idt, auto nv_tag) {
    using IdT = decltype(idt);
    constexpr int N = decltype(nv_tag)::value;
    hipLaunchKernelGGL((moe_route_topk<IdT, N>), grid, dim3(256), lds, st, logits, T, E,
                       (int)s.K, r.score_fn, r.renormalize, ng, tg, (IdT*)ids, weights);
  };
  auto by_nv = [&](auto idt) {
    switch (NV) {
      case 1: go(idt, std::integral_constant<int, 1>{}); break;
      case 2: go(idt, std::integral_constant<int, 2>{}); break;
      case 4: go(idt, std::integral_constant<int, 4>{}); break;
      case 8: go(idt, std::integral_constant<int, 8>{}); break;
      default: go(idt, std::integral_constant<int, 16>{}); break;
    }
  };
  if (s.ids_dtype == MOE_IDS_I64)
    by_nv(int64_t{});
  else
    by_nv(int32_t{});
  return hipGetLastError();
}

}  // namespace moe
