// Grouped GEMMs of the routed-experts layer on bf16 MFMA (gfx950).
//
// Dist-MoE 0.1.0 (PyPI page), "Understand the execution model": FPROP (W13 then W2), DGRAD and
// WGRAD expert GEMMs; "Choose a precision and pipeline / BF16": bf16 operands, fp32 accumulation.
// TeraMoE README, compute worker: gate/up projection, activation, down projection. MegaMoE (ROCm
// Primus guide): gated SwiGLU between the two grouped GEMMs.
//
// Every GEMM here has the form  C[r][c] = sum_k P[r][k] * Q[c][k]  over one expert's data:
//
//   GEMM          rows r          cols c         k            P layout      Q layout      epilogue
//   W13 FPROP     routed rows     f (gate & up)  d            xg  [r][k]    w13[e] [c][k]  SwiGLU
//   W2  FPROP     routed rows     d              f            a   [r][k]    w2[e]  [c][k]  store y
//   W2  DGRAD     routed rows     f              d            dy  [r][k]    w2[e]  [k][c]  SwiGLU'
//   W13 DGRAD     routed rows     d              j (2F)       dh13[r][k]    w13[e] [k][c]  store dxg
//   W2  WGRAD     d               f              e's rows     dy  [k][r]    a      [k][c]  store dW2
//   W13 WGRAD     j (2F)          d              e's rows     dh13[k][r]    xg     [k][c]  store dW13
//
// Tiles: BM x BN outputs per 256-thread workgroup, 2x2 wavefronts each owning BM/2 x BN/2, built
// from v_mfma_f32_32x32x16_bf16. The MFMA's A operand is the Q tile and its B operand the P tile, so
// each lane ends up holding 4 consecutive output columns of one output row (8-byte stores).
// K advances 64 at a time through a double-buffered LDS tile [rows][64] whose 16-byte chunks are
// XOR-swizzled (chunk ^ ((row ^ row>>3) & 7)) so that fragment reads (32 consecutive rows, one
// chunk) and tile writes are free of bank conflicts.
//
// Operands stored k-contiguous ([idx][k]) are copied 16 bytes per lane. Operands stored
// idx-contiguous ([k][idx]: the transposed weights in DGRAD, both operands of WGRAD) are read as
// 8x8 blocks (8 rows of 16 bytes), transposed in registers and stored k-contiguous, so one LDS
// layout and one MFMA loop serve every GEMM.
//
// Scheduling (nothing depends on host-side knowledge of the routing):
//   * row-ragged GEMMs (FPROP, DGRAD) read the plan's device list of (expert, first row) row
//     tiles and its device count; the grid is sized for the worst case and surplus workgroups exit.
//   * k-ragged GEMMs (WGRAD) give each expert a fixed M x N tile grid and walk the expert's rows as
//     the reduction; experts are taken in decreasing row count (longest first), and an expert with
//     no rows writes zeros. One workgroup owns each output tile: no atomics, no split-K.
//   * XCD-aware order: within each window of 256 consecutive workgroups, the 32 that the hardware
//     places on one XCD (workgroup id mod 8) take 32 consecutive logical tiles, and logical tiles
//     run 8 row tiles deep before the next column tiles, so concurrently running tiles of an XCD
//     share operand panels in that XCD's L2.
#include "moe_internal.h"

namespace moe {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kBK = 64;
constexpr int kThreads = 256;
constexpr int kGroupRows = 8;

enum { EPI_STORE = 0, EPI_SWIGLU_FWD = 1, EPI_SWIGLU_BWD = 2 };
enum { SCHED_ROWS = 0, SCHED_KSEG = 1 };

struct GemmArgs {
  const uint16_t* P;
  int64_t ldp;
  const uint16_t* Q;
  int64_t ldq;
  int64_t q_estride;  // elements between experts in Q (weights); 0 when Q is not per expert
  uint16_t* C;        // output (EPI_STORE), h13 (EPI_SWIGLU_FWD, may be null), dh13 (BWD)
  int64_t ldc;
  int64_t c_estride;  // elements between experts in C (WGRAD outputs)
  uint16_t* C2;       // a (EPI_SWIGLU_FWD)
  int64_t ldc2;
  const uint16_t* H;  // h13 (EPI_SWIGLU_BWD)
  int64_t ldh;
  int M_out;  // SCHED_KSEG: output rows per expert
  int N_out;  // output columns (EPI_SWIGLU_FWD: activation columns F)
  int Kdim;   // SCHED_ROWS: reduction length
  int F;
  int E;
  const int32_t* offsets;      // [E+1] expert row offsets
  const int2* mtiles;          // SCHED_ROWS: (expert, first row) per row tile
  const int32_t* mtile_count;  // SCHED_ROWS: number of row tiles (device)
  const int32_t* lpt;          // SCHED_KSEG: experts by decreasing row count
};

__device__ __forceinline__ int swz(int row, int ch) { return ch ^ ((row ^ (row >> 3)) & 7); }

struct Tile {
  int e, r0, r_lim, n0, kbeg, kend;
};

template <int BM, int BN, int SCHED, int EPI>
__device__ __forceinline__ bool decode_tile(const GemmArgs& g, Tile& t) {
  int total, ntn, mtm = 0;
  if (SCHED == SCHED_ROWS) {
    ntn = EPI == EPI_SWIGLU_FWD ? (g.N_out + BN / 2 - 1) / (BN / 2) : (g.N_out + BN - 1) / BN;
    total = g.mtile_count[0] * ntn;
  } else {
    mtm = (g.M_out + BM - 1) / BM;
    ntn = (g.N_out + BN - 1) / BN;
    total = g.E * mtm * ntn;
  }
  const int b = blockIdx.x;
  const int full = (total / 256) * 256;
  const int L = b < full ? (b & ~255) + (b & 7) * 32 + ((b & 255) >> 3) : b;
  if (L >= total) return false;
  if (SCHED == SCHED_ROWS) {
    const int mtc = g.mtile_count[0];
    const int grp = L / (kGroupRows * ntn), within = L % (kGroupRows * ntn);
    const int gm = min(kGroupRows, mtc - grp * kGroupRows);
    const int mt = grp * kGroupRows + within % gm, nt = within / gm;
    const int2 te = g.mtiles[mt];
    t.e = te.x;
    t.r0 = te.y;
    t.r_lim = g.offsets[te.x + 1];
    t.n0 = nt * (EPI == EPI_SWIGLU_FWD ? BN / 2 : BN);
    t.kbeg = 0;
    t.kend = g.Kdim;
  } else {
    const int per = mtm * ntn;
    const int er = L / per, rem = L % per;
    t.e = g.lpt[er];
    const int grp = rem / (kGroupRows * ntn), within = rem % (kGroupRows * ntn);
    const int gm = min(kGroupRows, mtm - grp * kGroupRows);
    const int mt = grp * kGroupRows + within % gm, nt = within / gm;
    t.r0 = mt * BM;
    t.r_lim = g.M_out;
    t.n0 = nt * BN;
    t.kbeg = g.offsets[t.e];
    t.kend = g.offsets[t.e + 1];
  }
  return true;
}

// ---- operand tiles ---------------------------------------------------------------------------

// k-contiguous operand: R rows of 64 k; thread copies R/32 chunks of 16 bytes per k step.
template <int R>
struct KcTile {
  static constexpr int IT = R / 32;
  const uint16_t* src[IT];
  int dst[IT];  // LDS element offset
  uint4 v[IT];

  __device__ __forceinline__ void init_row(int it, const uint16_t* rowptr) {
    const int row = it * 32 + (threadIdx.x >> 3), ch = threadIdx.x & 7;
    src[it] = rowptr + ch * 8;
    dst[it] = row * kBK + swz(row, ch) * 8;
  }
  __device__ __forceinline__ static int row_of(int it) { return it * 32 + (threadIdx.x >> 3); }
  __device__ __forceinline__ void load(int k0) {
#pragma unroll
    for (int it = 0; it < IT; ++it) v[it] = *(const uint4*)(src[it] + k0);
  }
  __device__ __forceinline__ void store(uint16_t* s) const {
#pragma unroll
    for (int it = 0; it < IT; ++it) *(uint4*)(s + dst[it]) = v[it];
  }
};

// idx-contiguous operand: tile of R idx x 64 k read as R 8x8 blocks (one per thread, threads < R).
template <int R, bool MASK_K>
struct McTile {
  const uint16_t* base;  // points at (k = 0, idx = this thread's first idx)
  int64_t ld;
  int kb;  // this thread's 8-row k block
  int ib;  // this thread's 8-wide idx block
  int kend;
  bool active;
  uint4 v[8];

  __device__ __forceinline__ void init(const uint16_t* b, int64_t ld_, int idx0, int idx_lim,
                                       int kend_) {
    const int tid = threadIdx.x;
    active = tid < R;
    ib = tid % (R / 8);
    kb = tid / (R / 8);
    int idx = idx0 + ib * 8;
    if (idx > idx_lim - 8) idx = idx_lim - 8;
    base = b + idx;
    ld = ld_;
    kend = kend_;
  }
  __device__ __forceinline__ void load(int k0) {
    if (!active) return;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      const int k = k0 + kb * 8 + kk;
      if (MASK_K && k >= kend)
        v[kk] = make_uint4(0, 0, 0, 0);
      else
        v[kk] = *(const uint4*)(base + (int64_t)k * ld);
    }
  }
  __device__ __forceinline__ void store(uint16_t* s) const {
    if (!active) return;
    const uint32_t* w = (const uint32_t*)v;  // w[kk*4 + q]: idx pair (2q, 2q+1) at row kk
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      uint32_t o[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t lo = w[(2 * q) * 4 + (i >> 1)], hi = w[(2 * q + 1) * 4 + (i >> 1)];
        o[q] = (i & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
      }
      const int row = ib * 8 + i;
      *(uint4*)(s + row * kBK + swz(row, kb) * 8) = make_uint4(o[0], o[1], o[2], o[3]);
    }
  }
};

// ---- the kernel -------------------------------------------------------------------------------

template <int BM, int BN, bool P_KC, bool Q_KC, int SCHED, int EPI>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1))) void k_gemm(
    GemmArgs g) {
  constexpr int WM = BM / 2, WN = BN / 2, FM = WM / 32, FN = WN / 32;
  static_assert(FM >= 1 && FN >= 2 && (FN % 2) == 0, "tile shape");
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * (BM + BN) * kBK];

  Tile t;
  if (!decode_tile<BM, BN, SCHED, EPI>(g, t)) return;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wr = wave & 1, wc = wave >> 1;

  // operand P (rows of the output)
  KcTile<BM> pk;
  McTile<BM, SCHED == SCHED_KSEG> pm;
  if constexpr (P_KC) {
#pragma unroll
    for (int it = 0; it < BM / 32; ++it) {
      int r = t.r0 + KcTile<BM>::row_of(it);
      if (r > t.r_lim - 1) r = t.r_lim - 1;
      pk.init_row(it, g.P + (int64_t)r * g.ldp);
    }
  } else {
    pm.init(g.P, g.ldp, t.r0, t.r_lim, t.kend);
  }
  // operand Q (columns of the output)
  const uint16_t* qbase = g.Q + (int64_t)t.e * g.q_estride;
  KcTile<BN> qk;
  McTile<BN, SCHED == SCHED_KSEG> qm;
  if constexpr (Q_KC) {
#pragma unroll
    for (int it = 0; it < BN / 32; ++it) {
      const int c = KcTile<BN>::row_of(it);
      int wrow;
      if constexpr (EPI == EPI_SWIGLU_FWD) {
        // tile column c -> wavefront column half, MFMA block, lane; the first FN/2 blocks of a
        // wavefront hold gate rows and the last FN/2 the up rows of the same f
        const int wq = c / WN, within = c % WN, blk = within / 32, ln = within % 32;
        const int half = blk / (FN / 2);
        int f = t.n0 + wq * (WN / 2) + (blk % (FN / 2)) * 32 + ln;
        if (f > g.F - 1) f = g.F - 1;
        wrow = half * g.F + f;
      } else {
        wrow = t.n0 + c;
        if (wrow > g.N_out - 1) wrow = g.N_out - 1;
      }
      qk.init_row(it, qbase + (int64_t)wrow * g.ldq);
    }
  } else {
    qm.init(qbase, g.ldq, t.n0, g.N_out, t.kend);
  }

  // buffer b: P tile at smem + b*(BM+BN)*64, Q tile right after it
  auto sP = [&](int b) { return smem + b * (BM + BN) * kBK; };
  auto sQ = [&](int b) { return smem + b * (BM + BN) * kBK + BM * kBK; };

  f32x16 acc[FN][FM];
#pragma unroll
  for (int i = 0; i < FN; ++i)
#pragma unroll
    for (int j = 0; j < FM; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.0f;

  const int nk = (t.kend - t.kbeg + kBK - 1) / kBK;

  auto load = [&](int k0) {
    if constexpr (P_KC) pk.load(k0); else pm.load(k0);
    if constexpr (Q_KC) qk.load(k0); else qm.load(k0);
  };
  auto store = [&](int buf) {
    if constexpr (P_KC) pk.store(sP(buf)); else pm.store(sP(buf));
    if constexpr (Q_KC) qk.store(sQ(buf)); else qm.store(sQ(buf));
  };

  if (nk > 0) {
    load(t.kbeg);
    store(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
      const int cur = kt & 1;
      if (kt + 1 < nk) load(t.kbeg + (kt + 1) * kBK);
      const uint16_t* P_s = sP(cur);
      const uint16_t* Q_s = sQ(cur);
#pragma unroll
      for (int ks = 0; ks < kBK / 16; ++ks) {
        const int ch = ks * 2 + (lane >> 5);
        bf16x8 qa[FN], pb[FM];
#pragma unroll
        for (int i = 0; i < FN; ++i) {
          const int row = wc * WN + i * 32 + (lane & 31);
          qa[i] = *(const bf16x8*)(Q_s + row * kBK + swz(row, ch) * 8);
        }
#pragma unroll
        for (int j = 0; j < FM; ++j) {
          const int row = wr * WM + j * 32 + (lane & 31);
          pb[j] = *(const bf16x8*)(P_s + row * kBK + swz(row, ch) * 8);
        }
#pragma unroll
        for (int i = 0; i < FN; ++i)
#pragma unroll
          for (int j = 0; j < FM; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[i], pb[j], acc[i][j], 0, 0, 0);
      }
      if (kt + 1 < nk) store(cur ^ 1);
      __syncthreads();
    }
  }

  // ---- epilogue: lane holds rows r = base + (lane & 31), columns 8*gq + 4*(lane >> 5) + 0..3
  const int cq = 4 * (lane >> 5);
  if constexpr (EPI == EPI_STORE) {
    uint16_t* C = g.C + (int64_t)t.e * g.c_estride;
#pragma unroll
    for (int j = 0; j < FM; ++j) {
      const int r = t.r0 + wr * WM + j * 32 + (lane & 31);
      if (r >= t.r_lim) continue;
#pragma unroll
      for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          const int c = t.n0 + wc * WN + i * 32 + gq * 8 + cq;
          if (c >= g.N_out) continue;
          const uint2 v = make_uint2(pack_bf16x2(acc[i][j][4 * gq], acc[i][j][4 * gq + 1]),
                                     pack_bf16x2(acc[i][j][4 * gq + 2], acc[i][j][4 * gq + 3]));
          *(uint2*)(C + (int64_t)r * g.ldc + c) = v;
        }
    }
  } else if constexpr (EPI == EPI_SWIGLU_FWD) {
#pragma unroll
    for (int j = 0; j < FM; ++j) {
      const int r = t.r0 + wr * WM + j * 32 + (lane & 31);
      if (r >= t.r_lim) continue;
#pragma unroll
      for (int i = 0; i < FN / 2; ++i)
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          const int f = t.n0 + wc * (WN / 2) + i * 32 + gq * 8 + cq;
          if (f >= g.F) continue;
          uint32_t gb[4], ub[4];
          float av[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            gb[q] = f32_to_bf16(acc[i][j][4 * gq + q]);
            ub[q] = f32_to_bf16(acc[i + FN / 2][j][4 * gq + q]);
            const float gv = bf16_to_f32(gb[q]), uv = bf16_to_f32(ub[q]);
            av[q] = gv * sigmoid_f32(gv) * uv;
          }
          if (g.C) {
            uint16_t* hrow = g.C + (int64_t)r * g.ldc;
            *(uint2*)(hrow + f) = make_uint2(gb[0] | (gb[1] << 16), gb[2] | (gb[3] << 16));
            *(uint2*)(hrow + g.F + f) = make_uint2(ub[0] | (ub[1] << 16), ub[2] | (ub[3] << 16));
          }
          *(uint2*)(g.C2 + (int64_t)r * g.ldc2 + f) =
              make_uint2(pack_bf16x2(av[0], av[1]), pack_bf16x2(av[2], av[3]));
        }
    }
  } else {  // EPI_SWIGLU_BWD: acc = da over columns f
#pragma unroll
    for (int j = 0; j < FM; ++j) {
      const int r = t.r0 + wr * WM + j * 32 + (lane & 31);
      if (r >= t.r_lim) continue;
#pragma unroll
      for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          const int f = t.n0 + wc * WN + i * 32 + gq * 8 + cq;
          if (f >= g.F) continue;
          const uint16_t* hrow = g.H + (int64_t)r * g.ldh;
          const uint2 gh = *(const uint2*)(hrow + f);
          const uint2 uh = *(const uint2*)(hrow + g.F + f);
          const uint32_t gw[4] = {gh.x & 0xffffu, gh.x >> 16, gh.y & 0xffffu, gh.y >> 16};
          const uint32_t uw[4] = {uh.x & 0xffffu, uh.x >> 16, uh.y & 0xffffu, uh.y >> 16};
          float dg[4], du[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float gv = bf16_to_f32(gw[q]), uv = bf16_to_f32(uw[q]);
            const float da = acc[i][j][4 * gq + q];
            const float sg = sigmoid_f32(gv);
            dg[q] = da * uv * sg * (1.0f + gv * (1.0f - sg));
            du[q] = da * gv * sg;
          }
          uint16_t* drow = g.C + (int64_t)r * g.ldc;
          *(uint2*)(drow + f) = make_uint2(pack_bf16x2(dg[0], dg[1]), pack_bf16x2(dg[2], dg[3]));
          *(uint2*)(drow + g.F + f) =
              make_uint2(pack_bf16x2(du[0], du[1]), pack_bf16x2(du[2], du[3]));
        }
    }
  }
}

template <int BM, int BN, bool P_KC, bool Q_KC, int SCHED, int EPI>
hipError_t launch(const GemmArgs& g, int grid, hipStream_t st) {
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL((k_gemm<BM, BN, P_KC, Q_KC, SCHED, EPI>), dim3(grid), dim3(kThreads), 0, st,
                     g);
  return hipGetLastError();
}

constexpr int kBM = 256, kBN = 256;

GemmArgs rows_args(const moe_shape& s, const PlanPtrs& p, int bm) {
  GemmArgs g{};
  g.F = (int)s.F;
  g.E = (int)s.E;
  g.offsets = p.offsets;
  const int ti = tile_size_index(bm);
  g.mtiles = (const int2*)p.mtiles[ti];
  g.mtile_count = p.status + 1 + ti;
  return g;
}

int rows_grid(const moe_shape& s, int bm, int ntn) {
  const int64_t mt_max = ceil_div(s.T * s.K, bm) + s.E;
  return (int)(mt_max * ntn);
}

}  // namespace

hipError_t launch_fprop_w13(const moe_shape& s, const PlanPtrs& p, const uint16_t* xg,
                            const uint16_t* w13, uint16_t* h13, uint16_t* a, hipStream_t st) {
  GemmArgs g = rows_args(s, p, kBM);
  g.P = xg; g.ldp = s.D;
  g.Q = w13; g.ldq = s.D; g.q_estride = 2 * s.F * s.D;
  g.C = h13; g.ldc = 2 * s.F;
  g.C2 = a; g.ldc2 = s.F;
  g.N_out = (int)s.F; g.Kdim = (int)s.D;
  const int ntn = (int)ceil_div(s.F, kBN / 2);
  return launch<kBM, kBN, true, true, SCHED_ROWS, EPI_SWIGLU_FWD>(g, rows_grid(s, kBM, ntn), st);
}

hipError_t launch_fprop_w2(const moe_shape& s, const PlanPtrs& p, const uint16_t* a,
                           const uint16_t* w2, uint16_t* y, hipStream_t st) {
  GemmArgs g = rows_args(s, p, kBM);
  g.P = a; g.ldp = s.F;
  g.Q = w2; g.ldq = s.F; g.q_estride = s.D * s.F;
  g.C = y; g.ldc = s.D;
  g.N_out = (int)s.D; g.Kdim = (int)s.F;
  const int ntn = (int)ceil_div(s.D, kBN);
  return launch<kBM, kBN, true, true, SCHED_ROWS, EPI_STORE>(g, rows_grid(s, kBM, ntn), st);
}

hipError_t launch_dgrad_w2(const moe_shape& s, const PlanPtrs& p, const uint16_t* dy,
                           const uint16_t* w2, const uint16_t* h13, uint16_t* dh13,
                           hipStream_t st) {
  GemmArgs g = rows_args(s, p, kBM);
  g.P = dy; g.ldp = s.D;
  g.Q = w2; g.ldq = s.F; g.q_estride = s.D * s.F;  // w2[e] read as [k = d][c = f]
  g.C = dh13; g.ldc = 2 * s.F;
  g.H = h13; g.ldh = 2 * s.F;
  g.N_out = (int)s.F; g.Kdim = (int)s.D;
  const int ntn = (int)ceil_div(s.F, kBN);
  return launch<kBM, kBN, true, false, SCHED_ROWS, EPI_SWIGLU_BWD>(g, rows_grid(s, kBM, ntn), st);
}

hipError_t launch_dgrad_w13(const moe_shape& s, const PlanPtrs& p, const uint16_t* dh13,
                            const uint16_t* w13, uint16_t* dxg, hipStream_t st) {
  GemmArgs g = rows_args(s, p, kBM);
  g.P = dh13; g.ldp = 2 * s.F;
  g.Q = w13; g.ldq = s.D; g.q_estride = 2 * s.F * s.D;  // w13[e] read as [k = j][c = d]
  g.C = dxg; g.ldc = s.D;
  g.N_out = (int)s.D; g.Kdim = (int)(2 * s.F);
  const int ntn = (int)ceil_div(s.D, kBN);
  return launch<kBM, kBN, true, false, SCHED_ROWS, EPI_STORE>(g, rows_grid(s, kBM, ntn), st);
}

hipError_t launch_wgrad_w2(const moe_shape& s, const PlanPtrs& p, const uint16_t* dy,
                           const uint16_t* a, uint16_t* dw2, hipStream_t st) {
  GemmArgs g{};
  g.F = (int)s.F; g.E = (int)s.E; g.offsets = p.offsets; g.lpt = p.lpt;
  g.P = dy; g.ldp = s.D;  // [k = routed row][r = d]
  g.Q = a; g.ldq = s.F;   // [k = routed row][c = f]
  g.C = dw2; g.ldc = s.F; g.c_estride = s.D * s.F;
  g.M_out = (int)s.D; g.N_out = (int)s.F;
  const int grid = (int)(s.E * ceil_div(s.D, kBM) * ceil_div(s.F, kBN));
  return launch<kBM, kBN, false, false, SCHED_KSEG, EPI_STORE>(g, grid, st);
}

hipError_t launch_wgrad_w13(const moe_shape& s, const PlanPtrs& p, const uint16_t* dh13,
                            const uint16_t* xg, uint16_t* dw13, hipStream_t st) {
  GemmArgs g{};
  g.F = (int)s.F; g.E = (int)s.E; g.offsets = p.offsets; g.lpt = p.lpt;
  g.P = dh13; g.ldp = 2 * s.F;  // [k = routed row][r = j]
  g.Q = xg; g.ldq = s.D;        // [k = routed row][c = d]
  g.C = dw13; g.ldc = s.D; g.c_estride = 2 * s.F * s.D;
  g.M_out = (int)(2 * s.F); g.N_out = (int)s.D;
  const int grid = (int)(s.E * ceil_div(2 * s.F, kBM) * ceil_div(s.D, kBN));
  return launch<kBM, kBN, false, false, SCHED_KSEG, EPI_STORE>(g, grid, st);
}

}  // namespace moe
