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
//                 (xg[r] = x[src[r] / K]: with a gather list the row copies read x directly)
//   W2  FPROP     routed rows     d              f            a   [r][k]    w2[e]  [c][k]  store y
//   W2  DGRAD     routed rows     f              d            dy  [r][k]    w2[e]  [k][c]  SwiGLU'
//   W13 DGRAD     routed rows     d              j (2F)       dh13[r][k]    w13[e] [k][c]  store dxg
//   W2  WGRAD     d               f              e's rows     dy  [k][r]    a      [k][c]  store dW2
//   W13 WGRAD     j (2F)          d              e's rows     dh13[k][r]    xg     [k][c]  store dW13
//
// Tiles: 256 x 256 outputs per 512-thread workgroup, 8 wavefronts (two per SIMD) in 4 row groups x
// 2 column halves, each owning 64 x 128 outputs, built from v_mfma_f32_32x32x16_bf16. The MFMA's A
// operand is the Q tile and its B operand the P tile, so each lane ends up holding 4 consecutive
// output columns of one output row. K advances 64 at a time through two LDS stages of 64 KiB,
// filled by LDS-DMA copies (global_load_lds_dwordx4) one stage ahead of their use.
//
// Operands stored k-contiguous ([idx][k]) sit in LDS as [rows][64] with XOR-swizzled 16-byte
// chunks (chunk ^ ((row ^ row>>3) & 7)), read as 16-byte fragments. Operands stored
// idx-contiguous ([k][idx]: the transposed weights in DGRAD, both operands of WGRAD) keep that
// orientation in LDS ([64 k][256 idx], 8-byte chunks swizzled by k) and become MFMA fragments
// through the LDS transpose read (ds_read_b64_tr_b16), so one MFMA loop serves every GEMM. Both
// layouts keep fragment reads and copies free of bank conflicts.
//
// Scheduling (nothing depends on host-side knowledge of the routing):
//   * row-ragged GEMMs (FPROP, DGRAD) read the plan's device list of (expert, first row) row
//     tiles and its device count; the grid is sized for the worst case and surplus workgroups exit.
//   * k-ragged GEMMs (WGRAD) give each expert a fixed M x N tile grid and walk the expert's rows as
//     the reduction; experts are taken in decreasing row count (longest first), and an expert with
//     no rows writes zeros. One workgroup owns each output tile: no atomics, no split-K.
//   * XCD-aware order: within each window of 256 consecutive workgroups, the 32 that the hardware
//     places on one XCD (workgroup id mod 8) take 32 consecutive logical tiles, and logical tiles
//     run 8 row tiles deep (one expert's row tiles at a time) before the next column tiles, so
//     concurrently running tiles of an XCD share operand panels in that XCD's L2.
#include <algorithm>
#include <type_traits>

#include "moe_internal.h"

namespace moe {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kBK = 64;  // k per LDS stage
constexpr int kBM = 256, kBN = 256;  // output tile
constexpr int kLdsElems = 2 * (kBM + kBN) * kBK;  // two stages (bf16 elements): 128 KiB
// Wavefronts per workgroup: 8, two per SIMD, each owning 64 x 128 of the 256 x 256 tile (128
// accumulator registers), so that while one wavefront of a SIMD waits (for LDS data, a copy, the
// barrier) the other can issue MFMAs.
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kEpWaveElems = 65536 / kWaves;  // per-wavefront epilogue staging area (bf16 elements)
constexpr int kGroupRows = 8;
static_assert(kRowTile % 32 == 0 && kRowTile <= kBM, "a plan row tile fits one output tile");

enum { EPI_STORE = 0, EPI_SWIGLU_FWD = 1, EPI_SWIGLU_BWD = 2 };
// EPI_STORE output: bf16 (C), bf16 added to the existing values, fp32 (Cf), fp32 added
enum { OUT_BF16 = 0, OUT_BF16_ACC = 1, OUT_F32 = 2, OUT_F32_ACC = 3 };
enum { SCHED_ROWS = 0, SCHED_KSEG = 1 };

struct GemmArgs {
  const uint16_t* P;
  int64_t ldp;
  const uint16_t* Q;
  int64_t ldq;
  int64_t q_estride;  // elements between experts in Q (weights); 0 when Q is not per expert
  uint16_t* C;        // output (EPI_STORE), h13 (EPI_SWIGLU_FWD, may be null), dh13 (BWD)
  float* Cf;          // fp32 output (EPI_STORE with OUT_F32 / OUT_F32_ACC), same ldc / c_estride
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
  const int32_t* mtile_start;  // SCHED_ROWS: each expert's first index in mtiles
  const int32_t* mtile_count;  // SCHED_ROWS: number of row tiles (device)
  const int32_t* lpt;          // SCHED_KSEG: experts by decreasing row count
  // P rows gathered from token rows (fused permute): P row r is row src[r] / gather_k of P
  const int32_t* gather_src;   // null: P rows are the routed rows themselves
  int gather_k;
  // extents in bytes of P, Q, C (or Cf), C2, H and gather_src from those pointers; the checked
  // build tests every access against them
  uint64_t ext_p, ext_q, ext_c, ext_c2, ext_h, ext_src;
};

// LDS tile layout: [rows][BK] bf16, each row BK/8 chunks of 16 bytes; logical chunk c of row r
// is stored at physical chunk c ^ t(r):
//   BK = 64 (8 chunks, 128-byte rows): t(r) = (r ^ r>>3) & 7
//   BK = 32 (4 chunks, 64-byte rows):  t(r) = (r>>1 ^ r>>3) & 3
// With these, a fragment read (32 consecutive rows at one chunk) and the tile writes touch every
// LDS bank at most once in each 8-lane (32-bank) or 16-lane (64-bank) phase.
template <int BK>
__device__ __forceinline__ int swz(int row, int ch) {
  if constexpr (BK == 64)
    return ch ^ ((row ^ (row >> 3)) & 7);
  else
    return ch ^ (((row >> 1) ^ (row >> 3)) & 3);
}


struct Tile {
  int e, r0, r_lim, n0, kbeg, kend;
};

template <int BM, int BN, int SCHED, int EPI>
__device__ __forceinline__ bool decode_tile(const GemmArgs& g, Tile& t, int b) {
  int total, ntn, mtm = 0;
  if (SCHED == SCHED_ROWS) {
    ntn = EPI == EPI_SWIGLU_FWD ? (g.N_out + BN / 2 - 1) / (BN / 2) : (g.N_out + BN - 1) / BN;
    total = g.mtile_count[0] * ntn;
  } else {
    mtm = (g.M_out + BM - 1) / BM;
    ntn = (g.N_out + BN - 1) / BN;
    total = g.E * mtm * ntn;
  }
  const int full = (total / 256) * 256;
  const int L = b < full ? (b & ~255) + (b & 7) * 32 + ((b & 255) >> 3) : b;
  if (L >= total) return false;
  if (SCHED == SCHED_ROWS) {
    // an expert's row tiles are consecutive in the list, so the logical tiles of expert e are
    // [ts*ntn, (ts+nt_e)*ntn) with ts its first row tile: L / ntn names a row tile of L's expert.
    // Groups of kGroupRows row tiles are formed within each expert, so the tiles that run side by
    // side on an XCD share one expert's weight panels. A tile ends where the expert's next tile
    // starts (at most kRowTile <= BM rows)
    const int e = g.mtiles[L / ntn].x, eend = g.offsets[e + 1];
    const int ts = g.mtile_start[e];
    const int nte = (eend - g.offsets[e] + kRowTile - 1) / kRowTile;
    const int Le = L - ts * ntn;
    const int grp = Le / (kGroupRows * ntn), within = Le % (kGroupRows * ntn);
    const int gm = min(kGroupRows, nte - grp * kGroupRows);
    const int mt = grp * kGroupRows + within % gm, nt = within / gm;  // row tile within e
    t.e = e;
    t.r0 = g.mtiles[ts + mt].y;
    t.r_lim = mt + 1 < nte ? g.mtiles[ts + mt + 1].y : eend;
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

// One 16-byte-per-lane copy global -> LDS (global_load_lds_dwordx4, scalar base + 32-bit lane
// offset): lane l's 16 bytes land at LDS byte address lds + 16*l. Issued through inline assembly
// so that the compiler's wait-count bookkeeping sees only the LDS reads of the MFMA loop (an
// LDS-DMA it knows about makes it wait for every outstanding LDS read); the copies are waited for
// explicitly (s_waitcnt 0) before each barrier. M0 carries the LDS address; the kernels that use
// this have no other use of M0.
__device__ __forceinline__ void dma16(const char* base, uint32_t off, uint32_t lds_addr) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_addr);
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(off), "s"(base), "s"(m0)
               : "memory", "m0");
}

// LDS byte address of a pointer into a __shared__ array. Taken once per kernel, of the array
// itself, and offset with integer arithmetic from there: the compiler folds the cast of the
// array's address to a constant, where a cast of a computed generic pointer would carry a null
// test.
__device__ __forceinline__ uint32_t lds_address(const uint16_t* p) {
  typedef __attribute__((address_space(3))) const uint16_t* lds_ptr;
  return (uint32_t)(uintptr_t)(lds_ptr)p;
}

__device__ __forceinline__ const char* uniform_ptr(const void* p) {
  const uint64_t v = (uint64_t)(uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (const char*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

// k-contiguous operand, copied global -> LDS by DMA: one instruction moves 64 lanes x 16 bytes
// into 1 KiB of LDS, i.e. 8 rows x 64 k of the tile with lane l landing in row l/8, physical
// chunk l%8. Each lane therefore fetches the logical chunk that the swizzle stores there. The R/8
// blocks of a tile are split evenly over the wavefronts (R/64 each). Addresses: a wave-uniform
// base plus a 32-bit byte offset per lane and block.
template <int R>
struct DmaTile {
  static constexpr int NB = R / 8 / kWaves;  // blocks per wavefront = copy actions per stage
  const char* base;                  // uniform
  uint32_t off[NB];                  // per lane, bytes from base (k = 0)
#ifdef MOE_CHECKED
  const char* lo;                    // the operand's buffer and its extent in bytes
  uint64_t ext;
#endif

  // row_off(row) -> byte offset of the start of tile row `row` (0 <= row < R) from base
  template <typename RowOff>
  __device__ __forceinline__ void init(const void* b, RowOff row_off) {
    base = uniform_ptr(b);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int blk = wave * NB + i;
      const int row = blk * 8 + (lane >> 3);
      off[i] = row_off(row) + swz<kBK>(row, lane & 7) * 16;
    }
  }
  // lds_tile: LDS byte address of the tile
  __device__ __forceinline__ void issue(uint32_t lds_tile, int k0, int i) const {
    const int blk = (threadIdx.x >> 6) * NB + i;
#ifdef MOE_CHECKED
    if (__any(!moe_check_range(base + (int64_t)k0 * 2 + off[i], 16, lo, ext))) return;
#endif
    dma16(base + (int64_t)k0 * 2, off[i], lds_tile + blk * 8 * kBK * 2);
  }
};

// idx-contiguous operand ([k][idx] in memory): the tile is kept in that orientation in LDS,
// [64 k][R idx] with 512-byte rows for R = 256, and turned into MFMA fragments by the LDS transpose
// read (ds_read_b64_tr_b16). Copy: 1 KiB DMA blocks of 2 k rows; lane l lands in row l/32 at
// physical 16-byte chunk l%32 and fetches the logical chunk stored there. Layout: the 8-byte chunk
// x of row k sits at x ^ ((k & 3) << 3), which keeps the transpose reads (4 rows x 8 chunks per
// 32 lanes) on distinct banks and keeps each lane's 16-byte DMA chunk contiguous.
// Rows past kend (ragged reduction of a weight gradient) are clamped to row kend-1 here and
// zeroed in the P fragments (mask_tail in the kernel), so every product past kend is 0.
template <int R>
struct MnTile {
  static constexpr int NB = 64 / 2 / kWaves;  // 1 KiB blocks per wavefront
  static_assert(R == 256, "MN tiles are 256 wide");
  const char* base;   // uniform: element (k = kbeg, idx = 0 of the tile's idx range)
  int64_t ldb;        // bytes between k rows
  uint32_t col[NB];   // per lane: byte offset of its 16-byte chunk within a row (clamped)
  int row[NB];        // per lane: k row within a stage (0..63)
#ifdef MOE_CHECKED
  const char* lo;     // the operand's buffer and its extent in bytes
  uint64_t ext;
#endif

  __device__ __forceinline__ void init(const void* b, int64_t ld, int idx0, int idx_lim) {
    base = uniform_ptr(b);
    ldb = ld * 2;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int blk = wave * NB + i;
      const int k = blk * 2 + (lane >> 5);
      const int logical = (lane & 31) ^ ((k & 3) << 2);  // 16-byte chunk within the row
      int idx = idx0 + logical * 8;
      if (idx > idx_lim - 8) idx = idx_lim - 8;
      col[i] = (uint32_t)(idx * 2);
      row[i] = k;
    }
  }
  // copy k rows [k0, k0+64) of the tile (k counted from kbeg); rows at or past klim (relative
  // count of valid rows) are clamped to klim - 1
  __device__ __forceinline__ void issue(uint32_t lds_tile, int k0, int klim, int i) const {
    const int blk = (threadIdx.x >> 6) * NB + i;
    int k = k0 + row[i];
    if (k > klim - 1) k = klim - 1;  // k0 <= klim - 1 whenever the stage exists
#ifdef MOE_CHECKED
    if (__any(!moe_check_range(base + (int64_t)k0 * ldb + (uint32_t)((k - k0) * ldb) + col[i], 16,
                               lo, ext)))
      return;
#endif
    dma16(base + (int64_t)k0 * ldb, (uint32_t)((k - k0) * ldb) + col[i], lds_tile + blk * 2 * R * 2);
  }
};

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
typedef __attribute__((address_space(3))) uint16_t lds_u16;

// Half h (k 4h..4h+3 of each 8) of the MFMA fragment of a [64][256] MN tile for the 32 idx
// starting at idx0 and k sub-step ks: lane l receives idx idx0 + (l & 31), k rows
// 16 ks + 8 (l >> 5) + 4 h + 0..3. Within each 16-lane group, lane 4q + p points at row q,
// idx chunk p of the 16 the group covers.
__device__ __forceinline__ v4i16 read_mn_half(const uint16_t* tile, int idx0, int ks, int h) {
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4, j = lane & 15;
  const int k = ks * 16 + (g >> 1) * 8 + h * 4 + (j >> 2);
  const int x = ((idx0 + (g & 1) * 16) >> 2) + (j & 3);  // 8-byte chunk
  const int xp = x ^ ((k & 3) << 3);
  const lds_u16* p = (const lds_u16*)(tile) + k * 256 + xp * 4;
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)p);
}

// ---- the kernel -------------------------------------------------------------------------------

template <int BM, int BN, bool P_KC, bool Q_KC, int SCHED, int EPI, int OUT = OUT_BF16>
// lds: the kernel's 128 KiB LDS array; b: the tile's index in the launch order of this GEMM
__device__ __forceinline__ void gemm_body(const GemmArgs& g, uint16_t* lds, int b) {
  constexpr int WR = kWaves / 2;  // wavefront rows (P) x 2 wavefront columns (Q)
  constexpr int WM = BM / WR, WN = BN / 2, FM = WM / 32, FN = WN / 32;
  constexpr int MPK = FN * FM;  // MFMAs per k sub-step and wavefront
  static_assert(BM == 256 && BN == 256, "the interleaved schedule below assumes 256x256 tiles");
  constexpr int BK = kBK;
  constexpr bool MASK_K = SCHED == SCHED_KSEG;
  static_assert(2 * (BM + BN) * BK == kLdsElems, "LDS stages");

  Tile t;
  if (!decode_tile<BM, BN, SCHED, EPI>(g, t, b)) return;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: wave-level branches
  // Wavefront row group wr owns the interleaved 32-row blocks wr, wr + WR, ... of the tile, and
  // wavefront w runs on SIMD w % 4, so SIMD s hosts wavefronts s and s + 4 (row groups s/2 and
  // s/2 + 2): the first rows of a tile spread over all four SIMDs, and a partly filled tile (the
  // ragged last row tile of an expert) runs in proportion to its rows
  const int wr = wave / 2, wc = wave % 2;
  const int klen = t.kend - t.kbeg;

  // operand P (rows of the output)
  DmaTile<BM> pd;
  MnTile<BM> pm;
  if constexpr (P_KC) {
    const int r0 = t.r0, rl = t.r_lim;
    const int64_t ldb = g.ldp * 2;
    if (g.gather_src) {
      // fused permute (Dist-MoE "Understand the execution model": routing metadata drives the
      // expert GEMMs; MoonEP FAQ: tokens go straight to their expert-grouped positions): the
      // copies read each routed row's token row of x; offsets from the base of x (the host
      // checks that x spans less than 4 GiB)
      const int32_t* src = g.gather_src;
      const int kk = g.gather_k;
      pd.init(g.P, [&](int row) -> uint32_t {
        int r = r0 + row;
        if (r > rl - 1) r = rl - 1;
        if (!MOE_IN(src + r, 4, src, g.ext_src)) return 0u;
        return (uint32_t)((int64_t)(src[r] / kk) * ldb);
      });
    } else {
      pd.init(g.P + (int64_t)r0 * g.ldp, [&](int row) -> uint32_t {
        int r = r0 + row;
        if (r > rl - 1) r = rl - 1;
        return (uint32_t)((int64_t)(r - r0) * ldb);
      });
    }
  } else {
    pm.init(g.P + (int64_t)t.kbeg * g.ldp + t.r0, g.ldp, 0, t.r_lim - t.r0);
  }
  // operand Q (columns of the output)
  const uint16_t* qbase = g.Q + (int64_t)t.e * g.q_estride;
  DmaTile<BN> qd;
  MnTile<BN> qm;
  if constexpr (Q_KC) {
    const int n0 = t.n0, F = g.F, nlim = g.N_out;
    const int64_t ldb = g.ldq * 2;
    qd.init(qbase, [&](int c) -> uint32_t {
      int wrow;
      if constexpr (EPI == EPI_SWIGLU_FWD) {
        // tile column c -> wavefront column half, MFMA block, lane; the first FN/2 blocks of a
        // wavefront hold gate rows and the last FN/2 the up rows of the same f
        const int wq = c / WN, within = c % WN, blk = within / 32, ln = within % 32;
        const int half = blk / (FN / 2);
        int f = n0 + wq * (WN / 2) + (blk % (FN / 2)) * 32 + ln;
        if (f > F - 1) f = F - 1;
        wrow = half * F + f;
      } else {
        wrow = n0 + c;
        if (wrow > nlim - 1) wrow = nlim - 1;
      }
      return (uint32_t)((int64_t)wrow * ldb);
    });
  } else {
    qm.init(qbase + (int64_t)t.kbeg * g.ldq + t.n0, g.ldq, 0, g.N_out - t.n0);
  }

#ifdef MOE_CHECKED
  pd.lo = pm.lo = (const char*)g.P;
  pd.ext = pm.ext = g.ext_p;
  qd.lo = qm.lo = (const char*)g.Q;
  qd.ext = qm.ext = g.ext_q;
#endif
  f32x16 acc[FN][FM];
#pragma unroll
  for (int i = 0; i < FN; ++i)
#pragma unroll
    for (int j = 0; j < FM; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.0f;

  const int nk = (klen + BK - 1) / BK;
  auto bufP = [&](int b) { return lds + b * (BM + BN) * BK; };
  auto bufQ = [&](int b) { return lds + b * (BM + BN) * BK + BM * BK; };
  const uint32_t lds0 = lds_address(lds);  // byte addresses of the stage buffers for the copies
  auto addrP = [&](int b) { return lds0 + (uint32_t)(b * (BM + BN) * BK * 2); };
  auto addrQ = [&](int b) { return lds0 + (uint32_t)((b * (BM + BN) * BK + BM * BK) * 2); };

  // this wavefront's 32-row blocks (jlim of FM) and 32-column blocks (ilim of FN; for the SwiGLU
  // forward per gate/up half) that hold any output: the products of the others (the ragged last
  // row tile of an expert, a column tail) are skipped
  const int tile_rows = t.r_lim - t.r0;
  const int nblk = tile_rows >= BM ? BM / 32 : (tile_rows + 31) / 32;  // 32-row blocks with rows
  const int jlim = nblk <= wr ? 0 : min(FM, (nblk - wr + WR - 1) / WR);
  int ilim;
  if constexpr (EPI == EPI_SWIGLU_FWD) {
    const int cols_left = g.F - (t.n0 + wc * (WN / 2));
    ilim = cols_left <= 0 ? 0 : (cols_left >= WN / 2 ? FN / 2 : (cols_left + 31) / 32);
  } else {
    const int cols_left = g.N_out - (t.n0 + wc * WN);
    ilim = cols_left <= 0 ? 0 : (cols_left >= WN ? FN : (cols_left + 31) / 32);
  }
  // P copies of a row-ragged tile: wavefront w copies the tile's 32-row block w (rows
  // 32w..32w+31, DmaTile with R = 256), so in a partly filled tile (an expert's ragged last row
  // tile) the wavefronts whose block holds no row copy nothing; those LDS rows feed only the
  // fragments of empty blocks, whose products are skipped (the fragment reads stay: skipping
  // them costs registers)
  static_assert(SCHED != SCHED_ROWS || (P_KC && DmaTile<BM>::NB * 8 * kWaves == BM && BM == 256),
                "row-ragged GEMMs copy one 32-row block of P per wavefront");
  const bool p_copy_on = SCHED != SCHED_ROWS || wave < nblk;
  // copy of one stage: NBO DMA blocks per operand and wavefront
  constexpr int NBO = DmaTile<BM>::NB, NC = 2 * NBO;
  static_assert(DmaTile<BM>::NB == MnTile<BM>::NB && DmaTile<BN>::NB == NBO, "copies per operand");
  auto copy_issue = [&](int b, int kt, int n) {
    const int k0 = kt * BK;  // relative to kbeg
    if (n < NBO) {
      if constexpr (P_KC) {
        if (p_copy_on) pd.issue(addrP(b), t.kbeg + k0, n);
      } else {
        pm.issue(addrP(b), k0, klen, n);
      }
    } else {
      if constexpr (Q_KC) qd.issue(addrQ(b), t.kbeg + k0, n - NBO); else qm.issue(addrQ(b), k0, klen, n - NBO);
    }
  };

  // LDS read operations of k sub-step ks: Q fragments then P fragments; a k-contiguous fragment
  // is one 16-byte read, an MN fragment two transpose reads (halves)
  constexpr int RQ = Q_KC ? FN : 2 * FN, RP = P_KC ? FM : 2 * FM, NR = RQ + RP;
  static_assert(NR <= 16, "read slots");
  bf16x8 qa[2][FN], pb[2][FM];
  auto read_op = [&](int b, int ks, int n) {
    if (n < RQ) {
      if constexpr (Q_KC) {
        const int row = wc * WN + n * 32 + (lane & 31);
        const int ch = ks * 2 + (lane >> 5);
        qa[ks & 1][n] = *(const bf16x8*)(bufQ(b) + row * BK + swz<BK>(row, ch) * 8);
      } else {
        const v4i16 h = read_mn_half(bufQ(b), wc * WN + (n >> 1) * 32, ks, n & 1);
        v4i16* dst = (v4i16*)&qa[ks & 1][n >> 1];
        dst[n & 1] = h;
      }
    } else {
      const int m = n - RQ;
      if constexpr (P_KC) {
        const int row = (wr + WR * m) * 32 + (lane & 31);
        const int ch = ks * 2 + (lane >> 5);
        pb[ks & 1][m] = *(const bf16x8*)(bufP(b) + row * BK + swz<BK>(row, ch) * 8);
      } else {
        const v4i16 h = read_mn_half(bufP(b), (wr + WR * (m >> 1)) * 32, ks, m & 1);
        v4i16* dst = (v4i16*)&pb[ks & 1][m >> 1];
        dst[m & 1] = h;
      }
    }
  };
  // ragged reduction: in the last stage, zero the P-fragment k elements at or past the segment
  // end (the copies clamp those rows to the last valid row, so both operands hold finite data)
  auto mask_tail = [&](int kt, int ks) {
    if constexpr (MASK_K) {
      const int kfirst = kt * BK + ks * 16 + 8 * (lane >> 5);
      if (kt * BK + BK > klen) {
#pragma unroll
        for (int j = 0; j < FM; ++j)
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (kfirst + e >= klen) pb[ks & 1][j][e] = (__bf16)0.0f;
      }
    }
  };

  // Schedule of one stage (MPK MFMAs m in each of the 4 k sub-steps ks): every other instruction
  // slips in between MFMAs, so after MFMA (ks, m):
  //   ks < 3:              the LDS read operations of sub-step ks+1, spread over the MPK slots
  //   ks = 0:              the NC DMA copies of the next stage (into the other buffer), spread
  //                        over the MPK slots of sub-step 0 (the earliest issue gives them the
  //                        most time to land before the barrier)
  //   before (3, B0):      wait for this wave's copies, barrier: every wave's copies of the next
  //                        stage have landed, and this buffer is no longer read after this point
  //   ks = 3, m >= B0:     the read operations of sub-step 0 of the next stage
  // The buffer written during stage s was last read before the barrier of stage s-1.
  constexpr int B0 = MPK * 3 / 4;
  auto block_on = [&](int i, int j) {
    return (EPI == EPI_SWIGLU_FWD ? (i % (FN / 2)) < ilim : i < ilim) && j < jlim;
  };
  // one k stage; MASKED: skip the products of empty blocks (a tile with a ragged edge; full tiles
  // run the unmasked copy of the body); MORE: a next stage exists (every stage but the last, which
  // is peeled off so that the others carry no per-slot test of it)
  auto stage = [&](int kt, auto masked_tag, auto more_tag) __attribute__((always_inline)) {
    constexpr bool MASKED = decltype(masked_tag)::value;
    constexpr bool more = decltype(more_tag)::value;
    const int cur = kt & 1, nxt = cur ^ 1;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      mask_tail(kt, ks);
#pragma unroll
      for (int m = 0; m < MPK; ++m) {
        if (ks == 3 && m == B0) {
          __builtin_amdgcn_s_waitcnt(0);
          __syncthreads();
        }
        __builtin_amdgcn_sched_barrier(0);
        if (!MASKED || block_on(m / FM, m % FM))
          acc[m / FM][m % FM] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              qa[ks & 1][m / FM], pb[ks & 1][m % FM], acc[m / FM][m % FM], 0, 0, 0);
        if (ks < 3) {
#pragma unroll
          for (int n = (m * NR) / MPK; n < ((m + 1) * NR) / MPK; ++n) read_op(cur, ks + 1, n);
        }
        if (more) {
          if (ks == 0) {
#pragma unroll
            for (int n = (m * NC) / MPK; n < ((m + 1) * NC) / MPK; ++n) copy_issue(nxt, kt + 1, n);
          }
          if (ks == 3 && m >= B0) {
#pragma unroll
            for (int n = ((m - B0) * NR) / (MPK - B0); n < ((m - B0 + 1) * NR) / (MPK - B0); ++n)
              read_op(nxt, 0, n);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };
  if (nk > 0) {
#pragma unroll
    for (int n = 0; n < NC; ++n) copy_issue(0, 0, n);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
#pragma unroll
    for (int n = 0; n < NR; ++n) read_op(0, 0, n);
    if (jlim == FM && ilim == (EPI == EPI_SWIGLU_FWD ? FN / 2 : FN)) {
      for (int kt = 0; kt < nk - 1; ++kt) stage(kt, std::false_type{}, std::true_type{});
      stage(nk - 1, std::false_type{}, std::false_type{});
    } else {
      for (int kt = 0; kt < nk - 1; ++kt) stage(kt, std::true_type{}, std::true_type{});
      stage(nk - 1, std::true_type{}, std::false_type{});
    }
  }

  // ---- epilogue ------------------------------------------------------------------------------
  // Lane (lane&31, lane>>5) of the wavefront holds, for MFMA block (i, j), output row
  // (wr + WR*j)*32 + (lane&31) of the tile and the 4 consecutive columns
  // i*32 + 8*gq + 4*(lane>>5) + 0..3, gq = 0..3. Per 32-row block j the wavefront converts its
  // values to bf16 (v_cvt_pk_bf16_f32, round to nearest even), parks them in a private LDS area
  // with padded rows (the 8-byte writes of 32 rows land on distinct banks), reads them back as
  // row segments and writes whole 16-byte chunks, 4 to 8 rows of contiguous bytes per
  // instruction. The LDS stages are no longer read once every wavefront is past the loop.
  __syncthreads();
  const int cq = 4 * (lane >> 5), rl = lane & 31;
  uint16_t* ep = lds + wave * kEpWaveElems;
  auto pk2 = [](float a, float b) -> uint32_t {
    bf16x2 v;
    v[0] = (__bf16)a;
    v[1] = (__bf16)b;
    return __builtin_bit_cast(uint32_t, v);
  };
  // read row segments of width W (bf16) out of a [32][W + 4] area and store them
  auto flush = [&](const uint16_t* area, int W, uint16_t* dst, int64_t ld, int row0, int rlim,
                   int col0, int clim, const void* lo, uint64_t ext) {
    const int per_row = W / 8;            // 16-byte chunks per row
    const int rows_per_pass = 64 / per_row;
#pragma unroll
    for (int pass = 0; pass < 32 / rows_per_pass; ++pass) {
      const int row = pass * rows_per_pass + lane / per_row, ch = lane % per_row;
      const uint16_t* src = area + row * (W + 4) + ch * 8;
      const uint2 lo4 = *(const uint2*)src, hi4 = *(const uint2*)(src + 4);
      const int r = row0 + row, c = col0 + ch * 8;
      if (r < rlim && c < clim && MOE_IN(dst + (int64_t)r * ld + c, 16, lo, ext))
        *(uint4*)(dst + (int64_t)r * ld + c) = make_uint4(lo4.x, lo4.y, hi4.x, hi4.y);
    }
  };
  if constexpr (EPI == EPI_STORE && OUT != OUT_BF16) {
    // fp32 staging ([32][W + 4] floats per wavefront, per 64-column half), then per 8 consecutive
    // outputs of a row: optionally the existing values added in fp32, then one rounding (bf16)
    // or none (fp32)
    constexpr int W = WN / 2, PW = W + 4;
    static_assert(32 * PW * 4 <= kEpWaveElems * 2, "fp32 staging area");
    float* epf = (float*)ep;
    const int64_t cofs = (int64_t)t.e * g.c_estride;
    constexpr int per_row = W / 8, rows_per_pass = 64 / per_row;
    constexpr int NP = 32 / rows_per_pass;  // flush passes per 32-row block
#pragma unroll
    for (int hj = 0; hj < 2 * FM; ++hj) {
      const int hlf = hj & 1, j = hj >> 1;
      if (j >= jlim) break;
      const int row0 = t.r0 + (wr + WR * j) * 32, col0 = t.n0 + wc * WN + hlf * W;
      // the existing values this lane adds to, loaded before the staging so that their latency
      // overlaps it
      uint4 oldb[OUT == OUT_BF16_ACC ? NP : 1];
      float4 oldf[OUT == OUT_F32_ACC ? 2 * NP : 1];
      if constexpr (OUT == OUT_BF16_ACC || OUT == OUT_F32_ACC) {
#pragma unroll
        for (int pass = 0; pass < NP; ++pass) {
          const int r = row0 + pass * rows_per_pass + lane / per_row;
          const int c = col0 + (lane % per_row) * 8;
          const bool in = r < t.r_lim && c < g.N_out;
          const int64_t o = cofs + (int64_t)(in ? r : 0) * g.ldc + (in ? c : 0);
          if constexpr (OUT == OUT_BF16_ACC) {
            oldb[pass] = MOE_IN(g.C + o, 16, g.C, g.ext_c) ? *(const uint4*)(g.C + o)
                                                            : make_uint4(0, 0, 0, 0);
          } else {
            const bool ok = MOE_IN(g.Cf + o, 32, g.Cf, g.ext_c);
            oldf[2 * pass] = ok ? *(const float4*)(g.Cf + o) : make_float4(0, 0, 0, 0);
            oldf[2 * pass + 1] = ok ? *(const float4*)(g.Cf + o + 4) : make_float4(0, 0, 0, 0);
          }
        }
      }
#pragma unroll
      for (int ii = 0; ii < FN / 2; ++ii)
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          const int i = hlf * (FN / 2) + ii;
          *(float4*)(epf + rl * PW + ii * 32 + gq * 8 + cq) =
              make_float4(acc[i][j][4 * gq], acc[i][j][4 * gq + 1], acc[i][j][4 * gq + 2],
                          acc[i][j][4 * gq + 3]);
        }
#pragma unroll
      for (int pass = 0; pass < NP; ++pass) {
        const int row = pass * rows_per_pass + lane / per_row, ch = lane % per_row;
        const float* src = epf + row * PW + ch * 8;
        float v[8];
        *(float4*)&v[0] = *(const float4*)src;
        *(float4*)&v[4] = *(const float4*)(src + 4);
        const int r = row0 + row, c = col0 + ch * 8;
        const int64_t o = cofs + (int64_t)r * g.ldc + c;
        if (r < t.r_lim && c < g.N_out &&
            MOE_IN(OUT == OUT_BF16_ACC ? (const void*)(g.C + o) : (const void*)(g.Cf + o),
                   OUT == OUT_BF16_ACC ? 16 : 32, g.Cf, g.ext_c)) {
          if constexpr (OUT == OUT_BF16_ACC) {
            const uint4 old = oldb[pass];
            const uint32_t w[4] = {old.x, old.y, old.z, old.w};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              v[2 * q] += bf16_to_f32(w[q] & 0xffffu);
              v[2 * q + 1] += bf16_to_f32(w[q] >> 16);
            }
            *(uint4*)(g.C + o) = make_uint4(pk2(v[0], v[1]), pk2(v[2], v[3]), pk2(v[4], v[5]),
                                            pk2(v[6], v[7]));
          } else {
            float4* d = (float4*)(g.Cf + o);
            float4 a = *(const float4*)&v[0], b = *(const float4*)&v[4];
            if constexpr (OUT == OUT_F32_ACC) {
              const float4 oa = oldf[2 * pass], ob = oldf[2 * pass + 1];
              a.x += oa.x; a.y += oa.y; a.z += oa.z; a.w += oa.w;
              b.x += ob.x; b.y += ob.y; b.z += ob.z; b.w += ob.w;
            }
            d[0] = a;
            d[1] = b;
          }
        }
      }
    }
  } else if constexpr (EPI == EPI_STORE) {
    uint16_t* C = g.C + (int64_t)t.e * g.c_estride;
    constexpr int PW = WN + 4;
#pragma unroll
    for (int j = 0; j < FM; ++j) {
      if (j >= jlim) break;
#pragma unroll
      for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int gq = 0; gq < 4; ++gq)
          *(uint2*)(ep + rl * PW + i * 32 + gq * 8 + cq) =
              make_uint2(pk2(acc[i][j][4 * gq], acc[i][j][4 * gq + 1]),
                         pk2(acc[i][j][4 * gq + 2], acc[i][j][4 * gq + 3]));
      flush(ep, WN, C, g.ldc, t.r0 + (wr + WR * j) * 32, t.r_lim, t.n0 + wc * WN, g.N_out, g.C,
            g.ext_c);
    }
  } else if constexpr (EPI == EPI_SWIGLU_FWD) {
    // the wavefront's 64 activation columns f0w .. f0w+63: a, g and u each through [32][68]
    constexpr int W = WN / 2, PW = W + 4;
    uint16_t* ea = ep;
    uint16_t* eg = ep + 32 * PW;
    uint16_t* eu = ep + 2 * 32 * PW;
    const int f0w = t.n0 + wc * W;
#pragma unroll
    for (int j = 0; j < FM; ++j) {
      if (j >= jlim) break;
#pragma unroll
      for (int i = 0; i < FN / 2; ++i)
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          float gv[4], uv[4], av[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            gv[q] = (float)(__bf16)acc[i][j][4 * gq + q];
            uv[q] = (float)(__bf16)acc[i + FN / 2][j][4 * gq + q];
            av[q] = gv[q] * sigmoid_f32(gv[q]) * uv[q];
          }
          const int o = rl * PW + i * 32 + gq * 8 + cq;
          *(uint2*)(eg + o) = make_uint2(pk2(gv[0], gv[1]), pk2(gv[2], gv[3]));
          *(uint2*)(eu + o) = make_uint2(pk2(uv[0], uv[1]), pk2(uv[2], uv[3]));
          *(uint2*)(ea + o) = make_uint2(pk2(av[0], av[1]), pk2(av[2], av[3]));
        }
      const int row0 = t.r0 + (wr + WR * j) * 32;
      flush(ea, W, g.C2, g.ldc2, row0, t.r_lim, f0w, g.F, g.C2, g.ext_c2);
      if (g.C) {
        flush(eg, W, g.C, g.ldc, row0, t.r_lim, f0w, g.F, g.C, g.ext_c);
        flush(eu, W, g.C + g.F, g.ldc, row0, t.r_lim, f0w, g.F, g.C, g.ext_c);
      }
    }
  } else {  // EPI_SWIGLU_BWD: acc = da over columns f; g, u come from the saved h13
    // two passes over 64-column halves of the wavefront's 128 columns; per 32-row block the g and
    // u row segments are loaded coalesced into [32][68] areas, replaced in place by dg and du,
    // and stored
    constexpr int W = WN / 2, PW = W + 4, per_row = W / 8, rows_per_pass = 64 / per_row;
    static_assert(2 * 32 * PW <= kEpWaveElems, "g/u staging area");
    uint16_t* e1 = ep;             // g, then dg
    uint16_t* e2 = ep + 32 * PW;   // u, then du
#pragma unroll
    for (int hlf = 0; hlf < 2; ++hlf) {
      const int f0w = t.n0 + wc * WN + hlf * W;
#pragma unroll
      for (int j = 0; j < FM; ++j) {
        if (j >= jlim) break;
        const int row0 = t.r0 + (wr + WR * j) * 32;
        // coalesced loads of the g and u row segments (rows past the segment clamped)
#pragma unroll
        for (int pass = 0; pass < 32 / rows_per_pass; ++pass) {
          const int row = pass * rows_per_pass + lane / per_row, ch = lane % per_row;
          int r = row0 + row;
          if (r > t.r_lim - 1) r = t.r_lim - 1;
          int c = f0w + ch * 8;
          if (c > g.F - 8) c = g.F - 8;
          const uint16_t* hrow = g.H + (int64_t)r * g.ldh + c;
          const bool hok = MOE_IN(hrow, 16, g.H, g.ext_h) && MOE_IN(hrow + g.F, 16, g.H, g.ext_h);
          const uint4 gv = hok ? *(const uint4*)hrow : make_uint4(0, 0, 0, 0);
          const uint4 uv = hok ? *(const uint4*)(hrow + g.F) : make_uint4(0, 0, 0, 0);
          uint16_t* d1 = e1 + row * PW + ch * 8;
          uint16_t* d2 = e2 + row * PW + ch * 8;
          *(uint2*)d1 = make_uint2(gv.x, gv.y);
          *(uint2*)(d1 + 4) = make_uint2(gv.z, gv.w);
          *(uint2*)d2 = make_uint2(uv.x, uv.y);
          *(uint2*)(d2 + 4) = make_uint2(uv.z, uv.w);
        }
#pragma unroll
        for (int ii = 0; ii < FN / 2; ++ii)
#pragma unroll
          for (int gq = 0; gq < 4; ++gq) {
            const int i = hlf * (FN / 2) + ii;
            const int o = rl * PW + ii * 32 + gq * 8 + cq;
            const uint2 gh = *(const uint2*)(e1 + o), uh = *(const uint2*)(e2 + o);
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
            *(uint2*)(e1 + o) = make_uint2(pk2(dg[0], dg[1]), pk2(dg[2], dg[3]));
            *(uint2*)(e2 + o) = make_uint2(pk2(du[0], du[1]), pk2(du[2], du[3]));
          }
        flush(e1, W, g.C, g.ldc, row0, t.r_lim, f0w, g.F, g.C, g.ext_c);
        flush(e2, W, g.C + g.F, g.ldc, row0, t.r_lim, f0w, g.F, g.C, g.ext_c);
      }
    }
  }
}

#define MOE_GEMM_KERNEL(name, P_KC, Q_KC, SCHED, EPI)                                          \
  __global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(kWaves / 4, kWaves / 4))) void name( \
      GemmArgs g) {                                                                            \
    __shared__ __attribute__((aligned(1024))) uint16_t lds[kLdsElems];                         \
    gemm_body<kBM, kBN, P_KC, Q_KC, SCHED, EPI>(g, lds, blockIdx.x);                           \
  }

MOE_GEMM_KERNEL(moe_fprop_w13_swiglu, true, true, SCHED_ROWS, EPI_SWIGLU_FWD)
MOE_GEMM_KERNEL(moe_fprop_w2, true, true, SCHED_ROWS, EPI_STORE)
MOE_GEMM_KERNEL(moe_dgrad_w13, true, false, SCHED_ROWS, EPI_STORE)
MOE_GEMM_KERNEL(moe_wgrad_w13, false, false, SCHED_KSEG, EPI_STORE)

// weight gradients accumulated into existing storage, or kept in fp32
#define MOE_WGRAD_KERNEL(name, OUT)                                                             \
  __global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(kWaves / 4, kWaves / 4))) void name( \
      GemmArgs g) {                                                                            \
    __shared__ __attribute__((aligned(1024))) uint16_t lds[kLdsElems];                         \
    gemm_body<kBM, kBN, false, false, SCHED_KSEG, EPI_STORE, OUT>(g, lds, blockIdx.x);         \
  }

MOE_WGRAD_KERNEL(moe_wgrad_w13_accum, OUT_BF16_ACC)
MOE_WGRAD_KERNEL(moe_wgrad_w13_f32, OUT_F32)
MOE_WGRAD_KERNEL(moe_wgrad_w13_f32_accum, OUT_F32_ACC)

// kernel of the W13 weight-gradient GEMM for the shape's storage flags
void (*wgrad_w13_kernel(const moe_shape& s))(GemmArgs) {
  const bool acc = (s.flags & MOE_WGRAD_ACCUMULATE) != 0, f32 = (s.flags & MOE_WGRAD_F32) != 0;
  if (f32) return acc ? moe_wgrad_w13_f32_accum : moe_wgrad_w13_f32;
  return acc ? moe_wgrad_w13_accum : moe_wgrad_w13;
}

// W2 DGRAD (+ SwiGLU derivative) and W2 WGRAD in one launch: the first grid_d workgroups take
// DGRAD's row tiles (the longer tiles: k = D), the others WGRAD's tiles. Both read dy and write
// disjoint outputs (dh13, dW2), so WGRAD's tiles run on the CUs that DGRAD's last, partly filled
// round of workgroups leaves idle. grid_d is a multiple of 8, so that every tile keeps its XCD.
template <int OUT>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(kWaves / 4, kWaves / 4)))
void moe_w2_backward(GemmArgs gd, GemmArgs gw, int grid_d) {
  __shared__ __attribute__((aligned(1024))) uint16_t lds[kLdsElems];
  const int b = blockIdx.x;
  if (b < grid_d)
    gemm_body<kBM, kBN, true, false, SCHED_ROWS, EPI_SWIGLU_BWD>(gd, lds, b);
  else
    gemm_body<kBM, kBN, false, false, SCHED_KSEG, EPI_STORE, OUT>(gw, lds, b - grid_d);
}

void (*w2_backward_kernel(const moe_shape& s))(GemmArgs, GemmArgs, int) {
  const bool acc = (s.flags & MOE_WGRAD_ACCUMULATE) != 0, f32 = (s.flags & MOE_WGRAD_F32) != 0;
  if (f32) return acc ? moe_w2_backward<OUT_F32_ACC> : moe_w2_backward<OUT_F32>;
  return acc ? moe_w2_backward<OUT_BF16_ACC> : moe_w2_backward<OUT_BF16>;
}

hipError_t launch(void (*kernel)(GemmArgs), const GemmArgs& g, int grid, hipStream_t st) {
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL(kernel, dim3(grid), dim3(kThreads), 0, st, g);
  return hipGetLastError();
}

// an extent in bytes as the kernels see it (checked builds: shortened by g_checked_shrink)
uint64_t ext(int64_t bytes) {
#ifdef MOE_CHECKED
  return bytes > g_checked_shrink ? (uint64_t)(bytes - g_checked_shrink) : 0;
#else
  return (uint64_t)bytes;
#endif
}

GemmArgs rows_args(const moe_shape& s, const PlanPtrs& p) {
  GemmArgs g{};
  g.F = (int)s.F;
  g.E = (int)s.E;
  g.offsets = p.offsets;
  g.mtiles = (const int2*)p.mtiles;
  g.mtile_start = p.tstart;
  g.mtile_count = p.status + 1;
  return g;
}

// the plan's worst-case row-tile count times the column tiles
int64_t rows_grid64(const moe_shape& s, int64_t ntn) {
  const int64_t mt_max = ceil_div(s.T * s.K, kRowTile) + s.E;
  return mt_max * ntn;
}

// callers have checked gemm_max_grid(s) <= INT32_MAX
int rows_grid(const moe_shape& s, int ntn) { return (int)rows_grid64(s, ntn); }

}  // namespace

int64_t gemm_max_grid(const moe_shape& s) {
  const int64_t fprop_w13 = rows_grid64(s, ceil_div(s.F, kBN / 2));
  const int64_t by_d = rows_grid64(s, ceil_div(s.D, kBN));  // W2 FPROP, W13 DGRAD
  const int64_t w2_bwd = (int64_t)align_up((size_t)rows_grid64(s, ceil_div(s.F, kBN)), 8) +
                         s.E * ceil_div(s.D, kBM) * ceil_div(s.F, kBN);
  const int64_t wgrad_w13 = s.E * ceil_div(2 * s.F, kBM) * ceil_div(s.D, kBN);
  return std::max(std::max(fprop_w13, by_d), std::max(w2_bwd, wgrad_w13));
}

hipError_t launch_fprop_w13(const moe_shape& s, const PlanPtrs& p, const uint16_t* xg,
                            const uint16_t* w13, uint16_t* h13, uint16_t* a, hipStream_t st,
                            bool gather) {
  GemmArgs g = rows_args(s, p);
  const int64_t N = s.T * s.K;
  g.P = xg; g.ldp = s.D; g.ext_p = ext(2 * N * s.D);
  if (gather) {  // xg is x: P rows come from the routed rows' tokens
    g.gather_src = p.src;
    g.gather_k = (int)s.K;
    g.ext_p = ext(2 * s.T * s.D);
    g.ext_src = ext(4 * N);
  }
  g.Q = w13; g.ldq = s.D; g.q_estride = 2 * s.F * s.D; g.ext_q = ext(2 * s.E * 2 * s.F * s.D);
  g.C = h13; g.ldc = 2 * s.F; g.ext_c = ext(2 * N * 2 * s.F);
  g.C2 = a; g.ldc2 = s.F; g.ext_c2 = ext(2 * N * s.F);
  g.N_out = (int)s.F; g.Kdim = (int)s.D;
  const int ntn = (int)ceil_div(s.F, kBN / 2);
  return launch(moe_fprop_w13_swiglu, g, rows_grid(s, ntn), st);
}

hipError_t launch_fprop_w2(const moe_shape& s, const PlanPtrs& p, const uint16_t* a,
                           const uint16_t* w2, uint16_t* y, hipStream_t st) {
  GemmArgs g = rows_args(s, p);
  const int64_t N = s.T * s.K;
  g.P = a; g.ldp = s.F; g.ext_p = ext(2 * N * s.F);
  g.Q = w2; g.ldq = s.F; g.q_estride = s.D * s.F; g.ext_q = ext(2 * s.E * s.D * s.F);
  g.C = y; g.ldc = s.D; g.ext_c = ext(2 * N * s.D);
  g.N_out = (int)s.D; g.Kdim = (int)s.F;
  const int ntn = (int)ceil_div(s.D, kBN);
  return launch(moe_fprop_w2, g, rows_grid(s, ntn), st);
}

static GemmArgs dgrad_w2_args(const moe_shape& s, const PlanPtrs& p, const uint16_t* dy,
                              const uint16_t* w2, const uint16_t* h13, uint16_t* dh13) {
  GemmArgs g = rows_args(s, p);
  const int64_t N = s.T * s.K;
  g.P = dy; g.ldp = s.D; g.ext_p = ext(2 * N * s.D);
  g.Q = w2; g.ldq = s.F; g.q_estride = s.D * s.F;  // w2[e] read as [k = d][c = f]
  g.ext_q = ext(2 * s.E * s.D * s.F);
  g.C = dh13; g.ldc = 2 * s.F; g.ext_c = ext(2 * N * 2 * s.F);
  g.H = h13; g.ldh = 2 * s.F; g.ext_h = ext(2 * N * 2 * s.F);
  g.N_out = (int)s.F; g.Kdim = (int)s.D;
  return g;
}

static GemmArgs wgrad_w2_args(const moe_shape& s, const PlanPtrs& p, const uint16_t* dy,
                              const uint16_t* a, void* dw2) {
  GemmArgs g{};
  g.F = (int)s.F; g.E = (int)s.E; g.offsets = p.offsets; g.lpt = p.lpt;
  const int64_t N = s.T * s.K, wb = (s.flags & MOE_WGRAD_F32) ? 4 : 2;
  g.P = dy; g.ldp = s.D; g.ext_p = ext(2 * N * s.D);  // [k = routed row][r = d]
  g.Q = a; g.ldq = s.F; g.ext_q = ext(2 * N * s.F);   // [k = routed row][c = f]
  g.C = (uint16_t*)dw2; g.Cf = (float*)dw2; g.ldc = s.F; g.c_estride = s.D * s.F;
  g.ext_c = ext(wb * s.E * s.D * s.F);
  g.M_out = (int)s.D; g.N_out = (int)s.F;
  return g;
}

hipError_t launch_w2_backward(const moe_shape& s, const PlanPtrs& p, const uint16_t* dy,
                              const uint16_t* w2, const uint16_t* h13, uint16_t* dh13,
                              const uint16_t* a, void* dw2, hipStream_t st) {
  const int grid_d = (int)align_up((size_t)rows_grid(s, (int)ceil_div(s.F, kBN)), 8);
  const int grid_w = (int)(s.E * ceil_div(s.D, kBM) * ceil_div(s.F, kBN));
  hipLaunchKernelGGL(w2_backward_kernel(s), dim3(grid_d + grid_w), dim3(kThreads), 0, st,
                     dgrad_w2_args(s, p, dy, w2, h13, dh13), wgrad_w2_args(s, p, dy, a, dw2),
                     grid_d);
  return hipGetLastError();
}

hipError_t launch_dgrad_w13(const moe_shape& s, const PlanPtrs& p, const uint16_t* dh13,
                            const uint16_t* w13, uint16_t* dxg, hipStream_t st) {
  GemmArgs g = rows_args(s, p);
  const int64_t N = s.T * s.K;
  g.P = dh13; g.ldp = 2 * s.F; g.ext_p = ext(2 * N * 2 * s.F);
  g.Q = w13; g.ldq = s.D; g.q_estride = 2 * s.F * s.D;  // w13[e] read as [k = j][c = d]
  g.ext_q = ext(2 * s.E * 2 * s.F * s.D);
  g.C = dxg; g.ldc = s.D; g.ext_c = ext(2 * N * s.D);
  g.N_out = (int)s.D; g.Kdim = (int)(2 * s.F);
  const int ntn = (int)ceil_div(s.D, kBN);
  return launch(moe_dgrad_w13, g, rows_grid(s, ntn), st);
}


hipError_t launch_wgrad_w13(const moe_shape& s, const PlanPtrs& p, const uint16_t* dh13,
                            const uint16_t* xg, void* dw13, hipStream_t st) {
  GemmArgs g{};
  g.F = (int)s.F; g.E = (int)s.E; g.offsets = p.offsets; g.lpt = p.lpt;
  const int64_t N = s.T * s.K, wb = (s.flags & MOE_WGRAD_F32) ? 4 : 2;
  g.P = dh13; g.ldp = 2 * s.F; g.ext_p = ext(2 * N * 2 * s.F);  // [k = routed row][r = j]
  g.Q = xg; g.ldq = s.D; g.ext_q = ext(2 * N * s.D);            // [k = routed row][c = d]
  g.C = (uint16_t*)dw13; g.Cf = (float*)dw13; g.ldc = s.D; g.c_estride = 2 * s.F * s.D;
  g.ext_c = ext(wb * s.E * 2 * s.F * s.D);
  g.M_out = (int)(2 * s.F); g.N_out = (int)s.D;
  const int grid = (int)(s.E * ceil_div(2 * s.F, kBM) * ceil_div(s.D, kBN));
  return launch(wgrad_w13_kernel(s), g, grid, st);
}

#ifdef MOE_CHECKED
hipError_t oob_counter_gemm(unsigned int** p) { return oob_counter_address(p); }
#endif

}  // namespace moe
