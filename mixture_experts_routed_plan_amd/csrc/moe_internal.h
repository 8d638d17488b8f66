// Internal declarations of the routed-experts library: buffer layouts (closed forms of the
// shape), bf16 helpers for device code, and the kernel launchers the C ABI sequences.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "moe_routed.h"  // include/ is on the include path

namespace moe {

// ------------------------------------------------------------------------------------------
// sizes and layouts

constexpr int kPlanChunk = 1024;  // slots per plan workgroup (a multiple of 64)
// Row tiles of the row-ragged GEMMs: an expert's rows in tiles of kRowTile (the last one holds
// the rest). The plan lists (expert, first row) of every tile, experts ascending, and each
// expert's first list index. (Splitting each expert's rows into equal tiles of 32-row multiples
// instead measured the same at 256 rows and slower at 224 or 192.)
constexpr int kRowTile = 256;
constexpr int kStatusWords = 16;  // [0] out-of-range ids, [1] row tiles in the list

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }
inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

struct PlanLayout {
  int64_t N, E, NB;
  size_t status, counts, offsets, pos, src, blkhist, blkbad, lpt, tstart, mtiles, total;
};

inline PlanLayout plan_layout(const moe_shape& s) {
  PlanLayout L{};
  L.N = s.T * s.K;
  L.E = s.E;
  L.NB = ceil_div(L.N, kPlanChunk);
  size_t o = 0;
  auto take = [&](size_t bytes) {
    size_t at = o;
    o = align_up(o + bytes, 256);
    return at;
  };
  L.status = take(sizeof(int32_t) * kStatusWords);
  L.counts = take(sizeof(int32_t) * L.E);
  L.offsets = take(sizeof(int32_t) * (L.E + 1));
  L.pos = take(sizeof(int32_t) * L.N);
  L.src = take(sizeof(int32_t) * L.N);
  L.blkhist = take(sizeof(int32_t) * L.E * L.NB);
  L.blkbad = take(sizeof(int32_t) * L.NB);
  L.lpt = take(sizeof(int32_t) * L.E);
  L.tstart = take(sizeof(int32_t) * L.E);
  L.mtiles = take(sizeof(int32_t) * 2 * (ceil_div(L.N, kRowTile) + L.E));
  L.total = o;
  return L;
}

// Unless MOE_KEEP_XG asks for xg, and when x spans less than 4 GiB (32-bit copy offsets from the
// base of x), the gate/up GEMM gathers x's token rows through the plan's src instead of reading
// xg, so the forward neither permutes nor saves xg (the backward permutes it into its workspace
// for the W13 weight gradient)
inline bool gather_x(const moe_shape& s) {
  return !(s.flags & MOE_KEEP_XG) && (uint64_t)s.T * (uint64_t)s.D * 2 < (1ull << 32);
}

struct SavedLayout {
  size_t xg, h13, a, y, total;
};

// With MOE_RECOMPUTE h13 and a are not saved (recomputed in the backward), and with gather_x no
// xg; the offsets of what is not saved are unused.
inline SavedLayout saved_layout(const moe_shape& s) {
  SavedLayout L{};
  const size_t N = (size_t)(s.T * s.K), D = (size_t)s.D, F = (size_t)s.F;
  const bool re = (s.flags & MOE_RECOMPUTE) != 0;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    size_t at = o;
    o = align_up(o + bytes, 256);
    return at;
  };
  L.xg = gather_x(s) ? 0 : take(2 * N * D);
  L.h13 = re ? 0 : take(2 * N * 2 * F);
  L.a = re ? 0 : take(2 * N * F);
  L.y = take(2 * N * D);
  L.total = o;
  return L;
}

// Workspace: the forward without saving keeps xg (unless gather_x), a, y here (with MOE_RECOMPUTE
// only a); the backward keeps dy and dh13, and once dy is dead (after the W2 weight gradient) its
// region holds xg for the W13 weight gradient (gather_x: permuted there from x) and then dxg;
// with MOE_RECOMPUTE also the recomputed a (a_re), and the recomputed h13 sits where dh13 goes
// (the SwiGLU-derivative GEMM reads each g, u and writes its dg, du in place).
struct WorkLayout {
  size_t xg, a, y, fwd_total;
  size_t dy, dh13, a_re, bwd_total;
  size_t total;
};

inline WorkLayout work_layout(const moe_shape& s) {
  WorkLayout L{};
  const size_t N = (size_t)(s.T * s.K), D = (size_t)s.D, F = (size_t)s.F;
  L.xg = 0;
  L.a = gather_x(s) ? 0 : align_up(2 * N * D, 256);  // no xg when the permute is fused
  L.y = L.a + align_up(2 * N * F, 256);
  L.fwd_total = L.y + align_up(2 * N * D, 256);
  L.dy = 0;
  L.dh13 = align_up(2 * N * D, 256);
  L.a_re = L.dh13 + align_up(2 * N * 2 * F, 256);
  L.bwd_total = (s.flags & MOE_RECOMPUTE) ? L.a_re + align_up(2 * N * F, 256) : L.a_re;
  L.total = L.fwd_total > L.bwd_total ? L.fwd_total : L.bwd_total;
  return L;
}

// ------------------------------------------------------------------------------------------
// device helpers

__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// fp32 -> bf16, round to nearest even; NaN -> canonical quiet NaN
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16(lo) | (f32_to_bf16(hi) << 16);
}

// logistic sigmoid in fp32: hardware exp2 (v_exp_f32) and reciprocal (v_rcp_f32, 1 ulp) instead
// of the IEEE division sequence; the result feeds a bf16 rounding
__device__ __forceinline__ float sigmoid_f32(float z) {
  return __builtin_amdgcn_rcpf(1.0f + __expf(-z));
}

// ------------------------------------------------------------------------------------------
// checked builds (compiled with MOE_CHECKED into libmoe_routed_checked.so): the kernels test
// their global memory accesses against the extent of the buffer each belongs to. An access
// outside is not made (a copy or store is skipped, a load reads zeros) and is counted in a device
// word of the kernel's source file, which moe_checked_violations sums on the host. In the
// product build the tests compile to nothing.
#ifdef MOE_CHECKED
static __device__ unsigned int g_oob_count;
__device__ __forceinline__ bool moe_check(bool ok) {
  if (!ok) atomicAdd(&g_oob_count, 1u);
  return ok;
}
// [p, p + n) lies within [lo, lo + bytes)
__device__ __forceinline__ bool moe_check_range(const void* p, uint64_t n, const void* lo,
                                                uint64_t bytes) {
  const uint64_t a = (uint64_t)(uintptr_t)p, b = (uint64_t)(uintptr_t)lo;
  return moe_check(lo != nullptr && a >= b && a - b <= bytes && n <= bytes - (a - b));
}
#define MOE_CHECK(cond) ::moe::moe_check(cond)
#define MOE_IN(p, n, lo, bytes) ::moe::moe_check_range((p), (n), (lo), (bytes))
// the device address of this source file's counter
static inline hipError_t oob_counter_address(unsigned int** p) {
  return hipGetSymbolAddress((void**)p, HIP_SYMBOL(g_oob_count));
}
hipError_t oob_counter_plan(unsigned int** p);
hipError_t oob_counter_rowops(unsigned int** p);
hipError_t oob_counter_gemm(unsigned int** p);
// host side: every extent the GEMM launchers pass is shortened by this many bytes (a test of the
// checks themselves: accesses near the end of a buffer then count although they are valid)
extern int64_t g_checked_shrink;
#else
#define MOE_CHECK(cond) true
#define MOE_IN(p, n, lo, bytes) true
#endif

// ------------------------------------------------------------------------------------------
// launchers (return hipSuccess or the launch error)

struct PlanPtrs {
  int32_t* status;
  int32_t* counts;
  int32_t* offsets;
  int32_t* pos;
  int32_t* src;
  int32_t* blkhist;
  int32_t* blkbad;
  int32_t* lpt;
  int32_t* tstart;
  int32_t* mtiles;
};

inline PlanPtrs plan_ptrs(const PlanLayout& L, void* base) {
  char* b = (char*)base;
  PlanPtrs p;
  p.status = (int32_t*)(b + L.status);
  p.counts = (int32_t*)(b + L.counts);
  p.offsets = (int32_t*)(b + L.offsets);
  p.pos = (int32_t*)(b + L.pos);
  p.src = (int32_t*)(b + L.src);
  p.blkhist = (int32_t*)(b + L.blkhist);
  p.blkbad = (int32_t*)(b + L.blkbad);
  p.lpt = (int32_t*)(b + L.lpt);
  p.tstart = (int32_t*)(b + L.tstart);
  p.mtiles = (int32_t*)(b + L.mtiles);
  return p;
}

hipError_t launch_plan_hist(const moe_shape& s, const PlanLayout& L, const PlanPtrs& p,
                            const void* ids, hipStream_t st);
hipError_t launch_plan_scan(const moe_shape& s, const PlanLayout& L, const PlanPtrs& p,
                            hipStream_t st);
hipError_t launch_plan_scatter(const moe_shape& s, const PlanLayout& L, const PlanPtrs& p,
                               const void* ids, hipStream_t st);

hipError_t launch_permute(const moe_shape& s, const int32_t* pos, const uint16_t* x, uint16_t* xg,
                          hipStream_t st);
// out[t] = bf16(sum_k w_k * rows[pos[t*K+k]]) with w_k = scores[t*K+k], or 1 when scores == null
hipError_t launch_combine(const moe_shape& s, const int32_t* pos, const uint16_t* rows,
                          const float* scores, uint16_t* out, hipStream_t st);
hipError_t launch_combine_bwd(const moe_shape& s, const int32_t* pos, const uint16_t* dout,
                              const uint16_t* y, const float* scores, uint16_t* dy,
                              float* dscores, hipStream_t st);

// router: logits[T,E] -> ids[T,K] (shape.ids_dtype), weights[T,K]; arguments validated by the caller
hipError_t launch_route(const moe_shape& s, const moe_router& r, const float* logits, void* ids,
                        float* weights, hipStream_t st);

// grouped GEMMs
// the largest workgroup count of any grouped-GEMM launch for this shape (launch grids and tile
// indices are 32-bit)
int64_t gemm_max_grid(const moe_shape& s);
// gather: xg is x[T,D] and the P rows are gathered through the plan's src (fused permute)
hipError_t launch_fprop_w13(const moe_shape& s, const PlanPtrs& p, const uint16_t* xg,
                            const uint16_t* w13, uint16_t* h13, uint16_t* a, hipStream_t st,
                            bool gather = false);

hipError_t launch_fprop_w2(const moe_shape& s, const PlanPtrs& p, const uint16_t* a,
                           const uint16_t* w2, uint16_t* y, hipStream_t st);
// W2 DGRAD (+ SwiGLU derivative) and W2 WGRAD in one launch; weight gradients in bf16 or fp32
// storage, overwritten or accumulated (shape flags)
hipError_t launch_w2_backward(const moe_shape& s, const PlanPtrs& p, const uint16_t* dy,
                              const uint16_t* w2, const uint16_t* h13, uint16_t* dh13,
                              const uint16_t* a, void* dw2, hipStream_t st);
hipError_t launch_dgrad_w13(const moe_shape& s, const PlanPtrs& p, const uint16_t* dh13,
                            const uint16_t* w13, uint16_t* dxg, hipStream_t st);
hipError_t launch_wgrad_w13(const moe_shape& s, const PlanPtrs& p, const uint16_t* dh13,
                            const uint16_t* xg, void* dw13, hipStream_t st);

}  // namespace moe
