// Routing plan on the GPU: a stable counting sort of the T*K routed slots by expert id.
//
// Dist-MoE 0.1.0 (PyPI page), "Understand the execution model": the routing metadata is generated
// on the GPU from the caller's expert ids. TeraMoE README, worker list: a scheduler forms
// per-expert compute batches -- here the row-tile list the grouped GEMMs walk.
//
// Three launches, all sized by the shape only (nothing is read back to the host):
//   1. moe_plan_hist    one wavefront per chunk of kPlanChunk slots: expert histogram in LDS.
//   2. moe_plan_scan    one workgroup: per-expert scan over chunks (chunk bases), counts, the
//                     exclusive scan of counts (offsets), the row-tile list of 256-row tiles
//                     with each expert's first index in it, the expert order by decreasing
//                     count, the out-of-range total.
//   3. moe_plan_scatter one wavefront per chunk, slots in ascending order, 64 at a time: lanes that
//                     share an expert id find each other with one ballot per id bit, take
//                     consecutive rows after the expert's running base in lane order, and the
//                     lowest such lane advances the base. This keeps the order of equal ids
//                     (stable), so pos/src are unique and match a sequential counting sort.
#include "moe_internal.h"

namespace moe {
namespace {

template <typename IdT>
__device__ __forceinline__ int load_expert(const IdT* ids, int i, int E) {
  const IdT v = ids[i];
  return (v >= 0 && v < (IdT)E) ? (int)v : -1;
}

template <typename IdT>
__global__ __launch_bounds__(64) void moe_plan_hist(const IdT* __restrict__ ids, int N, int E,
                                                  int NB, int32_t* __restrict__ blkhist,
                                                  int32_t* __restrict__ blkbad) {
  __shared__ int32_t h[MOE_MAX_EXPERTS];
  const int lane = threadIdx.x, b = blockIdx.x;
  for (int e = lane; e < E; e += 64) h[e] = 0;
  __syncthreads();
  // every id of the chunk is loaded before the first count, so the loads are in flight together
  constexpr int kPer = kPlanChunk / 64;
  const int lo = b * kPlanChunk, hi = min(N, lo + kPlanChunk);
  int v[kPer];
#pragma unroll
  for (int q = 0; q < kPer; ++q) {
    const int i = lo + lane + 64 * q;
    v[q] = i < hi ? load_expert(ids, i, E) : -2;  // -2: past the end of the slots
  }
  int bad = 0;
#pragma unroll
  for (int q = 0; q < kPer; ++q) {
    if (v[q] >= 0)
      atomicAdd(&h[v[q]], 1);
    else if (v[q] == -1)
      ++bad;
  }
  __syncthreads();
  for (int e = lane; e < E; e += 64) blkhist[(int64_t)e * NB + b] = h[e];
  for (int off = 32; off > 0; off >>= 1) bad += __shfl_xor(bad, off);
  if (lane == 0) blkbad[b] = bad;
}

// inclusive scan over the 1024 threads of the workgroup (scratch: 16 ints of LDS)
__device__ __forceinline__ int block_scan_1024(int v, int32_t* wsum) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(v, off);
    if (lane >= off) v += o;
  }
  if (lane == 63) wsum[wave] = v;
  __syncthreads();
  if (wave == 0) {
    int w = lane < 16 ? wsum[lane] : 0;
    for (int off = 1; off < 16; off <<= 1) {
      const int o = __shfl_up(w, off);
      if (lane >= off) w += o;
    }
    if (lane < 16) wsum[lane] = w;
  }
  __syncthreads();
  const int add = wave > 0 ? wsum[wave - 1] : 0;
  __syncthreads();  // wsum may be reused by the next call
  return v + add;
}

// The part of the scan kernel after the per-expert counts (every thread of the 1024 calls it;
// thread e < E holds cnt = counts[e], every thread a partial count badp of out-of-range ids): counts, offsets (also left in s_off[0..E]), the three
// row-tile list, the longest-first expert order, src = -1 past the last routed row, the status.
__device__ void plan_finish(int N, int E, int cnt, int badp, int32_t* s_cnt, int32_t* s_off,
                            int32_t* wsum, int32_t* status, int32_t* counts, int32_t* offsets,
                            int32_t* lpt, int32_t* src, int32_t* tstart, int32_t* mtiles) {
  const int tid = threadIdx.x;
  if (tid < E) counts[tid] = cnt;
  s_cnt[tid] = cnt;
  const int incl = block_scan_1024(cnt, wsum);
  s_off[tid] = incl - cnt;
  if (tid == 1023) s_off[MOE_MAX_EXPERTS] = incl;
  __syncthreads();
  const int nvalid = s_off[MOE_MAX_EXPERTS];
  if (tid < E) offsets[tid] = s_off[tid];
  if (tid == 0) offsets[E] = nvalid;

  // row-tile list: (expert, first row) of every row tile of kRowTile rows (the last of an expert
  // holds the rest), experts ascending, and each expert's first index in the list
  {
    const int nt = tid < E ? (cnt + kRowTile - 1) / kRowTile : 0;
    const int ti = block_scan_1024(nt, wsum);
    if (tid < E) {
      int2* list = (int2*)mtiles;
      const int start = ti - nt;
      tstart[tid] = start;
      for (int q = 0; q < nt; ++q)
        if (MOE_CHECK(start + q < (N + kRowTile - 1) / kRowTile + E))
          list[start + q] = make_int2(tid, s_off[tid] + q * kRowTile);
    }
    if (tid == 1023) status[1] = ti;
  }

  // experts by decreasing count (ties: lower index first)
  if (tid < E) {
    int rank = 0;
    for (int e2 = 0; e2 < E; ++e2) {
      const int c2 = s_cnt[e2];
      rank += (c2 > cnt) || (c2 == cnt && e2 < tid);
    }
    lpt[rank] = tid;
  }

  // rows past the last routed row have no source slot
  for (int r = nvalid + tid; r < N; r += 1024) src[r] = -1;

  const int bad = block_scan_1024(badp, wsum);
  if (tid == 1023) status[0] = bad;
  if (tid == 0)
    for (int w = 2; w < kStatusWords; ++w) status[w] = 0;
}

__global__ __launch_bounds__(1024) void moe_plan_scan(int N, int E, int NB, int32_t* status,
                                                    int32_t* counts, int32_t* offsets,
                                                    int32_t* blkhist, const int32_t* blkbad,
                                                    int32_t* lpt, int32_t* src, int32_t* tstart,
                                                    int32_t* mtiles) {
  __shared__ int32_t s_cnt[MOE_MAX_EXPERTS];
  __shared__ int32_t s_off[MOE_MAX_EXPERTS + 1];
  __shared__ int32_t wsum[16];
  const int tid = threadIdx.x;

  // chunk bases within each expert (exclusive scan over chunks, in place) and the counts
  // (the counts of a batch of chunks are loaded before any of them is overwritten, so the loads
  // of a batch are in flight together)
  int cnt = 0;
  if (tid < E) {
    constexpr int kBatch = 32;
    int32_t* row = blkhist + (int64_t)tid * NB;
    for (int b0 = 0; b0 < NB; b0 += kBatch) {
      int v[kBatch];
#pragma unroll
      for (int q = 0; q < kBatch; ++q) v[q] = b0 + q < NB ? row[b0 + q] : 0;
#pragma unroll
      for (int q = 0; q < kBatch; ++q) {
        if (b0 + q < NB) row[b0 + q] = cnt;
        cnt += v[q];
      }
    }
  }
  // out-of-range total: per-thread partial sums over the chunks
  int badp = 0;
  for (int b = tid; b < NB; b += 1024) badp += blkbad[b];
  plan_finish(N, E, cnt, badp, s_cnt, s_off, wsum, status, counts, offsets, lpt, src, tstart,
              mtiles);
}

// Orders a wavefront's LDS accesses before and after it, across its lanes (every lane's base
// reads before the leaders' base updates, and those before the next group's reads), without
// waiting for the wavefront's global stores.
__device__ __forceinline__ void lds_wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
}

// Lanes of a wavefront holding the same expert id (ok lanes only) find each other with one ballot
// per id bit; returns the lane's rank among its peers (lane order) and their number.
__device__ __forceinline__ void peer_rank(bool ok, int v, int nbits, int& rank, int& cnt) {
  const int lane = threadIdx.x & 63;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  uint64_t peers = __ballot(ok);
  for (int bit = 0; bit < nbits; ++bit) {
    const bool one = ((v >> bit) & 1) != 0;
    const uint64_t m = __ballot(ok && one);
    peers &= one ? m : ~m;
  }
  rank = __popcll(peers & below);
  cnt = __popcll(peers);
}

template <typename IdT>
__global__ __launch_bounds__(64) void moe_plan_scatter(const IdT* __restrict__ ids, int N, int E,
                                                     int NB, int nbits,
                                                     const int32_t* __restrict__ offsets,
                                                     const int32_t* __restrict__ blkhist,
                                                     int32_t* __restrict__ pos,
                                                     int32_t* __restrict__ src) {
  __shared__ int32_t base[MOE_MAX_EXPERTS];
  const int lane = threadIdx.x, b = blockIdx.x;
  // the chunk's ids are loaded up front, their loads in flight together with the bases'
  constexpr int kPer = kPlanChunk / 64;
  const int lo = b * kPlanChunk, hi = min(N, lo + kPlanChunk);
  int vv[kPer];
#pragma unroll
  for (int q = 0; q < kPer; ++q) {
    const int i = lo + lane + 64 * q;
    vv[q] = i < hi ? load_expert(ids, i, E) : -1;
  }
  for (int e = lane; e < E; e += 64) base[e] = offsets[e] + blkhist[(int64_t)e * NB + b];
  __syncthreads();
#pragma unroll
  for (int q = 0; q < kPer; ++q) {
    const int i0 = lo + 64 * q;
    if (i0 >= hi) break;  // uniform
    const int i = i0 + lane;
    const bool in = i < hi;
    const int v = vv[q];
    const bool ok = v >= 0;
    int rank, cnt;
    peer_rank(ok, v, nbits, rank, cnt);
    int p = -1;
    if (ok) p = base[v] + rank;
    lds_wave_sync();  // the workgroup is this one wavefront
    if (in) pos[i] = p;
    if (ok && MOE_CHECK(p >= 0 && p < N)) src[p] = i;
    if (ok && rank == 0) base[v] += cnt;
    lds_wave_sync();
  }
}

}  // namespace

hipError_t launch_plan_hist(const moe_shape& s, const PlanLayout& L, const PlanPtrs& p,
                            const void* ids, hipStream_t st) {
  const int N = (int)L.N, E = (int)s.E, NB = (int)L.NB;
  if (s.ids_dtype == MOE_IDS_I64)
    hipLaunchKernelGGL(moe_plan_hist<int64_t>, dim3(NB), dim3(64), 0, st, (const int64_t*)ids, N,
                       E, NB, p.blkhist, p.blkbad);
  else
    hipLaunchKernelGGL(moe_plan_hist<int32_t>, dim3(NB), dim3(64), 0, st, (const int32_t*)ids, N,
                       E, NB, p.blkhist, p.blkbad);
  return hipGetLastError();
}

hipError_t launch_plan_scan(const moe_shape& s, const PlanLayout& L, const PlanPtrs& p,
                            hipStream_t st) {
  hipLaunchKernelGGL(moe_plan_scan, dim3(1), dim3(1024), 0, st, (int)L.N, (int)s.E, (int)L.NB,
                     p.status, p.counts, p.offsets, p.blkhist, p.blkbad, p.lpt, p.src,
                     p.tstart, p.mtiles);
  return hipGetLastError();
}

hipError_t launch_plan_scatter(const moe_shape& s, const PlanLayout& L, const PlanPtrs& p,
                               const void* ids, hipStream_t st) {
  const int N = (int)L.N, E = (int)s.E, NB = (int)L.NB;
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  if (s.ids_dtype == MOE_IDS_I64)
    hipLaunchKernelGGL(moe_plan_scatter<int64_t>, dim3(NB), dim3(64), 0, st, (const int64_t*)ids,
                       N, E, NB, nbits, p.offsets, p.blkhist, p.pos, p.src);
  else
    hipLaunchKernelGGL(moe_plan_scatter<int32_t>, dim3(NB), dim3(64), 0, st, (const int32_t*)ids,
                       N, E, NB, nbits, p.offsets, p.blkhist, p.pos, p.src);
  return hipGetLastError();
}

#ifdef MOE_CHECKED
hipError_t oob_counter_plan(unsigned int** p) { return oob_counter_address(p); }
#endif

}  // namespace moe
