// C ABI of the routed-experts library: host-side checks, buffer layouts and the fixed launch
// sequence of each call. No call allocates, and only moe_plan_status waits for the stream.
#include <string.h>

#include <mutex>

#include "moe_internal.h"
#ifdef MOE_CHECKED
#include "moe_routed_checked.h"
#endif

using namespace moe;

#ifdef MOE_CHECKED
int64_t moe::g_checked_shrink = 0;
#endif

namespace {

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

moe_status check_shape(const moe_shape* s) {
  if (!s) return MOE_E_NULL;
  if (s->ids_dtype != MOE_IDS_I32 && s->ids_dtype != MOE_IDS_I64) return MOE_E_DTYPE;
  if (s->flags &
      ~(MOE_SAVE_FOR_BACKWARD | MOE_WGRAD_ACCUMULATE | MOE_WGRAD_F32 | MOE_RECOMPUTE | MOE_KEEP_XG))
    return MOE_E_DTYPE;
  if (s->T < 1 || s->K < 1 || s->K > MOE_MAX_TOPK) return MOE_E_SHAPE;
  if (s->E < 1 || s->E > MOE_MAX_EXPERTS) return MOE_E_SHAPE;
  if (s->D < 64 || s->F < 64 || (s->D % 64) != 0 || (s->F % 64) != 0) return MOE_E_SHAPE;
  // the GEMM copies take 32-bit byte offsets from a per-expert (weights) or per-tile (activation
  // rows) base: (2F - 1) rows of 2D bytes of w13[e] (4FD <= 2^32), and 255 rows of up to 4F or 2D
  // bytes of a 256-row tile (D, F <= 2^22)
  if (s->D > (1 << 22) || s->F > (1 << 22)) return MOE_E_SHAPE;
  if (4 * s->F * s->D > (int64_t(1) << 32)) return MOE_E_SHAPE;
  // slot and row indices are 32-bit in the kernels, and the plan's last 1024-slot chunk must end
  // below 2^31: at most 2^31 - 2^16 slots
  if (s->T > ((int64_t(1) << 31) - (int64_t(1) << 16)) / s->K) return MOE_E_SHAPE;
  if (gemm_max_grid(*s) > INT32_MAX) return MOE_E_SHAPE;
  return MOE_OK;
}

moe_status hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_E_HIP; }

struct Tracer {
  const moe_trace* tr;
  hipStream_t st;
  int next;
  hipError_t mark() {
    if (!tr || next >= tr->n_events || next >= MOE_TRACE_MAX_EVENTS) return hipSuccess;
    return hipEventRecord(tr->events[next++], st);
  }
};

#define MOE_TRY(expr)                             \
  do {                                            \
    hipError_t _e = (expr);                       \
    if (_e != hipSuccess) return MOE_E_HIP;       \
  } while (0)

// The forward's launch sequence after check_shape (moe_forward and moe_forward_noalloc)
moe_status forward_impl(const moe_shape* s, const void* plan, const uint16_t* x,
                        const float* scores, const uint16_t* w13, const uint16_t* w2,
                        uint16_t* out, void* saved, void* workspace, hipStream_t stream,
                        const moe_trace* trace) {
  const bool save = (s->flags & MOE_SAVE_FOR_BACKWARD) != 0;
  const bool re = save && (s->flags & MOE_RECOMPUTE) != 0;
  if (!plan || !x || !scores || !w13 || !w2 || !out) return MOE_E_NULL;
  if (save ? !saved : !workspace) return MOE_E_NULL;
  if (re && !workspace) return MOE_E_NULL;
  if (!aligned(plan, 16) || !aligned(x, 16) || !aligned(w13, 16) || !aligned(w2, 16) ||
      !aligned(out, 16) || !aligned(scores, 4) || (saved && !aligned(saved, 16)) ||
      (workspace && !aligned(workspace, 16)))
    return MOE_E_ALIGN;
  const PlanLayout L = plan_layout(*s);
  const PlanPtrs p = plan_ptrs(L, (void*)plan);
  const bool gx = gather_x(*s);
  uint16_t *xg = nullptr, *h13 = nullptr, *a, *y;
  if (save) {
    const SavedLayout S = saved_layout(*s);
    char* b = (char*)saved;
    if (!gx) xg = (uint16_t*)(b + S.xg);
    y = (uint16_t*)(b + S.y);
    if (re) {  // h13 is not kept; a lives in the workspace until W2 has read it
      a = (uint16_t*)((char*)workspace + work_layout(*s).a);
    } else {
      h13 = (uint16_t*)(b + S.h13);
      a = (uint16_t*)(b + S.a);
    }
  } else {
    const WorkLayout W = work_layout(*s);
    char* b = (char*)workspace;
    if (!gx) xg = (uint16_t*)(b + W.xg);
    a = (uint16_t*)(b + W.a);
    y = (uint16_t*)(b + W.y);
  }
  Tracer tr{trace, stream, 0};
  MOE_TRY(tr.mark());
  if (gx) {
    // no xg: the gate/up GEMM reads each routed row's token row of x (the permute stage is empty)
    MOE_TRY(tr.mark());
    MOE_TRY(launch_fprop_w13(*s, p, x, w13, h13, a, stream, true));
  } else {
    MOE_TRY(launch_permute(*s, p.pos, x, xg, stream));
    MOE_TRY(tr.mark());
    MOE_TRY(launch_fprop_w13(*s, p, xg, w13, h13, a, stream));
  }
  MOE_TRY(tr.mark());
  MOE_TRY(launch_fprop_w2(*s, p, a, w2, y, stream));
  MOE_TRY(tr.mark());
  MOE_TRY(launch_combine(*s, p.pos, y, scores, out, stream));
  MOE_TRY(tr.mark());
  return MOE_OK;
}

// ---- scratch of the allocation-free forward -------------------------------------------------
// moe_forward_noalloc keeps the forward's intermediates (xg when materialized, a, y) in this
// file-scope device array instead of a caller workspace: one copy per GPU, loaded with the code
// object and held until the process ends. Its name is a host-side stand-in in host code, never a
// device address: each device's address comes from hipGetSymbolAddress, taken once per device
// with that device current, and only that address reaches kernels.
static __device__ __align__(256) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_addr[kMaxDevices] = {};

// Address of the device's copy of scratch for work on `stream` (its device; the current device for
// the null stream).
moe_status scratch_address(hipStream_t stream, void** addr) {
  int dev = -1;
  if (stream) {
    if (hipStreamGetDevice(stream, &dev) != hipSuccess) return MOE_E_HIP;
  } else if (hipGetDevice(&dev) != hipSuccess) {
    return MOE_E_HIP;
  }
  if (dev < 0 || dev >= kMaxDevices) return MOE_E_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_addr[dev]) {
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) return MOE_E_HIP;
    if (cur != dev && hipSetDevice(dev) != hipSuccess) return MOE_E_HIP;
    void* a = nullptr;
    const hipError_t e = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));
    if (cur != dev && hipSetDevice(cur) != hipSuccess) return MOE_E_HIP;
    if (e != hipSuccess || !a) return MOE_E_HIP;
    g_scratch_addr[dev] = a;
  }
  *addr = g_scratch_addr[dev];
  return MOE_OK;
}

}  // namespace

extern "C" {

int moe_abi_version(void) { return MOE_ABI_VERSION; }

const char* moe_status_str(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_E_NULL: return "a required pointer is null";
    case MOE_E_SHAPE: return "shape outside the supported limits";
    case MOE_E_ALIGN: return "a pointer is not suitably aligned";
    case MOE_E_DTYPE: return "ids dtype or flags not recognised";
    case MOE_E_HIP: return "a HIP launch or runtime call failed";
    case MOE_E_BAD_IDS: return "routing held expert ids outside [0, E)";
    case MOE_E_STATE: return "backward needs a shape with MOE_SAVE_FOR_BACKWARD";
    case MOE_E_SCRATCH:
      return "the shape needs more scratch than the allocation-free forward holds";
    default: return "unknown status";
  }
}

size_t moe_plan_bytes(const moe_shape* s) {
  if (check_shape(s) != MOE_OK) return 0;
  return plan_layout(*s).total;
}

size_t moe_saved_bytes(const moe_shape* s) {
  if (check_shape(s) != MOE_OK) return 0;
  if (!(s->flags & MOE_SAVE_FOR_BACKWARD)) return 0;
  return saved_layout(*s).total;
}

size_t moe_workspace_bytes(const moe_shape* s) {
  if (check_shape(s) != MOE_OK) return 0;
  return work_layout(*s).total;
}

moe_status moe_plan(const moe_shape* s, const void* topk_ids, void* plan, hipStream_t stream,
                    const moe_trace* trace) {
  moe_status st = check_shape(s);
  if (st != MOE_OK) return st;
  if (!topk_ids || !plan) return MOE_E_NULL;
  if (!aligned(topk_ids, s->ids_dtype == MOE_IDS_I64 ? 8 : 4) || !aligned(plan, 16))
    return MOE_E_ALIGN;
  const PlanLayout L = plan_layout(*s);
  const PlanPtrs p = plan_ptrs(L, plan);
  Tracer tr{trace, stream, 0};
  MOE_TRY(tr.mark());
  MOE_TRY(launch_plan_hist(*s, L, p, topk_ids, stream));
  MOE_TRY(tr.mark());
  MOE_TRY(launch_plan_scan(*s, L, p, stream));
  MOE_TRY(tr.mark());
  MOE_TRY(launch_plan_scatter(*s, L, p, topk_ids, stream));
  MOE_TRY(tr.mark());
  return MOE_OK;
}

moe_status moe_forward(const moe_shape* s, const void* plan, const uint16_t* x,
                       const float* scores, const uint16_t* w13, const uint16_t* w2, uint16_t* out,
                       void* saved, void* workspace, hipStream_t stream, const moe_trace* trace) {
  moe_status st = check_shape(s);
  if (st != MOE_OK) return st;
  return forward_impl(s, plan, x, scores, w13, w2, out, saved, workspace, stream, trace);
}

moe_status moe_forward_noalloc(const moe_shape* s, const void* plan, const uint16_t* x,
                               const float* scores, const uint16_t* w13, const uint16_t* w2,
                               uint16_t* out, hipStream_t stream, const moe_trace* trace) {
  moe_status st = check_shape(s);
  if (st != MOE_OK) return st;
  if (s->flags & MOE_SAVE_FOR_BACKWARD) return MOE_E_STATE;
  if (!plan || !x || !scores || !w13 || !w2 || !out) return MOE_E_NULL;
  if (!aligned(plan, 16) || !aligned(x, 16) || !aligned(w13, 16) || !aligned(w2, 16) ||
      !aligned(out, 16) || !aligned(scores, 4))
    return MOE_E_ALIGN;
  if (work_layout(*s).fwd_total > (size_t)MOE_NOALLOC_SCRATCH_BYTES) return MOE_E_SCRATCH;
  void* ws = nullptr;
  st = scratch_address(stream, &ws);
  if (st != MOE_OK) return st;
  return forward_impl(s, plan, x, scores, w13, w2, out, nullptr, ws, stream, trace);
}

moe_status moe_backward(const moe_shape* s, const void* plan, const void* saved,
                        const uint16_t* x, const uint16_t* dout, const float* scores,
                        const uint16_t* w13,
                        const uint16_t* w2, uint16_t* dx, void* dw13, void* dw2,
                        float* dscores, void* workspace, hipStream_t stream,
                        const moe_trace* trace) {
  moe_status st = check_shape(s);
  if (st != MOE_OK) return st;
  if (!(s->flags & MOE_SAVE_FOR_BACKWARD)) return MOE_E_STATE;
  const bool gx = gather_x(*s);  // the GEMMs that read xg read x's token rows (xg is not saved)
  if (!plan || !saved || (gx && !x) || !dout || !scores || !w13 || !w2 || !dx || !dw13 || !dw2 ||
      !dscores || !workspace)
    return MOE_E_NULL;
  if (!aligned(plan, 16) || !aligned(saved, 16) || (x && !aligned(x, 16)) || !aligned(dout, 16) ||
      !aligned(w13, 16) || !aligned(w2, 16) || !aligned(dx, 16) || !aligned(dw13, 16) ||
      !aligned(dw2, 16) || !aligned(workspace, 16) || !aligned(scores, 4) ||
      !aligned(dscores, 4))
    return MOE_E_ALIGN;
  const PlanLayout L = plan_layout(*s);
  const PlanPtrs p = plan_ptrs(L, (void*)plan);
  const bool re = (s->flags & MOE_RECOMPUTE) != 0;
  const SavedLayout S = saved_layout(*s);
  const char* sb = (const char*)saved;
  const WorkLayout W = work_layout(*s);
  char* wb = (char*)workspace;
  const uint16_t* y = (const uint16_t*)(sb + S.y);
  uint16_t* dy = (uint16_t*)(wb + W.dy);
  uint16_t* dh13 = (uint16_t*)(wb + W.dh13);
  // dy is dead once the W2 weight gradient has been formed: its region then holds xg for the W13
  // weight gradient (gather_x: permuted there from x; otherwise xg is the saved one) and, after
  // that GEMM, dxg
  uint16_t* dxg = dy;
  const uint16_t* xg = gx ? dy : (const uint16_t*)(sb + S.xg);
  // recompute: h13 is rebuilt where dh13 goes (read and overwritten element by element by the
  // SwiGLU-derivative GEMM), a in its own workspace region
  const uint16_t* h13 = re ? dh13 : (const uint16_t*)(sb + S.h13);
  const uint16_t* a = re ? (const uint16_t*)(wb + W.a_re) : (const uint16_t*)(sb + S.a);
  Tracer tr{trace, stream, 0};
  MOE_TRY(tr.mark());
  MOE_TRY(launch_combine_bwd(*s, p.pos, dout, y, scores, dy, dscores, stream));
  MOE_TRY(tr.mark());
  if (re) {
    MOE_TRY(launch_fprop_w13(*s, p, gx ? x : xg, w13, dh13, (uint16_t*)(wb + W.a_re), stream,
                             gx));
    MOE_TRY(tr.mark());
  }
  MOE_TRY(launch_w2_backward(*s, p, dy, w2, h13, dh13, a, dw2, stream));
  MOE_TRY(tr.mark());
  if (gx) MOE_TRY(launch_permute(*s, p.pos, x, dy, stream));  // the stage is empty otherwise
  MOE_TRY(tr.mark());
  MOE_TRY(launch_wgrad_w13(*s, p, dh13, xg, dw13, stream));
  MOE_TRY(tr.mark());
  MOE_TRY(launch_dgrad_w13(*s, p, dh13, w13, dxg, stream));
  MOE_TRY(tr.mark());
  MOE_TRY(launch_combine(*s, p.pos, dxg, nullptr, dx, stream));
  MOE_TRY(tr.mark());
  return MOE_OK;
}

moe_status moe_permute(const moe_shape* s, const void* plan, const uint16_t* x, uint16_t* xg,
                       hipStream_t stream) {
  moe_status st = check_shape(s);
  if (st != MOE_OK) return st;
  if (!plan || !x || !xg) return MOE_E_NULL;
  if (!aligned(plan, 16) || !aligned(x, 16) || !aligned(xg, 16)) return MOE_E_ALIGN;
  const PlanPtrs p = plan_ptrs(plan_layout(*s), (void*)plan);
  MOE_TRY(launch_permute(*s, p.pos, x, xg, stream));
  return MOE_OK;
}

moe_status moe_combine(const moe_shape* s, const void* plan, const uint16_t* rows,
                       const float* scores, uint16_t* out, hipStream_t stream) {
  moe_status st = check_shape(s);
  if (st != MOE_OK) return st;
  if (!plan || !rows || !out) return MOE_E_NULL;
  if (!aligned(plan, 16) || !aligned(rows, 16) || !aligned(out, 16) ||
      (scores && !aligned(scores, 4)))
    return MOE_E_ALIGN;
  const PlanPtrs p = plan_ptrs(plan_layout(*s), (void*)plan);
  MOE_TRY(launch_combine(*s, p.pos, rows, scores, out, stream));
  return MOE_OK;
}

moe_status moe_combine_backward(const moe_shape* s, const void* plan, const uint16_t* dout,
                                const uint16_t* y, const float* scores, uint16_t* dy,
                                float* dscores, hipStream_t stream) {
  moe_status st = check_shape(s);
  if (st != MOE_OK) return st;
  if (!plan || !dout || !y || !scores || !dy || !dscores) return MOE_E_NULL;
  if (!aligned(plan, 16) || !aligned(dout, 16) || !aligned(y, 16) || !aligned(dy, 16) ||
      !aligned(scores, 4) || !aligned(dscores, 4))
    return MOE_E_ALIGN;
  const PlanPtrs p = plan_ptrs(plan_layout(*s), (void*)plan);
  MOE_TRY(launch_combine_bwd(*s, p.pos, dout, y, scores, dy, dscores, stream));
  return MOE_OK;
}

moe_status moe_route(const moe_shape* s, const moe_router* r, const float* logits,
                     void* topk_ids, float* scores, hipStream_t stream, const moe_trace* trace) {
  if (!s || !r) return MOE_E_NULL;
  if (s->ids_dtype != MOE_IDS_I32 && s->ids_dtype != MOE_IDS_I64) return MOE_E_DTYPE;
  if (r->score_fn != MOE_SCORE_SOFTMAX && r->score_fn != MOE_SCORE_SIGMOID) return MOE_E_DTYPE;
  if (s->T < 1 || s->E < 1 || s->E > MOE_MAX_EXPERTS || s->K < 1 || s->K > MOE_MAX_TOPK ||
      s->K > s->E || s->T > (int64_t)(INT32_MAX - 1) / s->K)
    return MOE_E_SHAPE;
  if (r->n_group > 1) {
    if (r->n_group > MOE_MAX_GROUPS || s->E % r->n_group != 0 || r->topk_group < 1 ||
        r->topk_group > r->n_group || s->K > (int64_t)r->topk_group * (s->E / r->n_group))
      return MOE_E_SHAPE;
  }
  if (!logits || !topk_ids || !scores) return MOE_E_NULL;
  if (!aligned(logits, 4) || !aligned(scores, 4) ||
      !aligned(topk_ids, s->ids_dtype == MOE_IDS_I64 ? 8 : 4))
    return MOE_E_ALIGN;
  Tracer tr{trace, stream, 0};
  MOE_TRY(tr.mark());
  MOE_TRY(launch_route(*s, *r, logits, topk_ids, scores, stream));
  MOE_TRY(tr.mark());
  return MOE_OK;
}

moe_status moe_plan_export(const moe_shape* s, const void* plan, int32_t* counts,
                           int32_t* offsets, int32_t* pos, int32_t* src, hipStream_t stream) {
  moe_status st = check_shape(s);
  if (st != MOE_OK) return st;
  if (!plan) return MOE_E_NULL;
  if (!aligned(plan, 16)) return MOE_E_ALIGN;
  const PlanLayout L = plan_layout(*s);
  const PlanPtrs p = plan_ptrs(L, (void*)plan);
  const size_t N = (size_t)L.N, E = (size_t)L.E;
  if (counts)
    MOE_TRY(hipMemcpyAsync(counts, p.counts, 4 * E, hipMemcpyDeviceToDevice, stream));
  if (offsets)
    MOE_TRY(hipMemcpyAsync(offsets, p.offsets, 4 * (E + 1), hipMemcpyDeviceToDevice, stream));
  if (pos) MOE_TRY(hipMemcpyAsync(pos, p.pos, 4 * N, hipMemcpyDeviceToDevice, stream));
  if (src) MOE_TRY(hipMemcpyAsync(src, p.src, 4 * N, hipMemcpyDeviceToDevice, stream));
  return MOE_OK;
}

moe_status moe_plan_status(const moe_shape* s, const void* plan, int64_t* bad_ids,
                           hipStream_t stream) {
  moe_status st = check_shape(s);
  if (st != MOE_OK) return st;
  if (!plan) return MOE_E_NULL;
  if (!aligned(plan, 16)) return MOE_E_ALIGN;
  const PlanLayout L = plan_layout(*s);
  const PlanPtrs p = plan_ptrs(L, (void*)plan);
  int32_t host = 0;
  MOE_TRY(hipMemcpyAsync(&host, p.status, sizeof host, hipMemcpyDeviceToHost, stream));
  MOE_TRY(hipStreamSynchronize(stream));
  if (bad_ids) *bad_ids = host;
  return host != 0 ? MOE_E_BAD_IDS : MOE_OK;
}

moe_status moe_saved_views(const moe_shape* s, void* saved, uint16_t** xg, uint16_t** h13,
                           uint16_t** a, uint16_t** y) {
  moe_status st = check_shape(s);
  if (st != MOE_OK) return st;
  if (!(s->flags & MOE_SAVE_FOR_BACKWARD)) return MOE_E_STATE;
  if (!saved) return MOE_E_NULL;
  const SavedLayout S = saved_layout(*s);
  char* b = (char*)saved;
  const bool re = (s->flags & MOE_RECOMPUTE) != 0;
  if (xg) *xg = gather_x(*s) ? nullptr : (uint16_t*)(b + S.xg);
  if (h13) *h13 = re ? nullptr : (uint16_t*)(b + S.h13);
  if (a) *a = re ? nullptr : (uint16_t*)(b + S.a);
  if (y) *y = (uint16_t*)(b + S.y);
  return MOE_OK;
}

#ifdef MOE_CHECKED
// Checked build only (declared in moe_routed_checked.h).
moe_status moe_checked_violations(uint64_t* count) {
  if (!count) return MOE_E_NULL;
  hipError_t (*const counters[])(unsigned int**) = {oob_counter_plan, oob_counter_rowops,
                                                    oob_counter_gemm};
  MOE_TRY(hipDeviceSynchronize());
  uint64_t total = 0;
  for (auto f : counters) {
    unsigned int* d = nullptr;
    unsigned int h = 0;
    MOE_TRY(f(&d));
    MOE_TRY(hipMemcpy(&h, d, sizeof h, hipMemcpyDeviceToHost));
    total += h;
  }
  *count = total;
  return MOE_OK;
}

moe_status moe_checked_reset(void) {
  hipError_t (*const counters[])(unsigned int**) = {oob_counter_plan, oob_counter_rowops,
                                                    oob_counter_gemm};
  MOE_TRY(hipDeviceSynchronize());
  for (auto f : counters) {
    unsigned int* d = nullptr;
    const unsigned int zero = 0;
    MOE_TRY(f(&d));
    MOE_TRY(hipMemcpy(d, &zero, sizeof zero, hipMemcpyHostToDevice));
  }
  return MOE_OK;
}

moe_status moe_checked_shrink(int64_t bytes) {
  if (bytes < 0) return MOE_E_SHAPE;
  g_checked_shrink = bytes;
  return MOE_OK;
}
#endif

}  // extern "C"
