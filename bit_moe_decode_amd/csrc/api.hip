// api.hip -- host side of the C ABI declared in include/moe_decode.h:
// argument validation, workspace layout and kernel launches.  All checks are
// host-only and run before anything is enqueued.
#include "moe_decode.h"

#include <mutex>
#include <new>

#include "device_common.h"

namespace moe {
hipError_t launch_router(const uint16_t* x, const Weights& w, const Ws& ws, const Dims& d,
                         hipStream_t stream);
hipError_t launch_route(int rfmt, const Weights& w, const Ws& ws, const Dims& d,
                        hipStream_t stream);
bool fused_route(const Dims& d);
hipError_t launch_upgate(int rfmt, int max_groups, const Weights& w, const Ws& ws,
                         const Dims& d, hipStream_t stream);
hipError_t launch_down(int rfmt, int max_groups, const Weights& w, const Ws& ws, const Dims& d,
                       hipStream_t stream);
hipError_t launch_combine(const Ws& ws, const Dims& d, uint16_t* out, hipStream_t stream);
int upgate_k_parts(int hidden, int routed_fmt);
hipError_t launch_lowbit_q1(const uint8_t* blocks, const uint16_t* x, uint16_t* y, int rows,
                            int n, int k, hipStream_t stream);
hipError_t launch_gemv_fp8(const uint8_t* codes, const float* scales, const uint16_t* x,
                           uint16_t* y, int rows, int n, int k, hipStream_t stream);
hipError_t launch_gemv_bf16(const uint16_t* w, const uint16_t* x, uint16_t* y, int rows, int n,
                            int k, hipStream_t stream);

__global__ void moe_fill_u32_kernel(uint32_t* p, size_t n, uint32_t v) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = v;
}
}  // namespace moe

using namespace moe;

// Device scratch of moe_decode_step_noalloc: the workspace of a step that
// brings none.  One copy per GPU the library runs on, held until the process
// ends.  In host code `scratch` names a host-side stand-in, not the device
// array: the device address comes from hipGetSymbolAddress, once per device
// (scratch_on_device below), and only that address is handed to kernels.
constexpr size_t kScratchBytes = MOE_DECODE_NOALLOC_MAX_WORKSPACE;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {

constexpr uint32_t kKnownFlags = MOE_F_NO_DEDUP;

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

struct Plan {
  int H, I, E, Is, R, imax, groups, ks;
  size_t off_logits, off_rstd, off_ids, off_gates, off_ngroups, off_gexpert,
      off_gowner, off_gmask, off_gslot, off_grows, off_gnrows, off_actq, off_actqp, off_acts, off_mid,
      off_midq, off_midqs, off_ypart, off_actu, off_blkrec, off_waitto, total;
};

bool is_mult(int v, int m) { return v > 0 && v % m == 0; }

moe_status plan_config(const moe_decode_config* c, Plan* p) {
  if (!c) return MOE_ERR_INVALID_ARG;
  if (c->top_k != 8) return MOE_ERR_UNSUPPORTED;
  if (!is_mult(c->hidden, 128) || c->hidden > 16384) return MOE_ERR_UNSUPPORTED;
  if (!is_mult(c->inter, 128) || c->inter > 16384) return MOE_ERR_UNSUPPORTED;
  // the shared expert, when present, has the routed experts' intermediate size
  if (c->shared_inter != 0 && c->shared_inter != c->inter) return MOE_ERR_UNSUPPORTED;
  if (!is_mult(c->n_experts, 16) || c->n_experts > 1024) return MOE_ERR_UNSUPPORTED;
  if (c->max_rows < 1 || c->max_rows > 8) return MOE_ERR_INVALID_ARG;
  if (c->routed_fmt != MOE_FMT_FP8_E4M3_B128 && c->routed_fmt != MOE_FMT_MXFP4 &&
      c->routed_fmt != MOE_FMT_Q1_G128)
    return MOE_ERR_UNSUPPORTED;
  // 1-bit routed experts: up/gate items of 4 groups (hidden % 512), down rows
  // of whole 36-byte chunks loaded at once (inter % 256, at most 4096), FP8
  // activations (their MFMA is FP8 x FP8)
  if (c->routed_fmt == MOE_FMT_Q1_G128 &&
      (c->hidden % 512 || c->inter % 256 || c->inter > 4096 || c->act_fmt != MOE_ACT_FP8_B128))
    return MOE_ERR_UNSUPPORTED;
  // MXFP4 up/gate items are two K blocks wide; the down GEMV keeps its
  // columns' mid split into bf16 hi + lo in LDS (4 bytes an element, up to 8
  // columns): I <= 4096
  if (c->routed_fmt == MOE_FMT_MXFP4 && (c->hidden % 256 || c->inter > 4096))
    return MOE_ERR_UNSUPPORTED;
  if (c->shared_inter > 0 && c->shared_fmt != MOE_FMT_FP8_E4M3_B128) return MOE_ERR_UNSUPPORTED;
  if (c->flags & ~kKnownFlags) return MOE_ERR_UNSUPPORTED;
  if (c->act_fmt != MOE_ACT_FP8_B128 && c->act_fmt != MOE_ACT_BF16) return MOE_ERR_UNSUPPORTED;
  // bf16 activations: the up/gate's bf16 MFMA takes FP8 weights only
  if (c->act_fmt == MOE_ACT_BF16 && c->routed_fmt != MOE_FMT_FP8_E4M3_B128)
    return MOE_ERR_UNSUPPORTED;
  if (!(c->rms_eps >= 0.0f) || c->rms_eps > 1.0f) return MOE_ERR_INVALID_ARG;

  p->H = c->hidden;
  p->I = c->inter;
  p->E = c->n_experts;
  p->Is = c->shared_inter;
  p->R = c->max_rows;
  p->imax = p->I > p->Is ? p->I : p->Is;
  const int picks = 8 * p->R;
  p->groups = (c->flags & MOE_F_NO_DEDUP) ? picks : (picks < p->E ? picks : p->E);
  p->ks = upgate_k_parts(p->H, c->routed_fmt);

  size_t o = 0;
  auto take = [&](size_t bytes) {
    size_t at = o;
    o = align_up(o + bytes, 256);
    return at;
  };
  const size_t R = p->R, E = p->E, H = p->H, G = p->groups, IM = p->imax;
  p->off_logits = take(R * E * 4);
  p->off_rstd = take(R * 4);
  p->off_ids = take(R * 8 * 4);
  p->off_gates = take(R * 8 * 4);
  p->off_ngroups = take(4);
  p->off_gexpert = take(G * 4);
  p->off_gowner = take(G * 2);
  p->off_gmask = take(G);
  p->off_gslot = take(G * 8);
  p->off_grows = take(G * 8);
  p->off_gnrows = take(G);
  p->off_actq = take(R * H);
  p->off_actqp = take(c->routed_fmt == MOE_FMT_Q1_G128 ? R * H : 0);  // 1-bit operand order
  p->off_acts = take(R * (H / 128) * 4);
  const size_t U = R * 9;  // (row, pick) pairs, pick 8 = the shared expert
  p->off_mid = take(U * IM * 4);
  p->off_midq = take(U * IM);
  p->off_midqs = take(U * (IM / 128) * 4);
  p->off_ypart = take(U * H * 4);
  p->off_actu = take(R * H * 2);
  // one record per up/gate block of the routing launch: at most Is/16 + G*I/16
  p->off_blkrec = take((p->Is / 16 + G * (p->I / 16)) * 8);
  p->off_waitto = take(4);
  p->total = o;
  return MOE_OK;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// The kernels' view of a workspace laid out by `p` from base address `b`.
Ws make_view(char* b, const Plan& p) {
  Ws v;
  v.logits = reinterpret_cast<float*>(b + p.off_logits);
  v.rstd = reinterpret_cast<float*>(b + p.off_rstd);
  v.ids = reinterpret_cast<int32_t*>(b + p.off_ids);
  v.gates = reinterpret_cast<float*>(b + p.off_gates);
  v.n_groups = reinterpret_cast<int32_t*>(b + p.off_ngroups);
  v.grp_expert = reinterpret_cast<int32_t*>(b + p.off_gexpert);
  v.grp_owner = reinterpret_cast<uint8_t*>(b + p.off_gowner);
  v.grp_mask = reinterpret_cast<uint8_t*>(b + p.off_gmask);
  v.grp_slot = reinterpret_cast<uint8_t*>(b + p.off_gslot);
  v.grp_rows = reinterpret_cast<uint8_t*>(b + p.off_grows);
  v.grp_nrows = reinterpret_cast<uint8_t*>(b + p.off_gnrows);
  v.act_q = reinterpret_cast<uint8_t*>(b + p.off_actq);
  v.act_qp = reinterpret_cast<uint8_t*>(b + p.off_actqp);
  v.act_s = reinterpret_cast<float*>(b + p.off_acts);
  v.mid = reinterpret_cast<float*>(b + p.off_mid);
  v.midq = reinterpret_cast<uint8_t*>(b + p.off_midq);
  v.midqs = reinterpret_cast<float*>(b + p.off_midqs);
  v.ypart = reinterpret_cast<float*>(b + p.off_ypart);
  v.act_u = reinterpret_cast<uint16_t*>(b + p.off_actu);
  v.blk_rec = reinterpret_cast<uint64_t*>(b + p.off_blkrec);
  v.wait_timeouts = reinterpret_cast<uint32_t*>(b + p.off_waitto);
  return v;
}

}  // namespace

struct moe_decode_ctx {
  moe_decode_config cfg;
  Plan plan;
  char* ws;
  Ws view;
  hipEvent_t events[MOE_DECODE_N_KERNELS + 1];
  bool timing;
  int last_rows;  // rows of the last step enqueued, 0 before the first
  uint32_t wait_ticks;  // cap of the routing launch's waits
  int withhold;         // 1: the routing block publishes no records
};

// Default cap of a routed up/gate block's wait for its record: 10 ms of the
// 100 MHz real-time counter, far beyond the routing's few microseconds.
constexpr uint32_t kDefaultWaitTicks = 1000000u;

extern "C" {

size_t moe_decode_workspace_size(const moe_decode_config* cfg) {
  Plan p;
  if (plan_config(cfg, &p) != MOE_OK) return 0;
  return p.total;
}

moe_status moe_decode_init(const moe_decode_config* cfg, void* workspace, size_t ws_bytes,
                           hipStream_t stream, moe_decode_ctx** out) {
  if (!out) return MOE_ERR_INVALID_ARG;
  *out = nullptr;
  Plan p;
  moe_status st = plan_config(cfg, &p);
  if (st != MOE_OK) return st;
  if (!workspace || ((uintptr_t)workspace & 255u)) return MOE_ERR_WORKSPACE;
  if (ws_bytes < p.total) return MOE_ERR_WORKSPACE;
  moe_decode_ctx* c = new (std::nothrow) moe_decode_ctx();
  if (!c) return MOE_ERR_DEVICE;
  c->cfg = *cfg;
  c->plan = p;
  c->ws = static_cast<char*>(workspace);
  c->timing = false;
  c->last_rows = 0;
  c->wait_ticks = kDefaultWaitTicks;
  c->withhold = 0;
  c->view = make_view(c->ws, p);
  // clear the whole workspace once, so that debug views read before the
  // first step are well defined
  const size_t words = p.total / 4;
  hipLaunchKernelGGL(moe_fill_u32_kernel, dim3(256), dim3(256), 0, stream,
                     reinterpret_cast<uint32_t*>(c->ws), words, 0u);
  if (hipGetLastError() != hipSuccess) {
    delete c;
    return MOE_ERR_DEVICE;
  }
  *out = c;
  return MOE_OK;
}

namespace {
// Validates the weights and fills the kernels' argument views for a step of
// `rows` rows of a layer with config `cfg` and plan `p`.
moe_status step_args(const moe_decode_config& cfg, const Plan& p, int rows,
                     const moe_decode_weights* w, Weights* wtp, Dims* dp) {
  if (!w) return MOE_ERR_INVALID_ARG;
  const void* need[] = {w->rms_gamma, w->router_w, w->gate.codes, w->up.codes, w->down.codes};
  for (const void* q : need)
    if (!q || !aligned16(q)) return MOE_ERR_INVALID_ARG;
  if (cfg.routed_fmt != MOE_FMT_Q1_G128) {  // 1-bit blocks hold their own scales
    const void* sc[] = {w->gate.scales, w->up.scales, w->down.scales};
    for (const void* q : sc)
      if (!q || !aligned16(q)) return MOE_ERR_INVALID_ARG;
  }
  if (p.Is > 0) {
    const void* sh[] = {w->sh_gate.codes, w->sh_gate.scales, w->sh_up.codes,
                        w->sh_up.scales, w->sh_down.codes, w->sh_down.scales};
    for (const void* q : sh)
      if (!q || !aligned16(q)) return MOE_ERR_INVALID_ARG;
  }
  Weights& wt = *wtp;
  wt.gamma = w->rms_gamma;
  wt.router = w->router_w;
  wt.gate_c = static_cast<const uint8_t*>(w->gate.codes);
  wt.up_c = static_cast<const uint8_t*>(w->up.codes);
  wt.down_c = static_cast<const uint8_t*>(w->down.codes);
  wt.gate_s = w->gate.scales;
  wt.up_s = w->up.scales;
  wt.down_s = w->down.scales;
  wt.sg_c = static_cast<const uint8_t*>(w->sh_gate.codes);
  wt.su_c = static_cast<const uint8_t*>(w->sh_up.codes);
  wt.sd_c = static_cast<const uint8_t*>(w->sh_down.codes);
  wt.sg_s = static_cast<const float*>(w->sh_gate.scales);
  wt.su_s = static_cast<const float*>(w->sh_up.scales);
  wt.sd_s = static_cast<const float*>(w->sh_down.scales);

  Dims& d = *dp;
  d.H = p.H;
  d.I = p.I;
  d.E = p.E;
  d.Is = p.Is;
  d.rows = rows;
  d.max_rows = p.R;
  d.imax = p.imax;
  d.ks = p.ks;
  d.no_dedup = (cfg.flags & MOE_F_NO_DEDUP) ? 1 : 0;
  d.eps = cfg.rms_eps;
  d.act_bf16 = cfg.act_fmt == MOE_ACT_BF16 ? 1 : 0;
  d.act_q1 = cfg.routed_fmt == MOE_FMT_Q1_G128 ? 1 : 0;
  const int picks = 8 * rows;
  d.groups = d.no_dedup ? picks : (picks < p.E ? picks : p.E);
  d.wait_ticks = kDefaultWaitTicks;
  d.withhold = 0;
  return MOE_OK;
}

// Groups a step of `rows` rows can produce: at most 8 * rows (and E with dedup).

// Host checks of a step's x and out (rows >= 1).
moe_status check_io(const Plan& p, const uint16_t* x, int rows, const moe_decode_weights* w,
                    const uint16_t* out) {
  if (!x || !w || !out || !aligned16(x) || !aligned16(out)) return MOE_ERR_INVALID_ARG;
  const size_t bytes = (size_t)rows * p.H * 2;
  const uintptr_t xa = (uintptr_t)x, oa = (uintptr_t)out;
  if (xa < oa + bytes && oa < xa + bytes) return MOE_ERR_INVALID_ARG;
  return MOE_OK;
}

// The device address of `scratch` on the current device, looked up once per
// device under a lock and kept.
moe_status scratch_on_device(char** out) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static char* addr[kMaxDevices] = {};
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MOE_ERR_DEVICE;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MOE_ERR_DEVICE;
    addr[dev] = static_cast<char*>(p);
  }
  *out = addr[dev];
  return MOE_OK;
}

// The step's five launches on `stream` over workspace view `v`; with `ev`,
// an event before the first and after each.
moe_status enqueue_step(int routed_fmt, const Plan& p, const Ws& v, const uint16_t* x,
                        const Weights& wt, const Dims& d, uint16_t* out, hipStream_t stream,
                        hipEvent_t* ev) {
  if (ev && hipEventRecord(ev[0], stream) != hipSuccess) return MOE_ERR_DEVICE;
  if (launch_router(x, wt, v, d, stream) != hipSuccess) return MOE_ERR_DEVICE;
  if (ev && hipEventRecord(ev[1], stream) != hipSuccess) return MOE_ERR_DEVICE;
  // routing, with the up/gate of the shared and the routed experts alongside
  // (or the routing alone, then the up/gate)
  if (launch_route(routed_fmt, wt, v, d, stream) != hipSuccess) return MOE_ERR_DEVICE;
  if (ev && hipEventRecord(ev[2], stream) != hipSuccess) return MOE_ERR_DEVICE;
  if (!fused_route(d) && launch_upgate(routed_fmt, d.groups, wt, v, d, stream) != hipSuccess)
    return MOE_ERR_DEVICE;
  if (ev && hipEventRecord(ev[3], stream) != hipSuccess) return MOE_ERR_DEVICE;
  if (launch_down(routed_fmt, d.groups, wt, v, d, stream) != hipSuccess) return MOE_ERR_DEVICE;
  if (ev && hipEventRecord(ev[4], stream) != hipSuccess) return MOE_ERR_DEVICE;
  if (launch_combine(v, d, out, stream) != hipSuccess) return MOE_ERR_DEVICE;
  if (ev && hipEventRecord(ev[5], stream) != hipSuccess) return MOE_ERR_DEVICE;
  return MOE_OK;
}
}  // namespace

moe_status moe_decode_step(moe_decode_ctx* ctx, const uint16_t* x, int32_t rows,
                           const moe_decode_weights* w, uint16_t* out, hipStream_t stream) {
  if (!ctx) return MOE_ERR_INVALID_ARG;
  const Plan& p = ctx->plan;
  if (rows < 0 || rows > p.R) return MOE_ERR_INVALID_ARG;
  if (rows == 0) return MOE_OK;
  moe_status st = check_io(p, x, rows, w, out);
  if (st != MOE_OK) return st;
  Weights wt;
  Dims d;
  st = step_args(ctx->cfg, p, rows, w, &wt, &d);
  if (st != MOE_OK) return st;
  d.wait_ticks = ctx->wait_ticks;
  d.withhold = ctx->withhold;
  ctx->last_rows = rows;
  return enqueue_step(ctx->cfg.routed_fmt, p, ctx->view, x, wt, d, out, stream,
                      ctx->timing ? ctx->events : nullptr);
}

moe_status moe_decode_step_noalloc(const moe_decode_config* cfg, const uint16_t* x,
                                   int32_t rows, const moe_decode_weights* w, uint16_t* out,
                                   hipStream_t stream) {
  Plan p;
  moe_status st = plan_config(cfg, &p);
  if (st != MOE_OK) return st;
  if (p.total > kScratchBytes) return MOE_ERR_WORKSPACE;
  if (rows < 0 || rows > p.R) return MOE_ERR_INVALID_ARG;
  if (rows == 0) return MOE_OK;
  st = check_io(p, x, rows, w, out);
  if (st != MOE_OK) return st;
  Weights wt;
  Dims d;
  st = step_args(*cfg, p, rows, w, &wt, &d);
  if (st != MOE_OK) return st;
  char* base = nullptr;
  st = scratch_on_device(&base);
  if (st != MOE_OK) return st;
  return enqueue_step(cfg->routed_fmt, p, make_view(base, p), x, wt, d, out, stream, nullptr);
}

moe_status moe_decode_debug_view(const moe_decode_ctx* ctx, moe_decode_debug* v) {
  if (!ctx || !v) return MOE_ERR_INVALID_ARG;
  const Ws& w = ctx->view;
  v->logits = w.logits;
  v->rstd = w.rstd;
  v->ids = w.ids;
  v->gates = w.gates;
  v->n_groups = w.n_groups;
  v->grp_expert = w.grp_expert;
  v->grp_owner = w.grp_owner;
  v->grp_mask = w.grp_mask;
  v->grp_slot = w.grp_slot;
  v->act_q = w.act_q;
  v->act_s = w.act_s;
  v->mid = w.mid;
  v->midq = w.midq;
  v->midqs = w.midqs;
  v->y = w.ypart;
  v->max_groups = ctx->plan.groups;
  v->mid_stride = ctx->plan.imax;
  return MOE_OK;
}

moe_status moe_decode_set_timing(moe_decode_ctx* ctx, hipEvent_t* events) {
  if (!ctx) return MOE_ERR_INVALID_ARG;
  if (!events) {
    ctx->timing = false;
    return MOE_OK;
  }
  for (int i = 0; i <= MOE_DECODE_N_KERNELS; i++) {
    if (!events[i]) return MOE_ERR_INVALID_ARG;
    ctx->events[i] = events[i];
  }
  ctx->timing = true;
  return MOE_OK;
}

moe_status moe_decode_relaunch(moe_decode_ctx* ctx, int32_t kernel,
                               const moe_decode_weights* w, int32_t reps, hipStream_t stream) {
  if (!ctx || reps < 0) return MOE_ERR_INVALID_ARG;
  if (kernel != MOE_DECODE_K_UPGATE && kernel != MOE_DECODE_K_DOWN) return MOE_ERR_INVALID_ARG;
  if (ctx->last_rows == 0) return MOE_ERR_INVALID_ARG;
  Weights wt;
  Dims d;
  const moe_status st = step_args(ctx->cfg, ctx->plan, ctx->last_rows, w, &wt, &d);
  if (st != MOE_OK) return st;
  d.wait_ticks = ctx->wait_ticks;
  const int rf = ctx->cfg.routed_fmt;
  for (int i = 0; i < reps; i++) {
    hipError_t e;
    if (kernel == MOE_DECODE_K_DOWN)
      e = launch_down(rf, d.groups, wt, ctx->view, d, stream);
    else if (fused_route(d))  // the up/gate runs in the routing launch: relaunch that
      e = launch_route(rf, wt, ctx->view, d, stream);
    else
      e = launch_upgate(rf, d.groups, wt, ctx->view, d, stream);
    if (e != hipSuccess) return MOE_ERR_DEVICE;
  }
  return MOE_OK;
}

moe_status moe_decode_set_wait(moe_decode_ctx* ctx, uint32_t cap_ticks, int32_t withhold) {
  if (!ctx || (withhold != 0 && withhold != 1)) return MOE_ERR_INVALID_ARG;
  ctx->wait_ticks = cap_ticks ? cap_ticks : kDefaultWaitTicks;
  ctx->withhold = withhold;
  return MOE_OK;
}

moe_status moe_decode_wait_timeouts(moe_decode_ctx* ctx, uint32_t* count, hipStream_t stream) {
  if (!ctx || !count) return MOE_ERR_INVALID_ARG;
  if (hipMemcpyAsync(count, ctx->view.wait_timeouts, sizeof(uint32_t), hipMemcpyDeviceToHost,
                     stream) != hipSuccess)
    return MOE_ERR_DEVICE;
  return hipStreamSynchronize(stream) == hipSuccess ? MOE_OK : MOE_ERR_DEVICE;
}

void moe_decode_destroy(moe_decode_ctx* ctx) { delete ctx; }

const char* moe_status_string(moe_status s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported shape or format";
    case MOE_ERR_WORKSPACE: return "workspace missing or too small";
    case MOE_ERR_DEVICE: return "HIP launch error";
  }
  return "unknown status";
}

moe_status lowbit_gemv(const lowbit_matrix* w, const uint16_t* x, int32_t rows, uint16_t* y,
                       hipStream_t stream) {
  if (!w) return MOE_ERR_INVALID_ARG;
  if (w->fmt == MOE_FMT_FP8_E4M3_B128) {
    // FP8 weights in 128x128 blocks, 1 to 8 bf16 input rows
    if (w->n < 0 || w->k <= 0) return MOE_ERR_INVALID_ARG;
    if (w->n % 128 || w->k % 128) return MOE_ERR_UNSUPPORTED;
    if (rows < 0) return MOE_ERR_INVALID_ARG;
    if (rows == 0 || w->n == 0) return MOE_OK;
    if (rows > 8) return MOE_ERR_UNSUPPORTED;
    if (!w->codes || !w->scales || !x || !y || !aligned16(w->codes) || !aligned16(x) ||
        ((uintptr_t)w->scales & 3u) || ((uintptr_t)y & 1u))
      return MOE_ERR_INVALID_ARG;
    const uintptr_t xa = (uintptr_t)x, ya = (uintptr_t)y;
    if (xa < ya + (size_t)rows * w->n * 2 && ya < xa + (size_t)rows * w->k * 2)
      return MOE_ERR_INVALID_ARG;
    if (launch_gemv_fp8(static_cast<const uint8_t*>(w->codes), static_cast<const float*>(w->scales),
                        x, y, rows, w->n, w->k, stream) != hipSuccess)
      return MOE_ERR_DEVICE;
    return MOE_OK;
  }
  if (w->fmt == MOE_FMT_BF16) {
    // bf16 weights, 1 to 8 bf16 input rows
    if (w->n < 0 || w->k <= 0) return MOE_ERR_INVALID_ARG;
    if (w->n % 128 || w->k % 64) return MOE_ERR_UNSUPPORTED;
    if (rows < 0) return MOE_ERR_INVALID_ARG;
    if (rows == 0 || w->n == 0) return MOE_OK;
    if (rows > 8) return MOE_ERR_UNSUPPORTED;
    if (!w->codes || !x || !y || !aligned16(w->codes) || !aligned16(x) || ((uintptr_t)y & 1u))
      return MOE_ERR_INVALID_ARG;
    const uintptr_t xa = (uintptr_t)x, ya = (uintptr_t)y;
    if (xa < ya + (size_t)rows * w->n * 2 && ya < xa + (size_t)rows * w->k * 2)
      return MOE_ERR_INVALID_ARG;
    if (launch_gemv_bf16(static_cast<const uint16_t*>(w->codes), x, y, rows, w->n, w->k,
                         stream) != hipSuccess)
      return MOE_ERR_DEVICE;
    return MOE_OK;
  }
  if (w->fmt != MOE_FMT_Q1_G128) return MOE_ERR_UNSUPPORTED;
  if (w->n < 0 || w->k <= 0) return MOE_ERR_INVALID_ARG;
  if (w->k % 128 || w->k > 16384) return MOE_ERR_UNSUPPORTED;
  if (rows < 0) return MOE_ERR_INVALID_ARG;
  if (rows == 0 || w->n == 0) return MOE_OK;
  // several rows: the MFMA form, which takes K in chunks of 256
  if (rows > 8 || (rows > 1 && w->k % 256)) return MOE_ERR_UNSUPPORTED;
  if (!w->codes || !x || !y || !aligned16(w->codes) || !aligned16(x) || !aligned16(y))
    return MOE_ERR_INVALID_ARG;
  const uintptr_t xa = (uintptr_t)x, ya = (uintptr_t)y;
  if (xa < ya + (size_t)rows * w->n * 2 && ya < xa + (size_t)rows * w->k * 2)
    return MOE_ERR_INVALID_ARG;
  if (launch_lowbit_q1(static_cast<const uint8_t*>(w->codes), x, y, rows, w->n, w->k, stream) !=
      hipSuccess)
    return MOE_ERR_DEVICE;
  return MOE_OK;
}

}  // extern "C"
