// abi.hip -- the C ABI of libmoe (declared in include/moe.h).
//
// Argument checking, workspace layout, weight packing entry, and the layer
// schedule.  The two-stream schedule follows the Hy3 on CANN NPU guide,
// section 8.5 (the shared expert is issued to a second stream whose start is
// ordered after Gating on the main stream; the main stream runs the routed
// path and waits for the shared expert before the final add) and the
// HunyuanImage-3.0 multi-stream article (the side stream is created once and
// handed to the module at construction, part 1-2; an input-ready event
// recorded on the main stream is awaited by the side stream, and a
// shared-done event recorded on the side stream is awaited by the main stream
// before output = shared + combined, part 3).
#include <hip/hip_runtime.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "../../include/moe.h"
#include "moe_common.hpp"
#include "moe_launch.hpp"

// Batches of at most this many tokens with 8- or 4-bit experts start the
// shared expert on the side stream before gating; the others start it beside
// the routed down GEMM.
constexpr int kSharedEarlyT = 64;

// Workspace of moe_layer_forward_noalloc: a static device array (one copy
// per GPU, held until the process ends).  In host code `scratch` names a
// host-side stand-in, not the device memory: its device address on each GPU
// comes from hipGetSymbolAddress (moe_ctx_create, with the device current)
// and only that address is ever passed to kernels.
static __device__ __align__(256) uint8_t scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch[kMaxDevices];     // device address of `scratch` per device, or null
}  // namespace

struct moe_ctx {
  int device;
  hipStream_t side;
  hipEvent_t ev_ready;   // recorded on the caller's stream where the shared expert may start
  hipEvent_t ev_done;    // recorded on the side stream after the shared expert
  char last_error[256];
  int profiling;
  hipEvent_t prof[2 * MOE_NUM_STAGES];   // start/stop per stage (timing events)
  unsigned ran;                          // stages recorded by the last call
};

namespace {

using namespace moe;

constexpr size_t kAlign = 256;
inline size_t align_up(size_t v) { return (v + kAlign - 1) & ~(kAlign - 1); }

int fmt_of(int dtype) {
  return dtype == MOE_F32 ? FMT_F32
         : dtype == MOE_BF16 ? FMT_BF16
         : dtype == MOE_MXFP4 ? FMT_MX4
         : dtype == MOE_FP8 ? FMT_FP8 : FMT_MX8;
}
size_t elem_bytes(int dtype) { return dtype == MOE_F32 ? 4 : dtype == MOE_BF16 ? 2 : 1; }
int chunk_elems(int dtype) { return dtype == MOE_F32 ? 64 : dtype == MOE_BF16 ? 128 : 256; }

// Block-scaled experts: the activations x and h are MX-fp8 (W8A8 and W4A8).
bool mx_act(const moe_desc *d) {
  return d->expert_dtype == MOE_MXFP8 || d->expert_dtype == MOE_MXFP4;
}
// Kernel weight format of the routed (shared = 0) or shared experts: a W4A8
// layer keeps its shared expert in MX-fp8 (the hybrid recipe of the Hy3 guide,
// section 8.2: routed experts W4A8, shared expert W8A8).
int weight_fmt(const moe_desc *d, int shared) {
  if (d->expert_dtype == MOE_MXFP4 && shared) return FMT_MX8;
  return fmt_of(d->expert_dtype);
}
// Bytes of one packed weight block (16 rows x one K chunk).
size_t wblock(int fmt) { return fmt == FMT_MX4 ? 2048 : kBlockBytes; }
// Static per-tensor FP8 experts: x and h are E4M3 under fixed scales.
bool fp8_act(const moe_desc *d) { return d->expert_dtype == MOE_FP8; }
// Bytes per activation element in the experts' input format (x, h).
size_t act_bytes(const moe_desc *d) {
  return (mx_act(d) || fp8_act(d)) ? 1 : elem_bytes(d->expert_dtype);
}
bool good_scale(float v) { return v > 0.0f && v < 3.0e38f; }
// moe_dtype of the routed (shared = 0) or shared experts' weights (the shared
// expert of a W4A8 layer is MX-fp8).
int weight_fmt_dtype(const moe_desc *d, int shared) {
  return (d->expert_dtype == MOE_MXFP4 && shared) ? MOE_MXFP8 : d->expert_dtype;
}

// Shape and dtype checks shared by every entry point.
moe_status check_desc(const moe_desc *d) {
  if (!d) return MOE_ERR_INVALID_ARG;
  if (d->hidden <= 0 || d->num_experts <= 0 || d->num_experts > 1024 || d->top_k <= 0 ||
      d->top_k > 16 || d->top_k > d->num_experts || d->inter <= 0 || d->shared_inter < 0)
    return MOE_ERR_INVALID_ARG;
  if (d->route_norm != 0 && d->route_norm != 1) return MOE_ERR_INVALID_ARG;
  for (int v : {d->act_dtype, d->expert_dtype, d->out_dtype})
    if (v < MOE_F32 || v > MOE_FP8) return MOE_ERR_INVALID_ARG;
  const bool f32 = d->act_dtype == MOE_F32 && d->expert_dtype == MOE_F32 && d->out_dtype == MOE_F32;
  const bool b16 = d->act_dtype == MOE_BF16 && d->expert_dtype == MOE_BF16 && d->out_dtype == MOE_BF16;
  const bool mx = d->act_dtype == MOE_BF16 && (d->expert_dtype == MOE_MXFP8 ||
                                              d->expert_dtype == MOE_MXFP4) &&
                  d->out_dtype == MOE_BF16;
  const bool f8 = d->act_dtype == MOE_BF16 && d->expert_dtype == MOE_FP8 &&
                  d->out_dtype == MOE_BF16;
  if (!(f32 || b16 || mx || f8)) return MOE_ERR_UNSUPPORTED;
  if (f8 && !(good_scale(d->fp8_x_scale) && good_scale(d->fp8_h_scale) &&
              good_scale(d->fp8_sh_h_scale)))
    return MOE_ERR_INVALID_ARG;
  // K chunks of 256 bytes; output tiles of 256 rows / 16-block groups
  const int im = (mx || f8) ? 256 : 128;
  if (d->hidden % 256 || d->inter % im || d->shared_inter % im) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

// Rows of the routed GEMMs and (token, slot) pair indices are int32: T * k
// must stay below 2^31.
bool too_many_pairs(const moe_desc *d, int32_t T) {
  return (long long)T * d->top_k > (long long)INT32_MAX;
}

// Layout of one call's workspace.  All offsets 256-byte aligned.
struct Layout {
  size_t logits, idx, w, counts, offsets, src, dest, perm, xq, xs, h, hs, sh_h, sh_hs, y, z, total;
};

Layout layout(const moe_desc *d, int T, int which) {
  Layout L;
  memset(&L, 0, sizeof L);
  const size_t P = (size_t)T * d->top_k, E = d->num_experts, H = d->hidden;
  const size_t I = d->inter, Is = d->shared_inter;
  const bool mx = mx_act(d);
  const size_t eh = act_bytes(d), eo = elem_bytes(d->out_dtype);
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off += align_up(bytes); return o; };
  const bool layer = which == MOE_WS_LAYER;
  if (which == MOE_WS_ROUTE || layer)
    L.logits = take(route_ws_bytes(T, (int)H, (int)E, d->act_dtype == MOE_BF16));
  if (layer) {
    L.idx = take(P * 4);
    L.w = take(P * 4);
    L.counts = take(E * 4);
    L.offsets = take((E + 1) * 4);
    L.src = take(P * 4);
    L.dest = take(P * 4);
  }
  if (which == MOE_WS_PERMUTE || layer) L.perm = take(permute_ws_bytes(T, (int)E));
  const bool routed = which == MOE_WS_GROUPED_FFN || layer;
  const bool shared = (which == MOE_WS_SHARED_FFN || layer) && Is > 0;
  if ((mx || fp8_act(d)) && (routed || shared)) {
    L.xq = take((size_t)T * H);
    if (mx) L.xs = take((size_t)T * H / 32);
  }
  if (routed) {
    L.h = take(P * I * eh);
    if (mx) L.hs = take(P * I / 32);
  }
  if (shared) {
    L.sh_h = take((size_t)T * Is * eh);
    if (mx) L.sh_hs = take((size_t)T * Is / 32);
  }
  if (layer) {
    L.y = take(P * H * eo);
    if (Is > 0) L.z = take((size_t)T * H * eo);
  }
  L.total = off;
  return L;
}

moe_status device_error(moe_ctx *ctx, hipError_t err, const char *where) {
  if (ctx) snprintf(ctx->last_error, sizeof ctx->last_error, "%s: %s", where, hipGetErrorString(err));
  return MOE_ERR_DEVICE;
}

// Stage timing: record the start/stop event of stage st on stream s.
struct StageTimer {
  moe_ctx *c;
  hipError_t start(int st, hipStream_t s) {
    if (!c->profiling) return hipSuccess;
    c->ran |= 1u << st;
    return hipEventRecord(c->prof[2 * st], s);
  }
  hipError_t stop(int st, hipStream_t s) {
    return c->profiling ? hipEventRecord(c->prof[2 * st + 1], s) : hipSuccess;
  }
};

moe_status check_ctx(moe_ctx *ctx) {
  if (!ctx) return MOE_ERR_INVALID_ARG;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev != ctx->device) return MOE_ERR_INVALID_ARG;
  return MOE_OK;
}

// One expert FFN (routed or shared) given activations already in the expert
// format (xa: x itself for f32/bf16, the MX codes for MX-fp8).  sh_y, sh_h
// (routed f32 / bf16 call only, shared and routed experts of one format and
// intermediate size): the shared expert rides along as one more segment of
// the routed grouped GEMMs, writing its h to sh_h and its output to sh_y.
hipError_t ffn(const moe_desc *d, const moe_weights *w, int shared, const void *xa,
               const uint8_t *xs, int T, const int32_t *sorted_src, const int32_t *offsets,
               void *y, void *h, uint8_t *hs, hipStream_t s, StageTimer *tm = nullptr,
               hipEvent_t after_first = nullptr, void *sh_y = nullptr, void *sh_h = nullptr) {
  const int st1 = shared ? MOE_STAGE_SHARED_GATE_UP : MOE_STAGE_GATE_UP;
  const int st2 = shared ? MOE_STAGE_SHARED_DOWN : MOE_STAGE_DOWN;
  const int F = weight_fmt(d, shared);
  const int H = d->hidden, I = shared ? d->shared_inter : d->inter;
  const int E = shared ? 1 : d->num_experts;
  const int rows = shared ? T : T * d->top_k;
  const size_t eb = act_bytes(d);                 // token-side bytes per element
  const int ce = chunk_elems(d->expert_dtype);
  const size_t wb = wblock(F);

  GemmArgs g1;
  memset(&g1, 0, sizeof g1);
  g1.w = (const uint8_t *)(shared ? w->sh_gate_up : w->gate_up);
  g1.w_scale = (const uint16_t *)(shared ? w->sh_gate_up_scale : w->gate_up_scale);
  g1.w_expert_stride = (size_t)(2 * I / 16) * (H / ce) * wb;
  g1.ws_expert_stride = (size_t)(2 * I / 16) * (H / ce) * 64;
  g1.a = (const uint8_t *)xa;
  g1.a_scale = xs;
  g1.a_row_bytes = (long long)H * eb;
  g1.a_bytes = (long long)T * H * (long long)eb;
  g1.sorted_src = shared ? nullptr : sorted_src;
  g1.k_route = d->top_k;
  g1.offsets = shared ? nullptr : offsets;
  g1.rows = rows;
  g1.E = E;
  g1.N = 2 * I;
  g1.K = H;
  g1.out = h;
  g1.out_scale = hs;
  g1.n_out = I;
  if (sh_y) {
    g1.w2 = (const uint8_t *)w->sh_gate_up;
    g1.a2 = (const uint8_t *)xa;
    g1.a2_bytes = g1.a_bytes;
    g1.out2 = sh_h;
    g1.rows2 = T;
  }
  // static per-tensor FP8: weight scales [E][2], the x scale, and the scale
  // h is quantised with (then the down GEMM's activation scale)
  const float sh = shared ? d->fp8_sh_h_scale : d->fp8_h_scale;
  if (F == FMT_FP8) {
    g1.w_tscale = (const float *)(shared ? w->sh_gate_up_scale : w->gate_up_scale);
    g1.w_scale = nullptr;
    g1.a_tscale = d->fp8_x_scale;
    g1.out_tscale = sh;
  }
  hipError_t err;
  if (tm && (err = tm->start(st1, s)) != hipSuccess) return err;
  // the SwiGLU output h is the down GEMM's input: MX-fp8 for MX experts,
  // E4M3 under its static scale for FP8
  err = launch_grouped_gemm(g1, F, EPI_SWIGLU, mx_act(d) ? FMT_MX8 : F, rows, s);
  if (err != hipSuccess) return err;
  if (tm && (err = tm->stop(st1, s)) != hipSuccess) return err;
  if (after_first && (err = hipEventRecord(after_first, s)) != hipSuccess) return err;

  GemmArgs g2;
  memset(&g2, 0, sizeof g2);
  g2.w = (const uint8_t *)(shared ? w->sh_down : w->down);
  g2.w_scale = (const uint16_t *)(shared ? w->sh_down_scale : w->down_scale);
  g2.w_expert_stride = (size_t)(H / 16) * (I / ce) * wb;
  g2.ws_expert_stride = (size_t)(H / 16) * (I / ce) * 64;
  g2.a = (const uint8_t *)h;
  g2.a_scale = hs;
  g2.a_row_bytes = (long long)I * eb;
  g2.a_bytes = (long long)rows * I * (long long)eb;
  g2.sorted_src = nullptr;
  g2.k_route = d->top_k;
  g2.offsets = shared ? nullptr : offsets;
  g2.rows = rows;
  g2.E = E;
  g2.N = H;
  g2.K = I;
  g2.out = y;
  g2.out_scale = nullptr;
  g2.n_out = H;
  if (sh_y) {
    g2.w2 = (const uint8_t *)w->sh_down;
    g2.a2 = (const uint8_t *)sh_h;
    g2.a2_bytes = (long long)T * I * (long long)eb;
    g2.out2 = sh_y;
    g2.rows2 = T;
  }
  if (F == FMT_FP8) {
    g2.w_tscale = (const float *)(shared ? w->sh_down_scale : w->down_scale);
    g2.w_scale = nullptr;
    g2.a_tscale = sh;
  }
  if (tm && (err = tm->start(st2, s)) != hipSuccess) return err;
  err = launch_grouped_gemm(g2, F, EPI_PLAIN, fmt_of(d->out_dtype), rows, s);
  if (err != hipSuccess) return err;
  if (tm) err = tm->stop(st2, s);
  return err;
}

// Device arrays the kernels read or write with 16-byte vector accesses
// (activations, outputs, workspaces, packed weights) must start 16-byte
// aligned; NULL passes (the callers check presence separately).
inline bool al16(const void *p) { return ((uintptr_t)p & 15) == 0; }

bool weights_ok(const moe_desc *d, const moe_weights *w, int need_router, int need_routed,
                int need_shared) {
  if (!w) return false;
  if (!al16(w->router_w) || !al16(w->gate_up) || !al16(w->down) || !al16(w->sh_gate_up) ||
      !al16(w->sh_down) || !al16(w->gate_up_scale) || !al16(w->down_scale) ||
      !al16(w->sh_gate_up_scale) || !al16(w->sh_down_scale))
    return false;
  const bool mx = mx_act(d) || fp8_act(d);     // both need the scale arrays
  if (need_router && !w->router_w) return false;
  if (need_routed && (!w->gate_up || !w->down || (mx && (!w->gate_up_scale || !w->down_scale))))
    return false;
  if (need_shared && d->shared_inter > 0 &&
      (!w->sh_gate_up || !w->sh_down || (mx && (!w->sh_gate_up_scale || !w->sh_down_scale))))
    return false;
  return true;
}

}  // namespace

extern "C" {

const char *moe_status_string(moe_status s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported configuration";
    case MOE_ERR_WORKSPACE: return "workspace too small";
    case MOE_ERR_DEVICE: return "device (HIP) error";
  }
  return "unknown status";
}

moe_status moe_ctx_create(int device, void *side_stream, moe_ctx **out) {
  if (!out) return MOE_ERR_INVALID_ARG;
  *out = nullptr;
  int n = 0;
  if (hipGetDeviceCount(&n) != hipSuccess || device < 0 || device >= n) return MOE_ERR_DEVICE;
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, device) != hipSuccess) return MOE_ERR_DEVICE;
  if (strncmp(prop.gcnArchName, "gfx950", 6) != 0) return MOE_ERR_DEVICE;
  int cur = -1;
  if (hipGetDevice(&cur) != hipSuccess) return MOE_ERR_DEVICE;
  if (cur != device && hipSetDevice(device) != hipSuccess) return MOE_ERR_DEVICE;
  if (device >= kMaxDevices) {
    if (cur != device) (void)hipSetDevice(cur);
    return MOE_ERR_DEVICE;
  }
  {
    // the no-allocation entry point's workspace on this device (current now)
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch[device]) {
      void *p = nullptr;
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
        if (cur != device) (void)hipSetDevice(cur);
        return MOE_ERR_DEVICE;
      }
      g_scratch[device] = p;
    }
  }
  moe_ctx *c = new (std::nothrow) moe_ctx;
  if (!c) return MOE_ERR_DEVICE;
  memset(c, 0, sizeof *c);
  c->device = device;
  c->side = (hipStream_t)side_stream;
  hipError_t e1 = hipEventCreateWithFlags(&c->ev_ready, hipEventDisableTiming);
  hipError_t e2 = hipEventCreateWithFlags(&c->ev_done, hipEventDisableTiming);
  if (cur != device) (void)hipSetDevice(cur);
  if (e1 != hipSuccess || e2 != hipSuccess) {
    if (e1 == hipSuccess) (void)hipEventDestroy(c->ev_ready);
    if (e2 == hipSuccess) (void)hipEventDestroy(c->ev_done);
    delete c;
    return MOE_ERR_DEVICE;
  }
  *out = c;
  return MOE_OK;
}

moe_status moe_ctx_destroy(moe_ctx *ctx) {
  if (!ctx) return MOE_ERR_INVALID_ARG;
  (void)hipEventDestroy(ctx->ev_ready);
  (void)hipEventDestroy(ctx->ev_done);
  if (ctx->profiling)
    for (int i = 0; i < 2 * MOE_NUM_STAGES; ++i) (void)hipEventDestroy(ctx->prof[i]);
  delete ctx;
  return MOE_OK;
}

const char *moe_ctx_last_error(const moe_ctx *ctx) { return ctx ? ctx->last_error : ""; }

moe_status moe_ctx_set_profiling(moe_ctx *ctx, int enable) {
  moe_status st = check_ctx(ctx);
  if (st != MOE_OK) return st;
  if (enable && !ctx->profiling) {
    for (int i = 0; i < 2 * MOE_NUM_STAGES; ++i) {
      hipError_t err = hipEventCreate(&ctx->prof[i]);
      if (err != hipSuccess) {
        for (int j = 0; j < i; ++j) (void)hipEventDestroy(ctx->prof[j]);
        return device_error(ctx, err, "moe_ctx_set_profiling");
      }
    }
    ctx->profiling = 1;
    ctx->ran = 0;
  } else if (!enable && ctx->profiling) {
    for (int i = 0; i < 2 * MOE_NUM_STAGES; ++i) (void)hipEventSynchronize(ctx->prof[i]);
    for (int i = 0; i < 2 * MOE_NUM_STAGES; ++i) (void)hipEventDestroy(ctx->prof[i]);
    ctx->profiling = 0;
    ctx->ran = 0;
  }
  return MOE_OK;
}

moe_status moe_ctx_stage_ms(moe_ctx *ctx, float *ms) {
  moe_status st = check_ctx(ctx);
  if (st != MOE_OK) return st;
  if (!ms || !ctx->profiling) return MOE_ERR_INVALID_ARG;
  for (int i = 0; i < MOE_NUM_STAGES; ++i) {
    ms[i] = 0.0f;
    if (!(ctx->ran & (1u << i))) continue;
    hipError_t err = hipEventSynchronize(ctx->prof[2 * i + 1]);
    if (err == hipSuccess) err = hipEventElapsedTime(&ms[i], ctx->prof[2 * i], ctx->prof[2 * i + 1]);
    if (err != hipSuccess) return device_error(ctx, err, "moe_ctx_stage_ms");
  }
  return MOE_OK;
}

size_t moe_workspace_bytes(const moe_desc *desc, int32_t T, int which) {
  if (check_desc(desc) != MOE_OK || T < 0 || too_many_pairs(desc, T) || which < MOE_WS_ROUTE ||
      which > MOE_WS_LAYER)
    return 0;
  return layout(desc, T, which).total;
}

size_t moe_packed_bytes(const moe_desc *desc, int shared, int which) {
  if (check_desc(desc) != MOE_OK || (shared != 0 && shared != 1)) return 0;
  const size_t E = shared ? 1 : desc->num_experts, H = desc->hidden;
  const size_t I = shared ? desc->shared_inter : desc->inter;
  const int F = weight_fmt(desc, shared);
  const bool mx = mx_act(desc);
  // bytes per 32 weights (E2M1 packs two per byte)
  const size_t per32 = F == FMT_F32 ? 128 : F == FMT_BF16 ? 64 : F == FMT_MX4 ? 16 : 32;
  const bool f8 = F == FMT_FP8;     // fp32 per-tensor scales
  switch (which) {
    case MOE_PACK_GATE_UP: return E * 2 * I * H / 32 * per32;
    case MOE_PACK_DOWN: return E * H * I / 32 * per32;
    case MOE_PACK_GATE_UP_SCALE: return f8 ? E * 2 * sizeof(float) : mx ? E * 2 * I * H / 32 : 0;
    case MOE_PACK_DOWN_SCALE: return f8 ? E * sizeof(float) : mx ? E * H * I / 32 : 0;
  }
  return 0;
}

moe_status moe_pack_experts(const moe_desc *desc, int shared, int src_dtype, const void *gate,
                            const void *up, const void *down, void *gate_up_out, void *down_out,
                            uint8_t *gate_up_scale_out, uint8_t *down_scale_out, void *stream) {
  moe_status st = check_desc(desc);
  if (st != MOE_OK) return st;
  if (shared != 0 && shared != 1) return MOE_ERR_INVALID_ARG;
  if (src_dtype != MOE_F32 && src_dtype != MOE_BF16) return MOE_ERR_INVALID_ARG;
  const int E = shared ? 1 : desc->num_experts, H = desc->hidden;
  const int I = shared ? desc->shared_inter : desc->inter;
  if (I == 0) return MOE_OK;
  const bool mx = mx_act(desc) || fp8_act(desc);
  if (!gate || !up || !down || !gate_up_out || !down_out) return MOE_ERR_INVALID_ARG;
  if (mx && (!gate_up_scale_out || !down_scale_out)) return MOE_ERR_INVALID_ARG;
  if (!al16(gate_up_out) || !al16(down_out) || !al16(gate_up_scale_out) || !al16(down_scale_out))
    return MOE_ERR_INVALID_ARG;
  const int F = weight_fmt(desc, shared);
  const bool f8 = F == FMT_FP8;
  hipStream_t s = (hipStream_t)stream;
  hipError_t err = launch_pack(gate, up, src_dtype == MOE_BF16, E, 2 * I, H, 1, F,
                               (uint8_t *)gate_up_out,
                               f8 ? nullptr : (uint16_t *)gate_up_scale_out,
                               f8 ? (float *)gate_up_scale_out : nullptr, s);
  if (err == hipSuccess)
    err = launch_pack(down, nullptr, src_dtype == MOE_BF16, E, H, I, 0, F, (uint8_t *)down_out,
                      f8 ? nullptr : (uint16_t *)down_scale_out,
                      f8 ? (float *)down_scale_out : nullptr, s);
  return err == hipSuccess ? MOE_OK : MOE_ERR_DEVICE;
}

moe_status moe_fp8_quantize(const void *src, int src_dtype, int64_t n, float scale, uint8_t *q,
                            void *stream) {
  if (n < 0 || n % 8 || !good_scale(scale)) return MOE_ERR_INVALID_ARG;
  if (src_dtype != MOE_F32 && src_dtype != MOE_BF16) return MOE_ERR_INVALID_ARG;
  if (n == 0) return MOE_OK;
  if (!src || !q) return MOE_ERR_INVALID_ARG;
  hipError_t err = launch_fp8_quantize(src, src_dtype == MOE_BF16, n, scale, q,
                                       (hipStream_t)stream);
  return err == hipSuccess ? MOE_OK : MOE_ERR_DEVICE;
}

moe_status moe_mx_quantize(const void *src, int src_dtype, int64_t rows, int64_t cols, uint8_t *q,
                           uint8_t *scale, void *stream) {
  if (rows < 0 || cols <= 0 || cols % 32) return MOE_ERR_INVALID_ARG;
  if (src_dtype != MOE_F32 && src_dtype != MOE_BF16) return MOE_ERR_INVALID_ARG;
  if (rows == 0) return MOE_OK;
  if (!src || !q || !scale) return MOE_ERR_INVALID_ARG;
  hipError_t err = launch_mx_quantize(src, src_dtype == MOE_BF16, rows, cols, q, scale,
                                      (hipStream_t)stream);
  return err == hipSuccess ? MOE_OK : MOE_ERR_DEVICE;
}

moe_status moe_route(moe_ctx *ctx, const moe_desc *desc, const void *x, int32_t T,
                     const float *router_w, const float *router_bias, int32_t *topk_idx,
                     float *topk_w, void *ws, size_t ws_bytes, void *stream) {
  moe_status st = check_desc(desc);
  if (st != MOE_OK) return st;
  if ((st = check_ctx(ctx)) != MOE_OK) return st;
  if (T < 0) return MOE_ERR_INVALID_ARG;
  if (too_many_pairs(desc, T)) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!x || !router_w || !topk_idx || !topk_w || !ws) return MOE_ERR_INVALID_ARG;
  if (!al16(x) || !al16(router_w) || !al16(ws)) return MOE_ERR_INVALID_ARG;
  Layout L = layout(desc, T, MOE_WS_ROUTE);
  if (ws_bytes < L.total) return MOE_ERR_WORKSPACE;
  hipError_t err = launch_route(x, desc->act_dtype == MOE_BF16, router_w, router_bias,
                                (float *)((char *)ws + L.logits), topk_idx, topk_w, T,
                                desc->hidden, desc->num_experts, desc->top_k,
                                desc->router_scaling_factor, desc->route_norm, (hipStream_t)stream);
  return err == hipSuccess ? MOE_OK : device_error(ctx, err, "moe_route");
}

moe_status moe_permute(moe_ctx *ctx, const moe_desc *desc, const int32_t *topk_idx, int32_t T,
                       int32_t *expert_counts, int32_t *expert_offsets, int32_t *sorted_src,
                       int32_t *dest, void *ws, size_t ws_bytes, void *stream) {
  moe_status st = check_desc(desc);
  if (st != MOE_OK) return st;
  if ((st = check_ctx(ctx)) != MOE_OK) return st;
  if (T < 0) return MOE_ERR_INVALID_ARG;
  if (too_many_pairs(desc, T)) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!topk_idx || !expert_counts || !expert_offsets || !sorted_src || !dest || !ws)
    return MOE_ERR_INVALID_ARG;
  Layout L = layout(desc, T, MOE_WS_PERMUTE);
  if (ws_bytes < L.total) return MOE_ERR_WORKSPACE;
  hipError_t err = launch_permute(topk_idx, T, desc->num_experts, desc->top_k, expert_counts,
                                  expert_offsets, sorted_src, dest, (char *)ws + L.perm,
                                  (hipStream_t)stream);
  return err == hipSuccess ? MOE_OK : device_error(ctx, err, "moe_permute");
}

moe_status moe_grouped_ffn(moe_ctx *ctx, const moe_desc *desc, const moe_weights *w, int shared,
                           const void *x, int32_t T, const int32_t *sorted_src,
                           const int32_t *expert_offsets, void *y, void *ws, size_t ws_bytes,
                           void *stream) {
  moe_status st = check_desc(desc);
  if (st != MOE_OK) return st;
  if ((st = check_ctx(ctx)) != MOE_OK) return st;
  if (shared != 0 && shared != 1) return MOE_ERR_INVALID_ARG;
  if (T < 0) return MOE_ERR_INVALID_ARG;
  if (too_many_pairs(desc, T)) return MOE_ERR_UNSUPPORTED;
  if (T == 0 || (shared && desc->shared_inter == 0)) return MOE_OK;
  if (!x || !y || !ws || !weights_ok(desc, w, 0, !shared, shared)) return MOE_ERR_INVALID_ARG;
  if (!shared && (!sorted_src || !expert_offsets)) return MOE_ERR_INVALID_ARG;
  if (!al16(x) || !al16(y) || !al16(ws)) return MOE_ERR_INVALID_ARG;
  Layout L = layout(desc, T, shared ? MOE_WS_SHARED_FFN : MOE_WS_GROUPED_FFN);
  if (ws_bytes < L.total) return MOE_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  char *base = (char *)ws;
  const bool mx = mx_act(desc);
  const void *xa = x;
  const uint8_t *xs = nullptr;
  hipError_t err = hipSuccess;
  if (mx) {
    err = launch_mx_quantize(x, 1, T, desc->hidden, (uint8_t *)base + L.xq,
                             (uint8_t *)base + L.xs, s);
    if (err != hipSuccess) return device_error(ctx, err, "moe_grouped_ffn");
    xa = base + L.xq;
    xs = (const uint8_t *)base + L.xs;
  } else if (fp8_act(desc)) {
    err = launch_fp8_quantize(x, 1, (long long)T * desc->hidden, desc->fp8_x_scale,
                              (uint8_t *)base + L.xq, s);
    if (err != hipSuccess) return device_error(ctx, err, "moe_grouped_ffn");
    xa = base + L.xq;
  }
  err = ffn(desc, w, shared, xa, xs, T, sorted_src, expert_offsets, y,
            base + (shared ? L.sh_h : L.h),
            mx ? (uint8_t *)base + (shared ? L.sh_hs : L.hs) : nullptr, s);
  return err == hipSuccess ? MOE_OK : device_error(ctx, err, "moe_grouped_ffn");
}

moe_status moe_combine(moe_ctx *ctx, const moe_desc *desc, const void *y, const int32_t *dest,
                       const float *topk_w, const void *shared_out, int32_t T, void *out,
                       void *stream) {
  moe_status st = check_desc(desc);
  if (st != MOE_OK) return st;
  if ((st = check_ctx(ctx)) != MOE_OK) return st;
  if (T < 0) return MOE_ERR_INVALID_ARG;
  if (too_many_pairs(desc, T)) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!y || !dest || !topk_w || !out) return MOE_ERR_INVALID_ARG;
  if (!al16(y) || !al16(shared_out) || !al16(out)) return MOE_ERR_INVALID_ARG;
  const int of = fmt_of(desc->out_dtype);
  hipError_t err = launch_combine(y, of, dest, topk_w, shared_out, T, desc->hidden, desc->top_k,
                                  out, of, (hipStream_t)stream);
  return err == hipSuccess ? MOE_OK : device_error(ctx, err, "moe_combine");
}

moe_status moe_layer_ws_topk(const moe_desc *desc, int32_t T, size_t *idx_offset,
                             size_t *w_offset) {
  moe_status st = check_desc(desc);
  if (st != MOE_OK) return st;
  if (T < 0 || !idx_offset || !w_offset) return MOE_ERR_INVALID_ARG;
  if (too_many_pairs(desc, T)) return MOE_ERR_UNSUPPORTED;
  Layout L = layout(desc, T, MOE_WS_LAYER);
  *idx_offset = L.idx;
  *w_offset = L.w;
  return MOE_OK;
}

moe_status moe_layer_forward(moe_ctx *ctx, const moe_desc *desc, const moe_weights *w,
                             const void *x, int32_t T, void *out, void *ws, size_t ws_bytes,
                             void *stream) {
  moe_status st = check_desc(desc);
  if (st != MOE_OK) return st;
  if ((st = check_ctx(ctx)) != MOE_OK) return st;
  if (T < 0) return MOE_ERR_INVALID_ARG;
  if (too_many_pairs(desc, T)) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!x || !out || !ws || !weights_ok(desc, w, 1, 1, 1)) return MOE_ERR_INVALID_ARG;
  if (!al16(x) || !al16(out) || !al16(ws)) return MOE_ERR_INVALID_ARG;
  Layout L = layout(desc, T, MOE_WS_LAYER);
  if (ws_bytes < L.total) return MOE_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  char *b = (char *)ws;
  const int H = desc->hidden, E = desc->num_experts, k = desc->top_k;
  const bool mx = mx_act(desc);
  const bool has_shared = desc->shared_inter > 0;
  int32_t *idx = (int32_t *)(b + L.idx);
  float *tw = (float *)(b + L.w);
  int32_t *offsets = (int32_t *)(b + L.offsets);
  int32_t *src = (int32_t *)(b + L.src);
  int32_t *dest = (int32_t *)(b + L.dest);
  hipError_t err;
  StageTimer tm{ctx};
  ctx->ran = 0;
#define MOE_TRY(call, where)                          \
  do {                                                \
    err = (call);                                     \
    if (err != hipSuccess) return device_error(ctx, err, where); \
  } while (0)

  const void *xa = x;
  const uint8_t *xs = nullptr;
  if (mx) {
    // the expert-format activations feed both the shared and the routed experts
    MOE_TRY(tm.start(MOE_STAGE_MX_QUANT, s), "timing");
    MOE_TRY(launch_mx_quantize(x, 1, T, H, (uint8_t *)b + L.xq, (uint8_t *)b + L.xs, s),
            "activation quantisation");
    MOE_TRY(tm.stop(MOE_STAGE_MX_QUANT, s), "timing");
    xa = b + L.xq;
    xs = (const uint8_t *)b + L.xs;
  } else if (fp8_act(desc)) {
    MOE_TRY(tm.start(MOE_STAGE_MX_QUANT, s), "timing");
    MOE_TRY(launch_fp8_quantize(x, 1, (long long)T * H, desc->fp8_x_scale, (uint8_t *)b + L.xq, s),
            "activation quantisation");
    MOE_TRY(tm.stop(MOE_STAGE_MX_QUANT, s), "timing");
    xa = b + L.xq;
  }
  // Shared expert on the side stream.  It needs only the activations.  For
  // larger batches it is started once the routed gate/up GEMM is queued (the
  // input-ready event is recorded after it), so it runs beside the routed
  // down GEMM: beside gating and permutation it slows those short,
  // latency-bound kernels by more than it saves.  For decode-sized batches
  // (T <= kSharedEarlyT) with 8- or 4-bit experts it starts at once,
  // beside gating and the routed gate/up GEMM: there the routed down GEMM
  // is shorter than the 8-bit shared expert, which would otherwise lengthen
  // the layer (W4A8 decode 0.398 -> 0.370 ms).  A bf16 decode batch keeps
  // the late start: the early one slows gating (24 -> 33 us) by more than it
  // saves (Hy3 decode 1.048 ms against 1.035).
  //
  // The side stream is used where the overlap pays.  The HunyuanImage-3.0
  // article (caveats) warns that under contention the second stream may not
  // lower the wall time, and that is what was measured at the two ends
  // (layer time, two streams against one, same build):
  //  * a layer whose shared expert holds under 1 MiB of weights is bound by
  //    launch latency, and the cross-stream events cost more than the
  //    overlap saves (fp32 H = 256 layer: 0.093 ms against 0.076);
  //  * with 256 or more rows per routed expert every GEMM is bound by the
  //    matrix cores and the shared expert's tiles only compete with the
  //    routed down GEMM's (Hy3 prefill, 341 rows per expert: 3.204 ms
  //    against 3.163);
  //  * in between the overlap pays: Hy3 decode 1.088 against 1.097 ms,
  //    Hy4-skew (64 rows per expert) 2.084 against 2.120, MX-fp8 at 4096
  //    tokens (171 rows per expert) 1.393 against 1.433.
  // Otherwise the shared expert runs on the caller's stream, in the same
  // place in the order.  There, for f32 / bf16 experts whose shared and
  // routed intermediate sizes agree, its two GEMMs are folded into the
  // routed ones as one more segment at the end of the tile list: its tiles
  // fill the routed GEMM's last, partial round instead of a launch of their
  // own (Hy3 prefill: 3.130 ms against 3.167; gate/up with the shared
  // expert's 1.780 ms against 1.602 + 0.208).
  const size_t shared_weight_bytes =
      (size_t)3 * H * desc->shared_inter * elem_bytes(weight_fmt_dtype(desc, 1));
  const bool side_pays = shared_weight_bytes >= ((size_t)1 << 20) &&
                         (long long)T * k < 256LL * E;
  const bool two = has_shared && ctx->side && ctx->side != s && side_pays;
  const bool early = two && (mx || fp8_act(desc)) && T <= kSharedEarlyT;
  const bool fold = has_shared && !two && !mx && !fp8_act(desc) &&
                    desc->shared_inter == desc->inter &&
                    weight_fmt(desc, 0) == weight_fmt(desc, 1) && E < 1024;
  auto shared_expert = [&]() -> hipError_t {
    hipStream_t ss = two ? ctx->side : s;
    hipError_t e;
    if (two && (e = hipStreamWaitEvent(ss, ctx->ev_ready, 0)) != hipSuccess) return e;
    e = ffn(desc, w, 1, xa, xs, T, nullptr, nullptr, b + L.z, b + L.sh_h,
            mx ? (uint8_t *)b + L.sh_hs : nullptr, ss, &tm);
    if (e != hipSuccess) return e;
    return two ? hipEventRecord(ctx->ev_done, ss) : hipSuccess;
  };
  if (early) {
    MOE_TRY(hipEventRecord(ctx->ev_ready, s), "input-ready event");
    MOE_TRY(shared_expert(), "shared expert");
  }
  // Gating on the main stream.
  MOE_TRY(tm.start(MOE_STAGE_ROUTE, s), "timing");
  MOE_TRY(launch_route(x, desc->act_dtype == MOE_BF16, w->router_w, w->router_bias,
                       (float *)(b + L.logits), idx, tw, T, H, E, k, desc->router_scaling_factor,
                       desc->route_norm, s),
          "gating");
  MOE_TRY(tm.stop(MOE_STAGE_ROUTE, s), "timing");
  // Routed path on the main stream: InitRouting, grouped GEMM.
  MOE_TRY(tm.start(MOE_STAGE_PERMUTE, s), "timing");
  MOE_TRY(launch_permute(idx, T, E, k, (int32_t *)(b + L.counts), offsets, src, dest, b + L.perm,
                         s),
          "permutation");
  MOE_TRY(tm.stop(MOE_STAGE_PERMUTE, s), "timing");
  MOE_TRY(ffn(desc, w, 0, xa, xs, T, src, offsets, b + L.y, b + L.h,
              mx ? (uint8_t *)b + L.hs : nullptr, s, &tm,
              two && !early ? ctx->ev_ready : nullptr, fold ? b + L.z : nullptr,
              fold ? b + L.sh_h : nullptr),
          "routed experts");
  if (has_shared && !early && !fold) MOE_TRY(shared_expert(), "shared expert");
  // Join, then FinalizeRouting + shared add.
  if (two) MOE_TRY(hipStreamWaitEvent(s, ctx->ev_done, 0), "main stream wait");
  const int of = fmt_of(desc->out_dtype);
  MOE_TRY(tm.start(MOE_STAGE_COMBINE, s), "timing");
  MOE_TRY(launch_combine(b + L.y, of, dest, tw, has_shared ? b + L.z : nullptr, T, H, k, out, of, s),
          "combine");
  MOE_TRY(tm.stop(MOE_STAGE_COMBINE, s), "timing");
#undef MOE_TRY
  return MOE_OK;
}

moe_status moe_layer_forward_noalloc(moe_ctx *ctx, const moe_desc *desc, const moe_weights *w,
                                     const void *x, int32_t T, void *out, void *stream) {
  moe_status st = check_desc(desc);
  if (st != MOE_OK) return st;
  if ((st = check_ctx(ctx)) != MOE_OK) return st;
  if (T < 0) return MOE_ERR_INVALID_ARG;
  if (too_many_pairs(desc, T)) return MOE_ERR_UNSUPPORTED;
  const size_t need = layout(desc, T, MOE_WS_LAYER).total;
  if (need > MOE_NOALLOC_SCRATCH_BYTES) {
    snprintf(ctx->last_error, sizeof ctx->last_error,
             "moe_layer_forward_noalloc: %d tokens need %zu bytes of workspace, above the "
             "%zu-byte static scratch",
             (int)T, need, (size_t)MOE_NOALLOC_SCRATCH_BYTES);
    return MOE_ERR_WORKSPACE;
  }
  void *ws;
  {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    ws = g_scratch[ctx->device];
  }
  if (!ws) return MOE_ERR_DEVICE;
  return moe_layer_forward(ctx, desc, w, x, T, out, ws, MOE_NOALLOC_SCRATCH_BYTES, stream);
}

}  // extern "C"
