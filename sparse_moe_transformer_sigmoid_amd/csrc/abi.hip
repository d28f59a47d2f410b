// C ABI of libmoe: argument validation, workspace layout and the launch
// sequence of each entry point (declared in include/moe.h).
#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "kernels.h"

using namespace moe;

namespace {

thread_local std::string g_err;
// profiling events armed by moe_profile_arm on this thread (one-shot)
thread_local hipEvent_t g_ev[MOE_KID_COUNT][2] = {};

constexpr int64_t kMaxTokens = 65536;

moe_status_t fail(moe_status_t s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
moe_status_t fail(moe_status_t s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}

// records the armed start event (if any) of kernel `kid` before its launch
// and the stop event after it; one-shot.  A launch into a stream that is being
// captured into a graph records nothing and leaves the events armed.
struct Probe {
  int kid;
  hipStream_t st;
  bool on = false;
  Probe(int k, hipStream_t s) : kid(k), st(s) {
    if (!g_ev[kid][0]) return;
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(st, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone) return;
    on = true;
    hipEventRecord(g_ev[kid][0], st);
  }
  ~Probe() {
    if (!on) return;
    hipEventRecord(g_ev[kid][1], st);
    g_ev[kid][0] = g_ev[kid][1] = nullptr;
  }
};

// hipGetLastError reports the last error of any HIP call on the thread; the
// entry points clear a stale one before their first launch so that only
// their own launch failures are reported
#define MOE_LAUNCH(kid, expr)                                                                \
  do {                                                                                       \
    hipError_t e_;                                                                           \
    {                                                                                        \
      Probe probe_(kid, st);                                                                 \
      e_ = (expr);                                                                           \
    }                                                                                        \
    if (e_ != hipSuccess)                                                                    \
      return fail(MOE_ERR_HIP, "%s: %s", #expr, hipGetErrorString(e_));                      \
  } while (0)

int act_size(int dt) { return dt == MOE_F32 ? 4 : 2; }
bool fp8(const moe_config_t* c) { return c->weight_dtype == MOE_FP8_E4M3; }
int shared_F(const moe_config_t* c) { return c->n_shared_experts * c->moe_intermediate_size; }

// `routing`: also check the fields only routing reads (k <= E, groups).  The
// expert FFN alone takes k as a row capacity per token, so one expert-parallel
// rank can hold fewer local experts than a token selects.
moe_status_t check_cfg(const moe_config_t* c, bool routing = true) {
  if (!c) return fail(MOE_ERR_INVALID_ARG, "cfg is NULL");
  if (c->scoring_func != MOE_SCORING_SIGMOID)
    return fail(MOE_ERR_UNSUPPORTED, "scoring_func %d: only sigmoid (0) is implemented", c->scoring_func);
  if (c->topk_method != MOE_TOPK_NOAUX_TC)
    return fail(MOE_ERR_UNSUPPORTED, "topk_method %d: only noaux_tc (0) is implemented", c->topk_method);
  const int H = c->hidden_size, F = c->moe_intermediate_size, E = c->n_routed_experts;
  const int k = c->num_experts_per_tok;
  if (H <= 0 || H % 128 || F <= 0 || F % 128)
    return fail(MOE_ERR_INVALID_ARG, "hidden_size %d and moe_intermediate_size %d must be positive multiples of 128", H, F);
  if (E < 1 || E > 1023) return fail(MOE_ERR_INVALID_ARG, "n_routed_experts %d not in 1..1023", E);
  if (k < 1 || k > 32) return fail(MOE_ERR_INVALID_ARG, "num_experts_per_tok %d not in 1..32", k);
  if (c->n_shared_experts < 0 || c->n_shared_experts > 8)
    return fail(MOE_ERR_INVALID_ARG, "n_shared_experts %d not in 0..8", c->n_shared_experts);
  if (routing) {
    if (k > E) return fail(MOE_ERR_INVALID_ARG, "num_experts_per_tok %d exceeds n_routed_experts %d", k, E);
    if (c->n_group < 1 || c->n_group > 64 || E % c->n_group)
      return fail(MOE_ERR_INVALID_ARG, "n_group %d must divide n_routed_experts %d and be <= 64", c->n_group, E);
    if (c->topk_group < 1 || c->topk_group > c->n_group)
      return fail(MOE_ERR_INVALID_ARG, "topk_group %d not in 1..n_group", c->topk_group);
    if (k > c->topk_group * (E / c->n_group))
      return fail(MOE_ERR_INVALID_ARG, "num_experts_per_tok %d exceeds the experts of topk_group groups", k);
  }
  const bool ok_dt = (c->act_dtype == MOE_F32 && c->weight_dtype == MOE_F32) ||
                     (c->act_dtype == MOE_BF16 && c->weight_dtype == MOE_BF16) ||
                     (c->act_dtype == MOE_BF16 && c->weight_dtype == MOE_FP8_E4M3);
  if (!ok_dt)
    return fail(MOE_ERR_UNSUPPORTED, "dtype pair act %d / weight %d not supported", c->act_dtype, c->weight_dtype);
  if (fp8(c) && (c->weight_block_size[0] != 128 || c->weight_block_size[1] != 128))
    return fail(MOE_ERR_UNSUPPORTED, "fp8 weights need weight_block_size {128,128}");
  if (c->act_dtype == MOE_F32 && (H > 8192 || shared_F(c) > 8192 || F > 8192))
    return fail(MOE_ERR_UNSUPPORTED, "fp32 path limited to hidden/intermediate sizes <= 8192");
  return MOE_OK;
}

moe_status_t check_T(int64_t T) {
  if (T < 0 || T > kMaxTokens) return fail(MOE_ERR_INVALID_ARG, "num_tokens %lld not in 0..%lld", (long long)T, (long long)kMaxTokens);
  return MOE_OK;
}

bool aligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

#define NEED(p)                                                                              \
  do {                                                                                       \
    if (!(p)) return fail(MOE_ERR_INVALID_ARG, "%s is NULL", #p);                            \
    if (!aligned(p)) return fail(MOE_ERR_INVALID_ARG, "%s is not 16-byte aligned", #p);      \
  } while (0)

// --------------------------------------------------------------------------
// workspace layout (one layout serves every entry point)
// --------------------------------------------------------------------------
struct Layout {
  size_t logits, ids, w, ccount, cbase, offsets, rows, inv, tiles, tcount, xq, xs, xst, h, hq, hs, hsh,
      hqsh, hssh, y, ysh, u, part, total;
};

FfnArgs ffn_shape(const moe_config_t* c, int64_t T);

Layout layout(const moe_config_t* c, int64_t T) {
  const int64_t E = c->n_routed_experts, k = c->num_experts_per_tok, H = c->hidden_size;
  const int64_t F = c->moe_intermediate_size, Fs = shared_F(c);
  const int64_t nchunk = (T + kPermChunk - 1) / kPermChunk;
  // SwiGLU output element: act dtype, or fp32 ahead of its fp8 re-quantisation
  const int64_t hsz = fp8(c) ? 4 : act_size(c->act_dtype);
  const int64_t asz = act_size(c->act_dtype);
  Layout L{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += (bytes + 255) & ~size_t(255);
    return o;
  };
  L.logits = take(router_kparts(T, static_cast<int>(E), static_cast<int>(H), c->act_dtype == MOE_BF16) * T * E * 4);
  L.ids = take(T * k * 4);
  L.w = take(T * k * 4);
  L.ccount = take(nchunk * E * 4);
  L.cbase = take(nchunk * E * 4);
  L.offsets = take((E + 1) * 4);
  L.rows = take((T * k + T) * 4);
  L.inv = take(T * k * 4);
  L.tiles = take(max_tiles(T, k, E, true, 16) * sizeof(Tile));
  L.tcount = take(4);
  L.xq = take(fp8(c) ? T * H : 0);
  L.xs = take(fp8(c) ? T * (H / 128) * 4 : 0);
  L.xst = take(fp8(c) ? (T * k + T) * (H / 128) * 4 : 0);
  L.h = take(T * k * F * hsz);
  L.hq = take(fp8(c) ? T * k * F : 0);
  L.hs = take(fp8(c) ? T * k * (F / 128) * 4 : 0);
  L.hsh = take(T * Fs * hsz);
  L.hqsh = take(fp8(c) ? T * Fs : 0);
  L.hssh = take(fp8(c) ? T * (Fs / 128) * 4 : 0);
  L.y = take(T * k * H * asz);
  L.ysh = take(T * H * asz);
  L.u = take(T * H * asz);
  {
    const FfnArgs f = ffn_shape(c, T);
    L.part = take(ffn_plan(f, c->weight_dtype, c->act_dtype).part_bytes(T, f.k, f.H, f.F, f.Fs));
  }
  L.total = off;
  return L;
}

template <typename P>
P* at(void* ws, size_t off) {
  return reinterpret_cast<P*>(static_cast<char*>(ws) + off);
}

moe_status_t check_ws(const moe_config_t* c, int64_t T, void* ws, size_t ws_bytes) {
  const size_t need = layout(c, T).total;
  if (!ws) return fail(MOE_ERR_INVALID_ARG, "ws is NULL");
  if (reinterpret_cast<uintptr_t>(ws) & 255u) return fail(MOE_ERR_INVALID_ARG, "ws is not 256-byte aligned");
  if (ws_bytes < need)
    return fail(MOE_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, need);
  return MOE_OK;
}

moe_status_t check_weights(const moe_config_t* c, const moe_weights_t* w) {
  if (!w) return fail(MOE_ERR_INVALID_ARG, "weights is NULL");
  NEED(w->w_gate);
  NEED(w->w_up);
  NEED(w->w_down);
  if (fp8(c)) {
    NEED(w->s_gate);
    NEED(w->s_up);
    NEED(w->s_down);
  }
  if (c->n_shared_experts > 0) {
    NEED(w->sh_gate);
    NEED(w->sh_up);
    NEED(w->sh_down);
    if (fp8(c)) {
      NEED(w->sh_s_gate);
      NEED(w->sh_s_up);
      NEED(w->sh_s_down);
    }
  }
  return MOE_OK;
}

#define TRY(expr)                         \
  do {                                    \
    moe_status_t s_ = (expr);             \
    if (s_ != MOE_OK) return s_;          \
  } while (0)

RouterArgs router_args(const moe_config_t* c, const void* x, const void* rw, const float* b,
                       int64_t T, float* logits, int32_t* ids, float* w) {
  RouterArgs a{};
  a.x = x;
  a.wr = rw;
  a.bias = b;
  a.T = static_cast<int>(T);
  a.E = c->n_routed_experts;
  a.H = c->hidden_size;
  a.k = c->num_experts_per_tok;
  a.n_group = c->n_group;
  a.topk_group = c->topk_group;
  a.norm = c->norm_topk_prob ? 1 : 0;
  a.scale = c->routed_scaling_factor;
  a.bf16 = c->act_dtype == MOE_BF16;
  a.logits = logits;
  a.ids = ids;
  a.w = w;
  return a;
}

// `quant_x`: (fp8 weights) the top-k launch also writes x's e4m3 codes and
// scales into the workspace
moe_status_t run_route(const moe_config_t* c, const void* x, const void* rw, const float* b,
                       int64_t T, int32_t* ids, float* w, void* ws, hipStream_t st, bool quant_x = false) {
  const Layout L = layout(c, T);
  RouterArgs a = router_args(c, x, rw, b, T, at<float>(ws, L.logits), ids, w);
  if (quant_x) {
    a.xq_codes = at<uint8_t>(ws, L.xq);
    a.xq_scales = at<float>(ws, L.xs);
  }
  MOE_LAUNCH(MOE_KID_ROUTER_LOGITS, launch_router(a, st));
  MOE_LAUNCH(MOE_KID_ROUTER_TOPK, launch_topk(a, st));
  return MOE_OK;
}

// `ft` (nullable): FFN arguments whose plan is already set (ffn_prepare); the
// single-block grouping of small batches then also writes their work list and
// `*tiles_built` says so
moe_status_t run_permute(const moe_config_t* c, const int32_t* ids, int64_t T, int32_t* offsets,
                         int32_t* sorted, int32_t* inv, bool tail, void* ws, hipStream_t st,
                         const FfnArgs* ft = nullptr, bool* tiles_built = nullptr) {
  const Layout L = layout(c, T);
  PermArgs p{};
  p.ids = ids;
  p.T = static_cast<int>(T);
  p.k = c->num_experts_per_tok;
  p.E = c->n_routed_experts;
  p.chunk_counts = at<int32_t>(ws, L.ccount);
  p.chunk_base = at<int32_t>(ws, L.cbase);
  p.offsets = offsets;
  p.sorted = sorted;
  p.inv = inv;
  p.identity_tail = tail;
  if (ft) {
    p.tiles = const_cast<Tile*>(ft->tiles);
    p.tile_count = const_cast<int32_t*>(ft->tile_count);
    p.bm = ft->bm;
    p.shared = ft->Fs > 0;
    p.cap = ft->tile_bound;
  }
  // the grouping kernels are timed as one unit
  MOE_LAUNCH(MOE_KID_PERMUTE, launch_permute(p, st, tiles_built));
  return MOE_OK;
}

// the plan and work-list fields of the FFN arguments
moe_status_t ffn_prepare(const moe_config_t* c, FfnArgs& f, int64_t T, void* ws) {
  const Layout L = layout(c, T);
  const FfnPlan plan = ffn_plan(f, c->weight_dtype, c->act_dtype);
  const int bm = plan.bm;
  f.bm = bm;
  f.kind = plan.kind;
  f.ks_gu = plan.ks_gu;
  f.ks_dn = plan.ks_dn;
  f.w_once = plan.w_once;
  f.part = at<float>(ws, L.part);
  f.tiles = at<Tile>(ws, L.tiles);
  f.tile_count = at<int32_t>(ws, L.tcount);
  f.tile_bound = max_tiles(T, f.k, f.E, f.Fs > 0, bm);
  if (f.tile_bound > 65535) return fail(MOE_ERR_UNSUPPORTED, "too many tiles (%lld) for one launch", (long long)f.tile_bound);
  return MOE_OK;
}

// gate_up + down over a work list built from `offsets` (`tiles_ready`: the
// list is already built, ffn_prepare already ran)
moe_status_t run_ffn(const moe_config_t* c, const moe_weights_t* w, FfnArgs& f, int64_t T,
                     void* ws, hipStream_t st, bool tiles_ready = false) {
  if (!tiles_ready) TRY(ffn_prepare(c, f, T, ws));
  f.w_gate = w->w_gate;
  f.w_up = w->w_up;
  f.w_down = w->w_down;
  f.s_gate = w->s_gate;
  f.s_up = w->s_up;
  f.s_down = w->s_down;
  f.sh_gate = w->sh_gate;
  f.sh_up = w->sh_up;
  f.sh_down = w->sh_down;
  f.sh_s_gate = w->sh_s_gate;
  f.sh_s_up = w->sh_s_up;
  f.sh_s_down = w->sh_s_down;
  f.xrs_t = fp8(c) ? at<float>(ws, layout(c, T).xst) : nullptr;
  TileArgs ta{};
  ta.offsets = f.offsets;
  ta.T = f.T;
  ta.k = f.k;
  ta.E = f.E;
  ta.bm = f.bm;
  ta.shared = f.Fs > 0;
  ta.cap = f.tile_bound;
  ta.tiles = const_cast<Tile*>(f.tiles);
  ta.tile_count = const_cast<int32_t*>(f.tile_count);
  if (!tiles_ready) MOE_LAUNCH(MOE_KID_TILES, launch_build_tiles(ta, st));
  MOE_LAUNCH(MOE_KID_GATE_UP, launch_gate_up(f, c->act_dtype, c->weight_dtype, st));
  MOE_LAUNCH(MOE_KID_DOWN, launch_down(f, c->act_dtype, c->weight_dtype, st));
  return MOE_OK;
}

// the shape fields of the FFN arguments (what ffn_plan reads)
FfnArgs ffn_shape(const moe_config_t* c, int64_t T) {
  FfnArgs f{};
  f.T = static_cast<int>(T);
  f.k = c->num_experts_per_tok;
  f.E = c->n_routed_experts;
  f.H = c->hidden_size;
  f.F = c->moe_intermediate_size;
  f.Fs = shared_F(c);
  return f;
}

FfnArgs ffn_args(const moe_config_t* c, int64_t T, void* ws) {
  const Layout L = layout(c, T);
  FfnArgs f = ffn_shape(c, T);
  f.h = at<void>(ws, L.h);
  f.h_sh = at<void>(ws, L.hsh);
  f.hq = at<void>(ws, L.hq);
  f.hq_sh = at<void>(ws, L.hqsh);
  f.h_scales = at<float>(ws, L.hs);
  f.h_sh_scales = at<float>(ws, L.hssh);
  return f;
}

// the layer's tensor arguments (after check_cfg, for T > 0)
moe_status_t check_layer_ptrs(const moe_config_t* cfg, const moe_weights_t* w, const void* x,
                              const void* router_w, const float* router_bias, void* out,
                              int32_t* topk_ids_out, float* topk_weights_out) {
  TRY(check_weights(cfg, w));
  NEED(x);
  NEED(router_w);
  NEED(router_bias);
  NEED(out);
  if (topk_ids_out && !aligned(topk_ids_out)) return fail(MOE_ERR_INVALID_ARG, "topk_ids_out is not 16-byte aligned");
  if (topk_weights_out && !aligned(topk_weights_out)) return fail(MOE_ERR_INVALID_ARG, "topk_weights_out is not 16-byte aligned");
  return MOE_OK;
}

moe_status_t check_layer_args(const moe_config_t* cfg, const moe_weights_t* w, const void* x,
                              const void* router_w, const float* router_bias, int64_t T, void* out,
                              int32_t* topk_ids_out, float* topk_weights_out, void* ws, size_t ws_bytes) {
  TRY(check_cfg(cfg));
  TRY(check_T(T));
  if (T == 0) return MOE_OK;
  TRY(check_layer_ptrs(cfg, w, x, router_w, router_bias, out, topk_ids_out, topk_weights_out));
  return check_ws(cfg, T, ws, ws_bytes);
}

// route -> group -> expert FFNs -> combine on layer input x; `resid` (nullable)
// is added in the combine; `x_quantised`: the fp8 codes of x are already in
// the workspace
moe_status_t run_layer(const moe_config_t* cfg, const moe_weights_t* w, const void* x, const void* router_w,
                       const float* router_bias, int64_t T, void* out, int32_t* topk_ids_out,
                       float* topk_weights_out, void* ws, hipStream_t st, const void* resid,
                       bool x_quantised) {
  const Layout L = layout(cfg, T);
  int32_t* ids = topk_ids_out ? topk_ids_out : at<int32_t>(ws, L.ids);
  float* wts = topk_weights_out ? topk_weights_out : at<float>(ws, L.w);
  // fp8 weights: the top-k launch quantises x as well (unless the norm pass did)
  TRY(run_route(cfg, x, router_w, router_bias, T, ids, wts, ws, st, fp8(cfg) && !x_quantised));
  int32_t* offsets = at<int32_t>(ws, L.offsets);
  int32_t* rows = at<int32_t>(ws, L.rows);
  int32_t* inv = at<int32_t>(ws, L.inv);
  FfnArgs f = ffn_args(cfg, T, ws);
  TRY(ffn_prepare(cfg, f, T, ws));
  bool tiles_ready = false;
  TRY(run_permute(cfg, ids, T, offsets, rows, inv, true, ws, st, &f, &tiles_ready));
  f.offsets = offsets;
  f.xr = x;
  f.xr_rows = rows;
  f.xs = x;
  f.y = at<void>(ws, L.y);
  f.y_sh = at<void>(ws, L.ysh);
  if (fp8(cfg)) {
    uint8_t* xq = at<uint8_t>(ws, L.xq);
    float* xs = at<float>(ws, L.xs);
    f.xr = xq;
    f.xr_scales = xs;
    f.xs = xq;
    f.xs_scales = xs;
  }
  TRY(run_ffn(cfg, w, f, T, ws, st, tiles_ready));
  CombineArgs a{f.y, cfg->n_shared_experts > 0 ? f.y_sh : nullptr, wts, inv, static_cast<int>(T),
                cfg->num_experts_per_tok, cfg->hidden_size, out, resid};
  MOE_LAUNCH(MOE_KID_COMBINE, launch_combine(a, cfg->act_dtype == MOE_BF16, st));
  return MOE_OK;
}

// ---------------------------------------------------------------------------
// The fixed scratch of moe_layer_forward_static: one array per GPU (each
// device that loads the library holds its own copy until the process ends),
// standing in for the caller's workspace.  In host code `scratch` is a
// host-side stand-in, never a device address: its device address is taken
// once per device with hipGetSymbolAddress (with that device current) and
// only that pointer is passed on.  Nothing in the workspace needs to start
// at zero (every piece is written before it is read), so it is not cleared.
constexpr size_t kStaticScratch = MOE_STATIC_SCRATCH_BYTES;
__device__ __attribute__((aligned(256))) unsigned char scratch[kStaticScratch];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices] = {};

// device address of the current device's scratch array (looked up once)
moe_status_t static_scratch(void** ptr) {
  int dev = -1;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(MOE_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(MOE_ERR_UNSUPPORTED, "device %d beyond %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    const hipError_t s = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (s != hipSuccess || !p)
      return fail(MOE_ERR_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(s));
    g_scratch[dev] = p;
  }
  *ptr = g_scratch[dev];
  return MOE_OK;
}

}  // namespace

// ---------------------------------------------------------------------------
extern "C" {

int moe_abi_version(void) { return MOE_ABI_VERSION; }

const char* moe_status_string(moe_status_t s) {
  switch (s) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE";
    case MOE_ERR_HIP: return "MOE_ERR_HIP";
  }
  return "MOE_ERR_UNKNOWN";
}

const char* moe_last_error(void) { return g_err.c_str(); }

size_t moe_workspace_size(const moe_config_t* cfg, int64_t T) {
  if (check_cfg(cfg, false) != MOE_OK || T < 0 || T > kMaxTokens) return 0;
  return layout(cfg, T).total;
}

moe_status_t moe_workspace_region(const moe_config_t* cfg, int64_t T, int32_t region, size_t* offset,
                                  size_t* bytes) {
  g_err.clear();
  TRY(check_cfg(cfg, false));
  TRY(check_T(T));
  if (!offset || !bytes) return fail(MOE_ERR_INVALID_ARG, "offset and bytes must not be NULL");
  if (region < 0 || region >= MOE_WS_COUNT) return fail(MOE_ERR_INVALID_ARG, "region %d out of range", region);
  const Layout L = layout(cfg, T);
  const int64_t k = cfg->num_experts_per_tok, H = cfg->hidden_size, F = cfg->moe_intermediate_size;
  const int64_t Fs = shared_F(cfg), asz = act_size(cfg->act_dtype);
  const int64_t hsz = fp8(cfg) ? 4 : asz;
  const bool q = fp8(cfg);
  size_t o = 0;
  int64_t n = 0;
  switch (region) {
    case MOE_WS_H: o = L.h; n = T * k * F * hsz; break;
    case MOE_WS_H_CODES: o = L.hq; n = q ? T * k * F : 0; break;
    case MOE_WS_H_SCALES: o = L.hs; n = q ? T * k * (F / 128) * 4 : 0; break;
    case MOE_WS_H_SHARED: o = L.hsh; n = T * Fs * hsz; break;
    case MOE_WS_H_SHARED_CODES: o = L.hqsh; n = q ? T * Fs : 0; break;
    case MOE_WS_H_SHARED_SCALES: o = L.hssh; n = q ? T * (Fs / 128) * 4 : 0; break;
    case MOE_WS_Y: o = L.y; n = T * k * H * asz; break;
    case MOE_WS_Y_SHARED: o = L.ysh; n = T * H * asz; break;
  }
  *offset = o;
  *bytes = static_cast<size_t>(n);
  return MOE_OK;
}

moe_status_t moe_profile_arm(int32_t kid, void* start, void* stop) {
  if (kid < 0 || kid >= MOE_KID_COUNT) return fail(MOE_ERR_INVALID_ARG, "kernel id %d out of range", kid);
  if ((start == nullptr) != (stop == nullptr)) return fail(MOE_ERR_INVALID_ARG, "arm both events or neither");
  g_ev[kid][0] = static_cast<hipEvent_t>(start);
  g_ev[kid][1] = static_cast<hipEvent_t>(stop);
  return MOE_OK;
}

moe_status_t moe_route(const moe_config_t* cfg, const void* x, const void* router_w,
                       const float* router_bias, int64_t T, int32_t* topk_ids, float* topk_weights,
                       void* ws, size_t ws_bytes, void* stream) {
  g_err.clear();
  TRY(check_cfg(cfg));
  TRY(check_T(T));
  if (T == 0) return MOE_OK;
  NEED(x);
  NEED(router_w);
  NEED(router_bias);
  NEED(topk_ids);
  NEED(topk_weights);
  TRY(check_ws(cfg, T, ws, ws_bytes));
  (void)hipGetLastError();
  return run_route(cfg, x, router_w, router_bias, T, topk_ids, topk_weights, ws,
                   static_cast<hipStream_t>(stream));
}

moe_status_t moe_permute(const moe_config_t* cfg, const void* x, const int32_t* topk_ids, int64_t T,
                         int32_t* expert_offsets, int32_t* sorted_token_ids, int32_t* inv_perm,
                         void* x_perm, float* x_perm_scales, void* ws, size_t ws_bytes,
                         void* stream) {
  g_err.clear();
  TRY(check_cfg(cfg));
  TRY(check_T(T));
  if (T == 0) return MOE_OK;
  NEED(topk_ids);
  NEED(expert_offsets);
  NEED(sorted_token_ids);
  NEED(inv_perm);
  if (x_perm) {
    NEED(x);
    if (fp8(cfg)) NEED(x_perm_scales);
  }
  TRY(check_ws(cfg, T, ws, ws_bytes));
  (void)hipGetLastError();
  hipStream_t st = static_cast<hipStream_t>(stream);
  TRY(run_permute(cfg, topk_ids, T, expert_offsets, sorted_token_ids, inv_perm, false, ws, st));
  if (!x_perm) return MOE_OK;
  const int64_t TK = T * cfg->num_experts_per_tok, H = cfg->hidden_size;
  if (fp8(cfg)) {
    const Layout L = layout(cfg, T);
    uint8_t* xq = at<uint8_t>(ws, L.xq);
    float* xs = at<float>(ws, L.xs);
    MOE_LAUNCH(MOE_KID_ACT_QUANT, launch_act_quant(static_cast<const uint16_t*>(x), T, H, xq, xs, st));
    const int32_t* n_rows = expert_offsets + cfg->n_routed_experts;
    MOE_LAUNCH(MOE_KID_GATHER, launch_gather(xq, sorted_token_ids, TK, n_rows, H, x_perm, st));
    MOE_LAUNCH(MOE_KID_GATHER, launch_gather(xs, sorted_token_ids, TK, n_rows, (H / 128) * 4, x_perm_scales, st));
  } else {
    MOE_LAUNCH(MOE_KID_GATHER, launch_gather(x, sorted_token_ids, TK, expert_offsets + cfg->n_routed_experts,
                                             H * act_size(cfg->act_dtype), x_perm, st));
  }
  return MOE_OK;
}

moe_status_t moe_expert_ffn(const moe_config_t* cfg, const moe_weights_t* w, const void* x,
                            const void* x_perm, const float* x_perm_scales,
                            const int32_t* expert_offsets, int64_t T, void* y_perm, void* y_shared,
                            void* ws, size_t ws_bytes, void* stream) {
  g_err.clear();
  TRY(check_cfg(cfg, false));
  TRY(check_T(T));
  if (T == 0) return MOE_OK;
  TRY(check_weights(cfg, w));
  NEED(x_perm);
  NEED(expert_offsets);
  NEED(y_perm);
  if (fp8(cfg)) NEED(x_perm_scales);
  if (cfg->n_shared_experts > 0) {
    NEED(x);
    NEED(y_shared);
  }
  TRY(check_ws(cfg, T, ws, ws_bytes));
  (void)hipGetLastError();
  hipStream_t st = static_cast<hipStream_t>(stream);
  FfnArgs f = ffn_args(cfg, T, ws);
  f.offsets = expert_offsets;
  f.xr = x_perm;
  f.xr_scales = x_perm_scales;
  f.xr_rows = nullptr;
  f.xs = x;
  f.y = y_perm;
  f.y_sh = y_shared;
  if (fp8(cfg) && cfg->n_shared_experts > 0) {
    const Layout L = layout(cfg, T);
    MOE_LAUNCH(MOE_KID_ACT_QUANT, launch_act_quant(static_cast<const uint16_t*>(x), T, cfg->hidden_size,
                                                   at<uint8_t>(ws, L.xq), at<float>(ws, L.xs), st));
    f.xs = at<void>(ws, L.xq);
    f.xs_scales = at<float>(ws, L.xs);
  }
  return run_ffn(cfg, w, f, T, ws, st);
}

moe_status_t moe_combine(const moe_config_t* cfg, const void* y_perm, const void* y_shared,
                         const float* topk_weights, const int32_t* inv_perm, int64_t T, void* out,
                         void* stream) {
  g_err.clear();
  TRY(check_cfg(cfg));
  TRY(check_T(T));
  if (T == 0) return MOE_OK;
  NEED(y_perm);
  NEED(topk_weights);
  NEED(inv_perm);
  NEED(out);
  if (cfg->n_shared_experts > 0) NEED(y_shared);
  (void)hipGetLastError();
  hipStream_t st = static_cast<hipStream_t>(stream);
  CombineArgs a{y_perm, cfg->n_shared_experts > 0 ? y_shared : nullptr, topk_weights, inv_perm,
                static_cast<int>(T), cfg->num_experts_per_tok, cfg->hidden_size, out};
  MOE_LAUNCH(MOE_KID_COMBINE, launch_combine(a, cfg->act_dtype == MOE_BF16, st));
  return MOE_OK;
}

moe_status_t moe_layer_forward(const moe_config_t* cfg, const moe_weights_t* w, const void* x,
                               const void* router_w, const float* router_bias, int64_t T, void* out,
                               int32_t* topk_ids_out, float* topk_weights_out, void* ws,
                               size_t ws_bytes, void* stream) {
  g_err.clear();
  TRY(check_layer_args(cfg, w, x, router_w, router_bias, T, out, topk_ids_out, topk_weights_out, ws, ws_bytes));
  if (T == 0) return MOE_OK;
  (void)hipGetLastError();
  return run_layer(cfg, w, x, router_w, router_bias, T, out, topk_ids_out, topk_weights_out, ws,
                   static_cast<hipStream_t>(stream), nullptr, false);
}

moe_status_t moe_layer_forward_static(const moe_config_t* cfg, const moe_weights_t* w, const void* x,
                                      const void* router_w, const float* router_bias, int64_t T, void* out,
                                      int32_t* topk_ids_out, float* topk_weights_out, void* stream) {
  g_err.clear();
  TRY(check_cfg(cfg));
  TRY(check_T(T));
  if (T == 0) return MOE_OK;
  const size_t need = layout(cfg, T).total;
  if (need > kStaticScratch)
    return fail(MOE_ERR_WORKSPACE, "%lld tokens need %zu bytes of workspace, more than the %zu of the fixed scratch",
                (long long)T, need, kStaticScratch);
  TRY(check_layer_ptrs(cfg, w, x, router_w, router_bias, out, topk_ids_out, topk_weights_out));
  // (every argument checked before the first HIP call)
  void* ws = nullptr;
  TRY(static_scratch(&ws));
  (void)hipGetLastError();
  return run_layer(cfg, w, x, router_w, router_bias, T, out, topk_ids_out, topk_weights_out, ws,
                   static_cast<hipStream_t>(stream), nullptr, false);
}

moe_status_t moe_block_forward(const moe_config_t* cfg, const moe_weights_t* w, const void* x,
                               const void* norm_weight, float rms_norm_eps, const void* router_w,
                               const float* router_bias, int64_t T, void* out, int32_t* topk_ids_out,
                               float* topk_weights_out, void* ws, size_t ws_bytes, void* stream) {
  g_err.clear();
  TRY(check_layer_args(cfg, w, x, router_w, router_bias, T, out, topk_ids_out, topk_weights_out, ws, ws_bytes));
  if (T == 0) return MOE_OK;
  NEED(norm_weight);
  if (!(rms_norm_eps >= 0.0f) || !(rms_norm_eps < 1.0f))
    return fail(MOE_ERR_INVALID_ARG, "rms_norm_eps %g not in [0, 1)", static_cast<double>(rms_norm_eps));
  (void)hipGetLastError();
  hipStream_t st = static_cast<hipStream_t>(stream);
  const Layout L = layout(cfg, T);
  void* u = at<void>(ws, L.u);
  // fp8 weights: the norm pass also writes the e4m3 codes of u
  uint8_t* codes = fp8(cfg) ? at<uint8_t>(ws, L.xq) : nullptr;
  float* scales = fp8(cfg) ? at<float>(ws, L.xs) : nullptr;
  MOE_LAUNCH(MOE_KID_NORM, launch_rmsnorm(x, norm_weight, static_cast<double>(rms_norm_eps), T, cfg->hidden_size,
                                          cfg->act_dtype == MOE_BF16, u, codes, scales, st));
  return run_layer(cfg, w, u, router_w, router_bias, T, out, topk_ids_out, topk_weights_out, ws, st, x,
                   fp8(cfg));
}

}  // extern "C"
