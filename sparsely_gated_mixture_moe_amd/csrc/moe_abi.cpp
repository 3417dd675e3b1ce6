// The C ABI of include/moe.h: argument validation, workspace layout and the
// order of kernel launches. Validation runs before any HIP call, so an invalid
// call launches nothing and writes nothing.
#include "../../include/moe.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>
#include <type_traits>

#include "moe_internal.h"

namespace {

thread_local std::string g_last_error;

moe_status fail(moe_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

moe_status ok() {
  g_last_error.clear();
  return MOE_OK;
}

constexpr size_t kAlign = 256;
size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

size_t dt_size(moe_dtype t) { return t == MOE_BF16 ? 2 : 4; }
moe::Dt to_dt(moe_dtype t) { return t == MOE_BF16 ? moe::kBF16 : moe::kF32; }

moe_status check_dims(const moe_dims* d) {
  if (!d) return fail(MOE_ERR_INVALID, "dims is NULL");
  if (d->tokens < 0) return fail(MOE_ERR_INVALID, "tokens = %lld < 0", (long long)d->tokens);
  if (d->n_experts < 1 || d->n_experts > 32768)
    return fail(MOE_ERR_INVALID, "n_experts = %d outside [1, 32768]", d->n_experts);
  if (d->k < 1 || d->k > d->n_experts)
    return fail(MOE_ERR_INVALID, "k = %d outside [1, n_experts = %d]", d->k, d->n_experts);
  if (d->k > 8) return fail(MOE_ERR_UNSUPPORTED, "k = %d > 8", d->k);
  if (d->capacity < 0) return fail(MOE_ERR_INVALID, "capacity = %d < 0", d->capacity);
  if (d->expert_layout != 0 && d->expert_layout != 1)
    return fail(MOE_ERR_INVALID, "expert_layout = %d is neither 0 nor 1", d->expert_layout);
  if (d->tokens * (int64_t)d->k > (int64_t)0x7FFFFFFE)
    return fail(MOE_ERR_INVALID, "tokens * k = %lld does not fit int32 indices",
                (long long)(d->tokens * d->k));
  if (d->d_model < 1 || d->d_hidden < 1)
    return fail(MOE_ERR_INVALID, "d_model = %d, d_hidden = %d must be positive", d->d_model,
                d->d_hidden);
  if (d->d_model % 64 != 0 || d->d_model > 512)
    return fail(MOE_ERR_UNSUPPORTED, "d_model = %d: supported values are 64, 128, 256, 512",
                d->d_model);
  if (d->d_model != 64 && d->d_model != 128 && d->d_model != 256 && d->d_model != 512)
    return fail(MOE_ERR_UNSUPPORTED, "d_model = %d: supported values are 64, 128, 256, 512",
                d->d_model);
  if (d->d_hidden % 128 != 0)
    return fail(MOE_ERR_UNSUPPORTED, "d_hidden = %d is not a multiple of 128", d->d_hidden);
  for (moe_dtype t : {d->act_dtype, d->expert_dtype, d->gate_dtype})
    if (t != MOE_F32 && t != MOE_BF16) return fail(MOE_ERR_INVALID, "unknown dtype %d", (int)t);
  if (d->expert_dtype != d->act_dtype)
    return fail(MOE_ERR_UNSUPPORTED, "expert_dtype must equal act_dtype");
  if (d->gate_dtype == MOE_BF16 && d->act_dtype != MOE_BF16)
    return fail(MOE_ERR_UNSUPPORTED, "bf16 gate weights need bf16 activations");
  return MOE_OK;
}

moe_status check_opts(const moe_gate_opts* o) {
  if (!o) return fail(MOE_ERR_INVALID, "opts is NULL");
  if (o->train != 0 && o->train != 1) return fail(MOE_ERR_INVALID, "train must be 0 or 1");
  if (!std::isfinite(o->noise_floor) || o->noise_floor < 0.f)
    return fail(MOE_ERR_INVALID, "noise_floor must be finite and >= 0");
  if (!std::isfinite(o->w_importance) || !std::isfinite(o->w_load))
    return fail(MOE_ERR_INVALID, "loss weights must be finite");
  if (o->gate_order != 0 && o->gate_order != 1)
    return fail(MOE_ERR_INVALID, "gate_order must be 0 or 1");
  return MOE_OK;
}

#define REQ(ptr, align)                                                                  \
  do {                                                                                   \
    if (!(ptr)) return fail(MOE_ERR_INVALID, "%s is NULL", #ptr);                        \
    if (!aligned((ptr), (align)))                                                        \
      return fail(MOE_ERR_INVALID, "%s is not %d-byte aligned", #ptr, (int)(align));     \
  } while (0)

// A required tensor of `count` elements: may be NULL only when it is empty.
#define REQN(ptr, align, count)                                                          \
  do {                                                                                   \
    if ((count) > 0) REQ(ptr, align);                                                    \
    else OPT(ptr, align);                                                                \
  } while (0)

#define OPT(ptr, align)                                                                  \
  do {                                                                                   \
    if ((ptr) && !aligned((ptr), (align)))                                               \
      return fail(MOE_ERR_INVALID, "%s is not %d-byte aligned", #ptr, (int)(align));     \
  } while (0)

// Workspace regions. Each call uses a prefix-free subset; moe_forward uses all.
struct Layout {
  size_t topk_idx, topk_gate, thresh, counts, offsets, perm_token, perm_gate, slot_pos,
      importance, blockcnt, ffn_blocks, expert_out, load_partial, load_corr, gate_cand, total;
  size_t route_bytes, ffn_bytes, aux_bytes, gate_bytes;  // standalone needs (from offset 0)
};

Layout layout(const moe_dims* d, const moe_gate_opts* o) {
  const int64_t B = d->tokens, k = d->k, n = d->n_experts;
  const int64_t pairs = B * k;
  Layout L{};
  size_t at = 0;
  auto take = [&](size_t bytes) {
    const size_t off = at;
    at += align_up(bytes);
    return off;
  };
  // standalone requirements (each placed at offset 0)
  L.route_bytes = align_up((size_t)n * moe::route_blocks(B) * sizeof(int32_t));
  L.ffn_bytes = align_up(moe::ffn_plan_bytes(pairs, (int)n, d->d_model, d->d_hidden, to_dt(d->act_dtype)));
  // the Load pass: per-block partial sums, then the selected pairs' corrections
  L.aux_bytes = (o && o->train) ? align_up((size_t)moe::gate_blocks(B) * n * sizeof(float)) +
                                      align_up(moe::corr_bytes(pairs, (int)n))
                                : 0;
  // a small batch's split selection: each expert range's candidates
  auto cand = [&](int train) {
    moe::GateLaunch g{};
    g.tokens = B;
    g.d = d->d_model;
    g.n = (int)n;
    g.k = (int)k;
    g.x_dt = to_dt(d->act_dtype);
    g.w_dt = to_dt(d->gate_dtype);
    g.train = train;
    return moe::gate_cand_bytes(g);
  };
  L.gate_bytes = align_up(o ? cand(o->train) : std::max(cand(0), cand(1)));
  // moe_forward
  L.topk_idx = take(pairs * sizeof(int32_t));
  L.topk_gate = take(pairs * sizeof(float));
  L.thresh = take(B * 2 * sizeof(float));
  L.counts = take(n * sizeof(int32_t));
  L.offsets = take((n + 1) * sizeof(int32_t));
  L.perm_token = take(pairs * sizeof(int32_t));
  L.perm_gate = take(pairs * sizeof(float));
  L.slot_pos = take(pairs * sizeof(int32_t));
  L.importance = take(n * sizeof(float));
  L.blockcnt = take(L.route_bytes);
  L.ffn_blocks = take(L.ffn_bytes);
  L.expert_out = take((size_t)pairs * d->d_model * dt_size(d->act_dtype));
  L.load_partial = take(L.aux_bytes);
  L.load_corr = L.load_partial + (L.aux_bytes ? align_up((size_t)moe::gate_blocks(B) * n *
                                                         sizeof(float))
                                              : 0);
  L.gate_cand = take(L.gate_bytes);
  L.total = at;
  return L;
}

moe_status check_ws(void* ws, size_t ws_bytes, size_t need) {
  if (need == 0) return MOE_OK;
  if (!ws) return fail(MOE_ERR_WORKSPACE, "workspace is NULL, %zu bytes needed", need);
  if (!aligned(ws, kAlign)) return fail(MOE_ERR_INVALID, "workspace is not 256-byte aligned");
  if (ws_bytes < need)
    return fail(MOE_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", ws_bytes, need);
  return MOE_OK;
}

moe_status device_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(MOE_ERR_DEVICE, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

template <typename T>
T* at(void* ws, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

moe::GateLaunch gate_launch(const moe_dims* d, const moe_gate_opts* o, const void* x,
                            const void* wg, const void* wn, const float* bias, const float* eps) {
  moe::GateLaunch g;
  g.x = x;
  g.w_gate = wg;
  g.w_noise = wn;
  g.bias = bias;
  g.eps = o->train ? eps : nullptr;
  g.tokens = d->tokens;
  g.d = d->d_model;
  g.n = d->n_experts;
  g.k = d->k;
  g.x_dt = to_dt(d->act_dtype);
  g.w_dt = to_dt(d->gate_dtype);
  g.train = o->train;
  g.noise_floor = o->noise_floor;
  g.gate_order = o->gate_order;
  return g;
}

moe_status check_gate_args(const moe_dims* d, const moe_gate_opts* o, const void* x,
                           const void* wg, const void* wn, const float* bias, const float* eps,
                           bool need_eps) {
  REQN(x, 16, d->tokens);
  REQ(wg, 16);
  if (o->train) REQ(wn, 16);
  else OPT(wn, 16);
  // the gate kernels copy biases and noise rows to LDS 16 bytes at a time
  OPT(bias, 16);
  if (o->train && need_eps) REQN(eps, 16, d->tokens);
  if (!moe::gate_supported(d->d_model, to_dt(d->act_dtype), to_dt(d->gate_dtype), d->k))
    return fail(MOE_ERR_UNSUPPORTED, "gate: unsupported shape or dtype combination");
  return MOE_OK;
}

// ---------------------------------------------------------------------------
// Hierarchical layer
// ---------------------------------------------------------------------------

moe_status check_hier_dims(const moe_hier_dims* h) {
  if (!h) return fail(MOE_ERR_INVALID, "dims is NULL");
  if (h->expert_layout != 0 && h->expert_layout != 1)
    return fail(MOE_ERR_INVALID, "expert_layout = %d is neither 0 nor 1", h->expert_layout);
  if (h->groups < 1 || h->group_experts < 1)
    return fail(MOE_ERR_INVALID, "groups = %d and group_experts = %d must be positive",
                h->groups, h->group_experts);
  if ((int64_t)h->groups * h->group_experts > 32768)
    return fail(MOE_ERR_INVALID, "groups * group_experts = %lld > 32768",
                (long long)h->groups * h->group_experts);
  if (h->k1 < 1 || h->k1 > h->groups)
    return fail(MOE_ERR_INVALID, "k1 = %d outside [1, groups = %d]", h->k1, h->groups);
  if (h->k2 < 1 || h->k2 > h->group_experts)
    return fail(MOE_ERR_INVALID, "k2 = %d outside [1, group_experts = %d]", h->k2,
                h->group_experts);
  if (h->k1 * h->k2 > 8) return fail(MOE_ERR_UNSUPPORTED, "k1 * k2 = %d > 8", h->k1 * h->k2);
  // the leaf layer: the same limits as a flat layer with k = k1 * k2
  moe_dims leaf{h->tokens, h->d_model, h->d_hidden, h->groups * h->group_experts,
                h->k1 * h->k2, h->act_dtype, h->expert_dtype, h->gate_dtype, 0, 0};
  return check_dims(&leaf);
}

struct HierLayout {
  size_t sel1, gate1, thr1, counts1, offsets1, perm_token1, perm_gate1, slot_pos1, perm_slot1,
      imp1, blockcnt1, units, unit_start, sel2, gate2, thr2, topk_idx, topk_gate, counts, offsets,
      perm_token, perm_gate, slot_pos, blockcnt, ffn_blocks, expert_out, load1, partial1, corr1,
      load2, partial2, corr2, total;
  int64_t max_units;
};

moe::GateLaunch hier_gate_launch(const moe_hier_dims* h, const moe_gate_opts* o, int level,
                                 const void* x, const void* wg, const void* wn, const float* eps) {
  moe::GateLaunch g;
  g.x = x;
  g.w_gate = wg;
  g.w_noise = wn;
  g.bias = nullptr;
  g.eps = o->train ? eps : nullptr;
  g.tokens = level == 1 ? h->tokens : h->tokens * h->k1;
  g.d = h->d_model;
  g.n = level == 1 ? h->groups : h->group_experts;
  g.k = level == 1 ? h->k1 : h->k2;
  g.x_dt = to_dt(h->act_dtype);
  g.w_dt = to_dt(h->gate_dtype);
  g.train = o->train;
  g.noise_floor = o->noise_floor;
  return g;
}

HierLayout hier_layout(const moe_hier_dims* h, const moe_gate_opts* o) {
  const int64_t B = h->tokens, a = h->groups, b = h->group_experts, k1 = h->k1;
  const int64_t n = a * b, K = k1 * h->k2;
  const int64_t rows2 = B * k1, pairs = B * K;
  const bool train = o && o->train;
  moe_gate_opts tmp{train ? 1 : 0, 0.01f, 0.f, 0.f};
  const int tile = moe::gate_tile_rows(hier_gate_launch(h, &tmp, 2, nullptr, nullptr, nullptr,
                                                        nullptr));
  HierLayout L{};
  L.max_units = moe::gate_max_units(rows2, (int)a, tile);
  size_t at = 0;
  auto take = [&](size_t bytes) {
    const size_t off = at;
    at += align_up(bytes);
    return off;
  };
  L.sel1 = take(rows2 * sizeof(int32_t));
  L.gate1 = take(rows2 * sizeof(float));
  L.thr1 = take(B * 2 * sizeof(float));
  L.counts1 = take(a * sizeof(int32_t));
  L.offsets1 = take((a + 1) * sizeof(int32_t));
  L.perm_token1 = take(rows2 * sizeof(int32_t));
  L.perm_gate1 = take(rows2 * sizeof(float));
  L.slot_pos1 = take(rows2 * sizeof(int32_t));
  L.perm_slot1 = take(rows2 * sizeof(int32_t));
  L.imp1 = take(a * sizeof(float));
  L.blockcnt1 = take((size_t)a * moe::route_blocks(B) * sizeof(int32_t));
  L.units = take((size_t)(1 + 2 * L.max_units) * sizeof(int32_t));
  L.unit_start = take((a + 1) * sizeof(int32_t));
  L.sel2 = take(pairs * sizeof(int32_t));
  L.gate2 = take(pairs * sizeof(float));
  L.thr2 = take(rows2 * 2 * sizeof(float));
  L.topk_idx = take(pairs * sizeof(int32_t));
  L.topk_gate = take(pairs * sizeof(float));
  L.counts = take(n * sizeof(int32_t));
  L.offsets = take((n + 1) * sizeof(int32_t));
  L.perm_token = take(pairs * sizeof(int32_t));
  L.perm_gate = take(pairs * sizeof(float));
  L.slot_pos = take(pairs * sizeof(int32_t));
  L.blockcnt = take((size_t)n * moe::route_blocks(B) * sizeof(int32_t));
  L.ffn_blocks = take(moe::ffn_plan_bytes(pairs, (int)n, h->d_model, h->d_hidden, to_dt(h->act_dtype)));
  L.expert_out = take((size_t)pairs * h->d_model * dt_size(h->act_dtype));
  L.load1 = take(a * sizeof(float));
  L.partial1 = take(train ? (size_t)moe::gate_blocks(B) * a * sizeof(float) : 0);
  L.corr1 = take(moe::corr_bytes(rows2, (int)a));
  L.load2 = take(n * sizeof(float));
  L.partial2 = take(train ? (size_t)L.max_units * b * sizeof(float) : 0);
  L.corr2 = take(moe::corr_bytes(pairs, (int)n));
  L.total = at;
  return L;
}

// Timing events around the expert-FFN kernel of forward calls (moe_ffn_timing).
constexpr int kTimedMax = 1024;
struct FfnTiming {
  bool on = false;
  int dev = -1;
  int used = 0;
  hipEvent_t ev[kTimedMax][2] = {};
};
std::mutex g_timing_mu;
FfnTiming g_timing;

// The next pair of events for a forward call on the current device, or
// nulls when timing is off, on another device or full.
void timing_pair(hipEvent_t* e0, hipEvent_t* e1) {
  *e0 = *e1 = nullptr;
  std::lock_guard<std::mutex> lk(g_timing_mu);
  int dev = -1;
  if (!g_timing.on || hipGetDevice(&dev) != hipSuccess || dev != g_timing.dev ||
      g_timing.used >= kTimedMax)
    return;
  *e0 = g_timing.ev[g_timing.used][0];
  *e1 = g_timing.ev[g_timing.used][1];
  ++g_timing.used;
}

}  // namespace

extern "C" {

int moe_abi_version(void) { return MOE_ABI_VERSION; }

moe_status moe_ffn_timing(int enable) {
  if (enable != 0 && enable != 1) return fail(MOE_ERR_INVALID, "enable = %d is not 0 or 1", enable);
  std::lock_guard<std::mutex> lk(g_timing_mu);
  if (!enable) {
    g_timing.on = false;
    return ok();
  }
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess && dev != g_timing.dev) {  // events belong to the device they were made on
    for (auto& pr : g_timing.ev)
      for (auto& ev : pr)
        if (ev) {
          (void)hipEventDestroy(ev);
          ev = nullptr;
        }
    for (int i = 0; i < kTimedMax && e == hipSuccess; ++i)
      for (int j = 0; j < 2 && e == hipSuccess; ++j) e = hipEventCreate(&g_timing.ev[i][j]);
  }
  if (e != hipSuccess) {
    g_timing.dev = -1;
    g_timing.on = false;
    return device_status(e, "moe_ffn_timing");
  }
  g_timing.dev = dev;
  g_timing.used = 0;
  g_timing.on = true;
  return ok();
}

moe_status moe_ffn_timing_read(int64_t* launches, double* total_ms) {
  if (!launches || !total_ms) return fail(MOE_ERR_INVALID, "NULL output");
  std::lock_guard<std::mutex> lk(g_timing_mu);
  double sum = 0.0;
  for (int i = 0; i < g_timing.used; ++i) {
    hipError_t e = hipEventSynchronize(g_timing.ev[i][1]);
    float ms = 0.f;
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, g_timing.ev[i][0], g_timing.ev[i][1]);
    if (e != hipSuccess) return device_status(e, "moe_ffn_timing_read");
    sum += ms;
  }
  *launches = g_timing.used;
  *total_ms = sum;
  return ok();
}

const char* moe_status_string(int s) {
  switch (s) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID: return "MOE_ERR_INVALID";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE";
    case MOE_ERR_DEVICE: return "MOE_ERR_DEVICE";
    default: return "MOE_ERR_UNKNOWN";
  }
}

const char* moe_last_error(void) { return g_last_error.c_str(); }

size_t moe_workspace_size(const moe_dims* dims, const moe_gate_opts* opts) {
  if (check_dims(dims) != MOE_OK) return 0;
  if (opts && check_opts(opts) != MOE_OK) return 0;
  return layout(dims, opts).total;
}

moe_status moe_gate(const moe_dims* dims, const moe_gate_opts* opts, const void* x,
                    const void* w_gate, const void* w_noise, const float* gate_bias,
                    const float* eps, int32_t* topk_idx, float* topk_gate, float* thresh, void* ws,
                    size_t ws_bytes, void* stream) {
  moe_status s;
  if ((s = check_dims(dims)) != MOE_OK || (s = check_opts(opts)) != MOE_OK) return s;
  if ((s = check_gate_args(dims, opts, x, w_gate, w_noise, gate_bias, eps, true)) != MOE_OK) return s;
  REQN(topk_idx, 4, dims->tokens);
  REQN(topk_gate, 4, dims->tokens);
  REQN(thresh, 4, dims->tokens);
  // the workspace is optional here: it only lets a small batch split its sweep
  const size_t need = ws ? layout(dims, opts).gate_bytes : 0;
  if ((s = check_ws(ws, ws_bytes, need)) != MOE_OK) return s;
  const moe::GateLaunch g = gate_launch(dims, opts, x, w_gate, w_noise, gate_bias, eps);
  return device_status(moe::launch_gate(g, topk_idx, topk_gate, thresh, (hipStream_t)stream,
                                        need ? ws : nullptr),
                       "moe_gate");
}

moe_status moe_route(const moe_dims* dims, const int32_t* topk_idx, const float* topk_gate,
                     int32_t* counts, int32_t* offsets, int32_t* perm_token, float* perm_gate,
                     int32_t* slot_pos, float* importance, void* ws, size_t ws_bytes,
                     void* stream) {
  moe_status s;
  if ((s = check_dims(dims)) != MOE_OK) return s;
  REQN(topk_idx, 4, dims->tokens);
  REQN(topk_gate, 4, dims->tokens);
  REQ(counts, 4);
  REQ(offsets, 4);
  REQN(perm_token, 4, dims->tokens);
  REQN(perm_gate, 4, dims->tokens);
  REQN(slot_pos, 4, dims->tokens);
  OPT(importance, 4);
  const Layout L = layout(dims, nullptr);
  if ((s = check_ws(ws, ws_bytes, L.route_bytes)) != MOE_OK) return s;
  return device_status(
      moe::launch_route(dims->tokens, dims->k, dims->n_experts, topk_idx, topk_gate,
                        at<int32_t>(ws, 0), counts, offsets, perm_token, perm_gate, slot_pos,
                        importance, (hipStream_t)stream, dims->capacity),
      "moe_route");
}

moe_status moe_expert_ffn(const moe_dims* dims, const void* x, const int32_t* offsets,
                          const int32_t* perm_token, const void* w1, const void* b1,
                          const void* w2, const void* b2, void* expert_out, void* ws,
                          size_t ws_bytes, void* stream) {
  moe_status s;
  if ((s = check_dims(dims)) != MOE_OK) return s;
  REQN(x, 16, dims->tokens);
  REQ(offsets, 4);
  REQN(perm_token, 4, dims->tokens);
  REQ(w1, 16);
  REQ(w2, 16);
  OPT(b1, 4);
  OPT(b2, 4);
  REQN(expert_out, 16, dims->tokens);
  if (!moe::ffn_supported(dims->d_model, dims->d_hidden, to_dt(dims->act_dtype)))
    return fail(MOE_ERR_UNSUPPORTED, "expert_ffn: unsupported shape");
  const Layout L = layout(dims, nullptr);
  if ((s = check_ws(ws, ws_bytes, L.ffn_bytes)) != MOE_OK) return s;
  return device_status(
      moe::launch_ffn(dims->tokens, dims->k, dims->d_model, dims->d_hidden, dims->n_experts,
                      to_dt(dims->act_dtype), x, offsets, perm_token, w1, b1, w2, b2, expert_out,
                      at<int32_t>(ws, 0), (hipStream_t)stream, nullptr, nullptr, dims->capacity,
                      nullptr, 0, dims->expert_layout == 1),
      "moe_expert_ffn");
}

moe_status moe_pack_expert_weights(const moe_dims* dims, const void* w1, const void* w2,
                                   void* w1_packed, void* w2_packed, void* stream) {
  moe_status s;
  if ((s = check_dims(dims)) != MOE_OK) return s;
  if (!moe::ffn_supported(dims->d_model, dims->d_hidden, to_dt(dims->act_dtype)))
    return fail(MOE_ERR_UNSUPPORTED, "pack_expert_weights: unsupported shape");
  REQ(w1, 16);
  REQ(w2, 16);
  REQ(w1_packed, 16);
  REQ(w2_packed, 16);
  const int64_t es = dims->expert_dtype == MOE_BF16 ? 2 : 4;
  const int64_t n = dims->n_experts, d = dims->d_model, h = dims->d_hidden;
  const int64_t bytes = n * h * d * es;  // each of w1, w2
  const void* ins[2] = {w1, w2};
  void* outs[2] = {w1_packed, w2_packed};
  for (const void* a : ins)
    for (void* b : outs) {
      const uintptr_t pa = (uintptr_t)a, pb = (uintptr_t)b;
      if (pa < pb + (uintptr_t)bytes && pb < pa + (uintptr_t)bytes)
        return fail(MOE_ERR_INVALID, "pack_expert_weights: a packed output overlaps an input");
    }
  if ((uintptr_t)w1_packed < (uintptr_t)w2_packed + (uintptr_t)bytes &&
      (uintptr_t)w2_packed < (uintptr_t)w1_packed + (uintptr_t)bytes)
    return fail(MOE_ERR_INVALID, "pack_expert_weights: w1_packed and w2_packed overlap");
  hipError_t e = moe::launch_pack_weights(w1, w1_packed, n * h, d * es, (hipStream_t)stream);
  if (e == hipSuccess)
    e = moe::launch_pack_weights(w2, w2_packed, n * d, h * es, (hipStream_t)stream);
  return device_status(e, "moe_pack_expert_weights");
}

moe_status moe_combine(const moe_dims* dims, const void* expert_out, const int32_t* slot_pos,
                       const float* topk_gate, void* y, void* stream) {
  moe_status s;
  if ((s = check_dims(dims)) != MOE_OK) return s;
  REQN(expert_out, 16, dims->tokens);
  REQN(slot_pos, 4, dims->tokens);
  REQN(topk_gate, 4, dims->tokens);
  REQN(y, 16, dims->tokens);
  return device_status(moe::launch_combine(dims->tokens, dims->k, dims->d_model,
                                           to_dt(dims->act_dtype), expert_out, slot_pos, topk_gate,
                                           y, (hipStream_t)stream),
                       "moe_combine");
}

moe_status moe_aux_losses(const moe_dims* dims, const moe_gate_opts* opts, const void* x,
                          const void* w_gate, const void* w_noise, const float* gate_bias,
                          const float* thresh, const int32_t* offsets, const int32_t* perm_token,
                          const float* importance, float* load, float* losses, void* ws,
                          size_t ws_bytes, void* stream) {
  moe_status s;
  if ((s = check_dims(dims)) != MOE_OK || (s = check_opts(opts)) != MOE_OK) return s;
  REQ(importance, 4);
  REQ(load, 4);
  REQ(losses, 4);
  REQ(offsets, 4);
  const hipStream_t st = (hipStream_t)stream;
  if (opts->train) {
    if ((s = check_gate_args(dims, opts, x, w_gate, w_noise, gate_bias, nullptr, false)) !=
        MOE_OK)
      return s;
    REQN(thresh, 4, dims->tokens);
    REQN(perm_token, 4, dims->tokens);
    const Layout L = layout(dims, opts);
    if ((s = check_ws(ws, ws_bytes, L.aux_bytes)) != MOE_OK) return s;
    const moe::GateLaunch g = gate_launch(dims, opts, x, w_gate, w_noise, gate_bias, nullptr);
    hipError_t e = moe::launch_load(g, thresh, offsets, perm_token, at<float>(ws, 0),
                                    at<float>(ws, L.load_corr - L.load_partial), load, st);
    if (e != hipSuccess) return device_status(e, "moe_aux_losses (load)");
  } else {
    hipError_t e = moe::launch_offsets_to_load(offsets, dims->n_experts, load, st);
    if (e != hipSuccess) return device_status(e, "moe_aux_losses (counts)");
  }
  return device_status(moe::launch_cv2_losses(importance, load, dims->n_experts,
                                               opts->w_importance, opts->w_load, losses, st),
                       "moe_aux_losses (cv2)");
}

moe_status moe_forward(const moe_dims* dims, const moe_gate_opts* opts, const void* x,
                       const void* w_gate, const void* w_noise, const float* gate_bias,
                       const float* eps, const void* w1, const void* b1, const void* w2,
                       const void* b2, void* y, float* importance, float* load, float* losses,
                       int32_t* topk_idx_out, float* topk_gate_out, float* thresh_out,
                       int32_t* counts_out, int32_t* perm_token_out, void* ws, size_t ws_bytes,
                       void* stream) {
  moe_status s;
  if ((s = check_dims(dims)) != MOE_OK || (s = check_opts(opts)) != MOE_OK) return s;
  if ((s = check_gate_args(dims, opts, x, w_gate, w_noise, gate_bias, eps, true)) != MOE_OK) return s;
  REQ(w1, 16);
  REQ(w2, 16);
  OPT(b1, 4);
  OPT(b2, 4);
  REQN(y, 16, dims->tokens);
  REQ(importance, 4);
  REQ(load, 4);
  REQ(losses, 4);
  OPT(topk_idx_out, 4);
  OPT(topk_gate_out, 4);
  OPT(thresh_out, 4);
  OPT(counts_out, 4);
  OPT(perm_token_out, 4);
  if (!moe::ffn_supported(dims->d_model, dims->d_hidden, to_dt(dims->act_dtype)))
    return fail(MOE_ERR_UNSUPPORTED, "expert_ffn: unsupported shape");
  const Layout L = layout(dims, opts);
  if ((s = check_ws(ws, ws_bytes, L.total)) != MOE_OK) return s;

  const hipStream_t st = (hipStream_t)stream;
  int32_t* topk_idx = topk_idx_out ? topk_idx_out : at<int32_t>(ws, L.topk_idx);
  float* topk_gate = topk_gate_out ? topk_gate_out : at<float>(ws, L.topk_gate);
  float* thresh = thresh_out ? thresh_out : at<float>(ws, L.thresh);
  int32_t* counts = counts_out ? counts_out : at<int32_t>(ws, L.counts);
  int32_t* offsets = at<int32_t>(ws, L.offsets);
  int32_t* perm_token = perm_token_out ? perm_token_out : at<int32_t>(ws, L.perm_token);
  float* perm_gate = at<float>(ws, L.perm_gate);
  int32_t* slot_pos = at<int32_t>(ws, L.slot_pos);
  void* expert_out = at<char>(ws, L.expert_out);

  const moe::GateLaunch g = gate_launch(dims, opts, x, w_gate, w_noise, gate_bias, eps);
  hipError_t e = moe::launch_gate(g, topk_idx, topk_gate, thresh, st,
                                  L.gate_bytes ? at<char>(ws, L.gate_cand) : nullptr);
  if (e != hipSuccess) return device_status(e, "moe_forward (gate)");
  e = moe::launch_route(dims->tokens, dims->k, dims->n_experts, topk_idx, topk_gate,
                        at<int32_t>(ws, L.blockcnt), counts, offsets, perm_token, perm_gate,
                        slot_pos, importance, st, dims->capacity);
  if (e != hipSuccess) return device_status(e, "moe_forward (route)");
  hipEvent_t t0, t1;
  timing_pair(&t0, &t1);
  e = moe::launch_ffn(dims->tokens, dims->k, dims->d_model, dims->d_hidden, dims->n_experts,
                      to_dt(dims->act_dtype), x, offsets, perm_token, w1, b1, w2, b2, expert_out,
                      at<int32_t>(ws, L.ffn_blocks), st, t0, t1, dims->capacity, nullptr, 0,
                      dims->expert_layout == 1);
  if (e != hipSuccess) return device_status(e, "moe_forward (expert_ffn)");
  e = moe::launch_combine(dims->tokens, dims->k, dims->d_model, to_dt(dims->act_dtype), expert_out,
                          slot_pos, topk_gate, y, st);
  if (e != hipSuccess) return device_status(e, "moe_forward (combine)");
  if (opts->train)
    e = moe::launch_load(g, thresh, offsets, perm_token, at<float>(ws, L.load_partial),
                         at<float>(ws, L.load_corr), load, st);
  else
    e = moe::launch_counts_to_load(counts, dims->n_experts, load, st);
  if (e != hipSuccess) return device_status(e, "moe_forward (load)");
  e = moe::launch_cv2_losses(importance, load, dims->n_experts, opts->w_importance, opts->w_load,
                             losses, st);
  return device_status(e, "moe_forward (losses)");
}

namespace {

// The static scratch of moe_forward_noalloc: each device the library runs on
// holds its own copy until the process ends. Host code never passes the
// array's name to a kernel (on the host it is a stand-in, not a device
// address); it uses the address hipGetSymbolAddress gives for the current
// device, kept per device on the device's first call.
__device__ __align__(256) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];

constexpr int kScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kScratchDevices] = {};

moe_status scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return device_status(e, "moe_forward_noalloc (current device)");
  if (dev < 0 || dev >= kScratchDevices)
    return fail(MOE_ERR_UNSUPPORTED, "moe_forward_noalloc: device %d, at most %d devices", dev,
                kScratchDevices);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return device_status(e, "moe_forward_noalloc (scratch address)");
    if (!p || !aligned(p, kAlign))
      return fail(MOE_ERR_DEVICE, "moe_forward_noalloc: scratch address %p is not usable", p);
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

moe_status check_batchwise(const moe_dims* d, const moe_gate_opts* o, int32_t m) {
  moe_status s;
  if ((s = check_dims(d)) != MOE_OK || (s = check_opts(o)) != MOE_OK) return s;
  if (d->capacity != 0)
    return fail(MOE_ERR_UNSUPPORTED, "batchwise gating: capacity must be 0 (m bounds each expert)");
  if (o->gate_order != 0)
    return fail(MOE_ERR_UNSUPPORTED, "batchwise gating: gate_order must be 0");
  if (d->tokens > 65536)
    return fail(MOE_ERR_UNSUPPORTED, "batchwise gating: tokens = %lld > 65536",
                (long long)d->tokens);
  if (m < 1) return fail(MOE_ERR_INVALID, "rows_per_expert = %d < 1", m);
  if ((int64_t)m * d->n_experts > (int64_t)0x7FFFFFFE)
    return fail(MOE_ERR_INVALID, "n_experts * rows_per_expert does not fit int32 indices");
  if (!moe::ffn_supported(d->d_model, d->d_hidden, to_dt(d->act_dtype)))
    return fail(MOE_ERR_UNSUPPORTED, "expert_ffn: unsupported shape");
  return MOE_OK;
}

}  // namespace

moe_status moe_forward_noalloc(const moe_dims* dims, const moe_gate_opts* opts, const void* x,
                               const void* w_gate, const void* w_noise, const float* gate_bias,
                               const float* eps, const void* w1, const void* b1, const void* w2,
                               const void* b2, void* y, float* importance, float* load,
                               float* losses, int32_t* topk_idx_out, float* topk_gate_out,
                               float* thresh_out, int32_t* counts_out, int32_t* perm_token_out,
                               void* stream) {
  moe_status s;
  if ((s = check_dims(dims)) != MOE_OK || (s = check_opts(opts)) != MOE_OK) return s;
  const size_t need = layout(dims, opts).total;
  if (need > (size_t)MOE_NOALLOC_SCRATCH_BYTES)
    return fail(MOE_ERR_WORKSPACE,
                "moe_forward_noalloc: these dims need %zu bytes of scratch, more than the "
                "library's static %zu bytes (use moe_forward with a workspace)",
                need, (size_t)MOE_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  if ((s = scratch_address(&ws)) != MOE_OK) return s;
  return moe_forward(dims, opts, x, w_gate, w_noise, gate_bias, eps, w1, b1, w2, b2, y,
                     importance, load, losses, topk_idx_out, topk_gate_out, thresh_out, counts_out,
                     perm_token_out, ws, (size_t)MOE_NOALLOC_SCRATCH_BYTES, stream);
}

size_t moe_backward_workspace_size(const moe_dims* dims, const moe_gate_opts* opts) {
  if (check_dims(dims) != MOE_OK) return 0;
  if (opts && check_opts(opts) != MOE_OK) return 0;
  return moe::backward_ws_bytes(dims->tokens, dims->n_experts, dims->k, dims->d_model,
                                dims->d_hidden, to_dt(dims->act_dtype));
}

moe_status moe_backward(const moe_dims* dims, const moe_gate_opts* opts, const void* x,
                        const void* w_gate, const void* w_noise, const float* gate_bias,
                        const float* eps, const void* w1, const void* b1, const void* w2,
                        const void* b2, const int32_t* topk_idx, const float* topk_gate,
                        const float* thresh, const float* importance, const float* load,
                        const void* dy, float aux_scale, float* dx, float* dw_gate,
                        float* dw_noise, float* dgate_bias, float* dw1, float* db1, float* dw2,
                        float* db2, void* ws, size_t ws_bytes, void* stream) {
  moe_status s;
  if ((s = check_dims(dims)) != MOE_OK || (s = check_opts(opts)) != MOE_OK) return s;
  if (dims->capacity != 0)
    return fail(MOE_ERR_UNSUPPORTED, "moe_backward: capacity must be 0");
  if (dims->expert_layout != 0)
    return fail(MOE_ERR_UNSUPPORTED, "moe_backward: expert_layout must be 0");
  if (opts->gate_order != 0)
    return fail(MOE_ERR_UNSUPPORTED, "moe_backward: gate_order must be 0");
  if (!std::isfinite(aux_scale)) return fail(MOE_ERR_INVALID, "aux_scale must be finite");
  if ((s = check_gate_args(dims, opts, x, w_gate, w_noise, gate_bias, eps, true)) != MOE_OK) return s;
  REQ(w1, 16);
  REQ(w2, 16);
  OPT(b1, 4);
  OPT(b2, 4);
  REQN(topk_idx, 4, dims->tokens);
  REQN(topk_gate, 4, dims->tokens);
  REQN(thresh, 4, dims->tokens);
  REQ(importance, 4);
  REQ(load, 4);
  REQN(dy, 16, dims->tokens);
  REQN(dx, 16, dims->tokens);
  REQ(dw_gate, 16);
  REQ(dw_noise, 16);
  OPT(dgate_bias, 4);
  REQ(dw1, 16);
  OPT(db1, 4);
  REQ(dw2, 16);
  OPT(db2, 4);
  if (!moe::ffn_supported(dims->d_model, dims->d_hidden, to_dt(dims->act_dtype)))
    return fail(MOE_ERR_UNSUPPORTED, "expert_ffn: unsupported shape");
  const size_t need = moe::backward_ws_bytes(dims->tokens, dims->n_experts, dims->k,
                                             dims->d_model, dims->d_hidden, to_dt(dims->act_dtype));
  if ((s = check_ws(ws, ws_bytes, need)) != MOE_OK) return s;
  moe::BackwardLaunch b;
  b.tokens = dims->tokens;
  b.d = dims->d_model;
  b.h = dims->d_hidden;
  b.n = dims->n_experts;
  b.k = dims->k;
  b.act_dt = to_dt(dims->act_dtype);
  b.gate_dt = to_dt(dims->gate_dtype);
  b.train = opts->train;
  b.noise_floor = opts->noise_floor;
  b.w_importance = opts->w_importance;
  b.w_load = opts->w_load;
  b.aux_scale = aux_scale;
  b.x = x;
  b.w_gate = w_gate;
  b.w_noise = w_noise;
  b.gate_bias = gate_bias;
  b.eps = opts->train ? eps : nullptr;
  b.w1 = w1;
  b.b1 = b1;
  b.w2 = w2;
  b.b2 = b2;
  b.topk_idx = topk_idx;
  b.topk_gate = topk_gate;
  b.thresh = thresh;
  b.importance = importance;
  b.load = load;
  b.dy = dy;
  b.dx = dx;
  b.dw_gate = dw_gate;
  b.dw_noise = dw_noise;
  b.dgate_bias = dgate_bias;
  b.dw1 = dw1;
  b.db1 = db1;
  b.dw2 = dw2;
  b.db2 = db2;
  return device_status(moe::launch_backward(b, ws, (hipStream_t)stream), "moe_backward");
}

size_t moe_batchwise_workspace_size(const moe_dims* dims, const moe_gate_opts* opts,
                                    int32_t rows_per_expert) {
  if (check_batchwise(dims, opts, rows_per_expert) != MOE_OK) return 0;
  return moe::batchwise_ws_bytes(dims->tokens, dims->n_experts, rows_per_expert, dims->d_model,
                                 dims->d_hidden, to_dt(dims->act_dtype));
}

moe_status moe_batchwise_forward(const moe_dims* dims, const moe_gate_opts* opts,
                                 int32_t rows_per_expert, const float* expert_threshold,
                                 const void* x, const void* w_gate, const void* w_noise,
                                 const float* gate_bias, const float* eps, const void* w1,
                                 const void* b1, const void* w2, const void* b2, void* y,
                                 int32_t* counts, int32_t* sel_token, float* sel_score,
                                 float* sel_gate, float* importance, float* load, float* losses,
                                 void* ws, size_t ws_bytes, void* stream) {
  moe_status s;
  if ((s = check_batchwise(dims, opts, rows_per_expert)) != MOE_OK) return s;
  if ((s = check_gate_args(dims, opts, x, w_gate, w_noise, gate_bias, eps, true)) != MOE_OK) return s;
  OPT(expert_threshold, 4);
  REQ(w1, 16);
  REQ(w2, 16);
  OPT(b1, 4);
  OPT(b2, 4);
  REQN(y, 16, dims->tokens);
  REQ(counts, 4);
  REQ(sel_token, 4);
  REQ(sel_score, 4);
  REQ(sel_gate, 4);
  REQ(importance, 4);
  REQ(load, 4);
  REQ(losses, 4);
  const moe::Dt adt = to_dt(dims->act_dtype);
  const size_t need = moe::batchwise_ws_bytes(dims->tokens, dims->n_experts, rows_per_expert,
                                              dims->d_model, dims->d_hidden, adt);
  if ((s = check_ws(ws, ws_bytes, need)) != MOE_OK) return s;
  moe::BatchwiseLaunch b;
  b.gate = gate_launch(dims, opts, x, w_gate, w_noise, gate_bias, eps);
  b.m = rows_per_expert;
  b.threshold = expert_threshold;
  b.h = dims->d_hidden;
  b.act_dt = adt;
  b.w1 = w1;
  b.b1 = b1;
  b.w2 = w2;
  b.b2 = b2;
  b.packed = dims->expert_layout == 1;
  b.w_importance = opts->w_importance;
  b.w_load = opts->w_load;
  b.y = y;
  b.counts = counts;
  b.sel_token = sel_token;
  b.sel_score = sel_score;
  b.sel_gate = sel_gate;
  b.importance = importance;
  b.load = load;
  b.losses = losses;
  moe::batchwise_carve(b, ws, dims->d_model, dims->d_hidden, adt);
  hipEvent_t t0, t1;
  timing_pair(&t0, &t1);
  return device_status(moe::launch_batchwise(b, (hipStream_t)stream, t0, t1),
                       "moe_batchwise_forward");
}

size_t moe_hier_workspace_size(const moe_hier_dims* dims, const moe_gate_opts* opts) {
  if (check_hier_dims(dims) != MOE_OK) return 0;
  if (opts && check_opts(opts) != MOE_OK) return 0;
  return hier_layout(dims, opts).total;
}

moe_status moe_hier_forward(const moe_hier_dims* dims, const moe_gate_opts* opts, const void* x,
                            const void* w_gate1, const void* w_noise1, const float* eps1,
                            const void* w_gate2, const void* w_noise2, const float* eps2,
                            const void* w1, const void* b1, const void* w2, const void* b2,
                            void* y, float* importance, float* load, float* losses,
                            const moe_hier_outputs* extra, void* ws, size_t ws_bytes,
                            void* stream) {
  moe_status s;
  if ((s = check_hier_dims(dims)) != MOE_OK || (s = check_opts(opts)) != MOE_OK) return s;
  if (opts->gate_order != 0)
    return fail(MOE_ERR_UNSUPPORTED, "moe_hier_forward: gate_order 1 applies to the flat layer");
  const int64_t B = dims->tokens;
  REQN(x, 16, B);
  REQ(w_gate1, 16);
  REQ(w_gate2, 16);
  if (opts->train) {
    REQ(w_noise1, 16);
    REQ(w_noise2, 16);
    REQN(eps1, 16, B);
    REQN(eps2, 16, B);
  } else {
    OPT(w_noise1, 16);
    OPT(w_noise2, 16);
  }
  REQ(w1, 16);
  REQ(w2, 16);
  OPT(b1, 4);
  OPT(b2, 4);
  REQN(y, 16, B);
  REQ(importance, 4);
  REQ(load, 4);
  REQ(losses, 4);
  moe_hier_outputs none{};
  const moe_hier_outputs* ex = extra ? extra : &none;
  OPT(ex->topk_idx, 4);
  OPT(ex->topk_gate, 4);
  OPT(ex->counts, 4);
  OPT(ex->group_idx, 4);
  OPT(ex->group_gate, 4);
  OPT(ex->group_thresh, 4);
  OPT(ex->group_rows, 4);
  OPT(ex->group_importance, 4);
  OPT(ex->group_load, 4);
  OPT(ex->sub_idx, 4);
  OPT(ex->sub_gate, 4);
  OPT(ex->sub_thresh, 4);
  OPT(ex->sub_load, 4);
  const moe::Dt x_dt = to_dt(dims->act_dtype), w_dt = to_dt(dims->gate_dtype);
  if (!moe::gate_supported(dims->d_model, x_dt, w_dt, dims->k1) ||
      !moe::gate_supported(dims->d_model, x_dt, w_dt, dims->k2))
    return fail(MOE_ERR_UNSUPPORTED, "gate: unsupported shape or dtype combination");
  if (!moe::ffn_supported(dims->d_model, dims->d_hidden, x_dt))
    return fail(MOE_ERR_UNSUPPORTED, "expert_ffn: unsupported shape");
  const HierLayout L = hier_layout(dims, opts);
  if ((s = check_ws(ws, ws_bytes, L.total)) != MOE_OK) return s;

  const hipStream_t st = (hipStream_t)stream;
  const int a = dims->groups, b = dims->group_experts, k1 = dims->k1, k2 = dims->k2;
  const int n = a * b, K = k1 * k2;
  auto pick = [&](auto* given, size_t off) {
    using T = std::remove_pointer_t<decltype(given)>;
    return given ? given : at<T>(ws, off);
  };
  int32_t* sel1 = pick(ex->group_idx, L.sel1);
  float* gate1 = pick(ex->group_gate, L.gate1);
  float* thr1 = pick(ex->group_thresh, L.thr1);
  int32_t* counts1 = pick(ex->group_rows, L.counts1);
  float* imp1 = pick(ex->group_importance, L.imp1);
  float* load1 = pick(ex->group_load, L.load1);
  int32_t* sel2 = pick(ex->sub_idx, L.sel2);
  float* gate2 = pick(ex->sub_gate, L.gate2);
  float* thr2 = pick(ex->sub_thresh, L.thr2);
  float* load2 = pick(ex->sub_load, L.load2);
  int32_t* topk_idx = pick(ex->topk_idx, L.topk_idx);
  float* topk_gate = pick(ex->topk_gate, L.topk_gate);
  int32_t* counts = pick(ex->counts, L.counts);
  int32_t* offsets1 = at<int32_t>(ws, L.offsets1);
  int32_t* perm_token1 = at<int32_t>(ws, L.perm_token1);
  int32_t* perm_slot1 = at<int32_t>(ws, L.perm_slot1);
  int32_t* unit_start = at<int32_t>(ws, L.unit_start);
  int32_t* units = at<int32_t>(ws, L.units);
  int32_t* offsets = at<int32_t>(ws, L.offsets);
  int32_t* perm_token = at<int32_t>(ws, L.perm_token);
  int32_t* slot_pos = at<int32_t>(ws, L.slot_pos);
  void* expert_out = at<char>(ws, L.expert_out);

  // primary gate and the routing of each token's k1 slots to their groups
  const moe::GateLaunch g1 = hier_gate_launch(dims, opts, 1, x, w_gate1, w_noise1, eps1);
  hipError_t e = moe::launch_gate(g1, sel1, gate1, thr1, st);
  if (e != hipSuccess) return device_status(e, "moe_hier_forward (primary gate)");
  e = moe::launch_route(B, k1, a, sel1, gate1, at<int32_t>(ws, L.blockcnt1), counts1, offsets1,
                        perm_token1, at<float>(ws, L.perm_gate1), at<int32_t>(ws, L.slot_pos1),
                        imp1, st);
  if (e != hipSuccess) return device_status(e, "moe_hier_forward (primary route)");
  e = moe::launch_invert_slots(at<int32_t>(ws, L.slot_pos1), B * k1, perm_slot1, st);
  if (e != hipSuccess) return device_status(e, "moe_hier_forward (slots)");
  // secondary gates over each group's routed rows
  moe::GateLaunch g2 = hier_gate_launch(dims, opts, 2, x, w_gate2, w_noise2, eps2);
  g2.units = units;
  g2.seg_off = offsets1;
  g2.row_token = perm_token1;
  g2.row_slot = perm_slot1;
  g2.max_units = L.max_units;
  e = moe::launch_group_plan(offsets1, a, moe::gate_tile_rows(g2), units, unit_start, st);
  if (e != hipSuccess) return device_status(e, "moe_hier_forward (plan)");
  e = moe::launch_gate(g2, sel2, gate2, thr2, st);
  if (e != hipSuccess) return device_status(e, "moe_hier_forward (secondary gate)");
  // leaves, then the flat path over them
  e = moe::launch_hier_leaves(B, k1, k2, b, sel1, gate1, sel2, gate2, topk_idx, topk_gate, st);
  if (e != hipSuccess) return device_status(e, "moe_hier_forward (leaves)");
  e = moe::launch_route(B, K, n, topk_idx, topk_gate, at<int32_t>(ws, L.blockcnt), counts, offsets,
                        perm_token, at<float>(ws, L.perm_gate), slot_pos, importance, st);
  if (e != hipSuccess) return device_status(e, "moe_hier_forward (route)");
  hipEvent_t t0, t1;
  timing_pair(&t0, &t1);
  e = moe::launch_ffn(B, K, dims->d_model, dims->d_hidden, n, x_dt, x, offsets, perm_token, w1, b1,
                      w2, b2, expert_out, at<int32_t>(ws, L.ffn_blocks), st, t0, t1, 0, nullptr,
                      0, dims->expert_layout == 1);
  if (e != hipSuccess) return device_status(e, "moe_hier_forward (expert_ffn)");
  e = moe::launch_combine(B, K, dims->d_model, x_dt, expert_out, slot_pos, topk_gate, y, st);
  if (e != hipSuccess) return device_status(e, "moe_hier_forward (combine)");
  // both levels' Load, then the leaf Load and the losses
  if (opts->train) {
    e = moe::launch_load(g1, thr1, offsets1, perm_token1, at<float>(ws, L.partial1),
                         at<float>(ws, L.corr1), load1, st);
    if (e == hipSuccess)
      e = moe::launch_load_grouped(g2, a, unit_start, thr2, offsets, perm_token, sel1, k1,
                                   at<float>(ws, L.partial2), at<float>(ws, L.corr2), load2, st);
  } else {
    e = moe::launch_counts_to_load(counts1, a, load1, st);
    if (e == hipSuccess) e = moe::launch_counts_to_load(counts, n, load2, st);
  }
  if (e != hipSuccess) return device_status(e, "moe_hier_forward (load)");
  e = moe::launch_hier_leaf_load(a, b, load1, load2, counts1, load, st);
  if (e != hipSuccess) return device_status(e, "moe_hier_forward (leaf load)");
  e = moe::launch_cv2_losses(importance, load, n, opts->w_importance, opts->w_load, losses, st);
  return device_status(e, "moe_hier_forward (losses)");
}

}  // extern "C"
