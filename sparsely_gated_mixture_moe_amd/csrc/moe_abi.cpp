// The C ABI of include/moe.h: argument validation, workspace layout and the
// order of kernel launches. Validation runs before any HIP call, so an invalid
// call launches nothing and writes nothing.
#include "../../include/moe.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <string>

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
      importance, blockcnt, ffn_blocks, expert_out, load_partial, total;
  size_t route_bytes, ffn_bytes, aux_bytes;  // standalone needs (from offset 0)
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
  L.ffn_bytes = align_up((size_t)(1 + 2 * moe::ffn_max_blocks(pairs, (int)n, d->d_model,
                                                             to_dt(d->act_dtype))) *
                         sizeof(int32_t));
  L.aux_bytes = (o && o->train) ? align_up((size_t)moe::gate_blocks(B) * n * sizeof(float)) : 0;
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
  return g;
}

moe_status check_gate_args(const moe_dims* d, const moe_gate_opts* o, const void* x,
                           const void* wg, const void* wn, const float* bias, const float* eps,
                           bool need_eps) {
  REQN(x, 16, d->tokens);
  REQ(wg, 16);
  if (o->train) REQ(wn, 16);
  else OPT(wn, 16);
  OPT(bias, 4);
  if (o->train && need_eps) REQN(eps, 4, d->tokens);
  if (!moe::gate_supported(d->d_model, to_dt(d->act_dtype), to_dt(d->gate_dtype), d->k))
    return fail(MOE_ERR_UNSUPPORTED, "gate: unsupported shape or dtype combination");
  return MOE_OK;
}

}  // namespace

extern "C" {

int moe_abi_version(void) { return MOE_ABI_VERSION; }

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
  (void)ws;
  (void)ws_bytes;
  moe_status s;
  if ((s = check_dims(dims)) != MOE_OK || (s = check_opts(opts)) != MOE_OK) return s;
  if ((s = check_gate_args(dims, opts, x, w_gate, w_noise, gate_bias, eps, true)) != MOE_OK) return s;
  REQN(topk_idx, 4, dims->tokens);
  REQN(topk_gate, 4, dims->tokens);
  REQN(thresh, 4, dims->tokens);
  const moe::GateLaunch g = gate_launch(dims, opts, x, w_gate, w_noise, gate_bias, eps);
  return device_status(moe::launch_gate(g, topk_idx, topk_gate, thresh, (hipStream_t)stream),
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
                        importance, (hipStream_t)stream),
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
                      at<int32_t>(ws, 0), (hipStream_t)stream),
      "moe_expert_ffn");
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
                          const int32_t* topk_idx, const float* thresh, const int32_t* counts,
                          const float* importance, float* load, float* losses, void* ws,
                          size_t ws_bytes, void* stream) {
  moe_status s;
  if ((s = check_dims(dims)) != MOE_OK || (s = check_opts(opts)) != MOE_OK) return s;
  REQ(importance, 4);
  REQ(load, 4);
  REQ(losses, 4);
  const hipStream_t st = (hipStream_t)stream;
  if (opts->train) {
    if ((s = check_gate_args(dims, opts, x, w_gate, w_noise, gate_bias, nullptr, false)) !=
        MOE_OK)
      return s;
    REQN(topk_idx, 4, dims->tokens);
    REQN(thresh, 4, dims->tokens);
    const Layout L = layout(dims, opts);
    if ((s = check_ws(ws, ws_bytes, L.aux_bytes)) != MOE_OK) return s;
    const moe::GateLaunch g = gate_launch(dims, opts, x, w_gate, w_noise, gate_bias, nullptr);
    hipError_t e = moe::launch_load(g, topk_idx, thresh, at<float>(ws, 0), load, st);
    if (e != hipSuccess) return device_status(e, "moe_aux_losses (load)");
  } else {
    REQ(counts, 4);
    hipError_t e = moe::launch_counts_to_load(counts, dims->n_experts, load, st);
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
  hipError_t e = moe::launch_gate(g, topk_idx, topk_gate, thresh, st);
  if (e != hipSuccess) return device_status(e, "moe_forward (gate)");
  e = moe::launch_route(dims->tokens, dims->k, dims->n_experts, topk_idx, topk_gate,
                        at<int32_t>(ws, L.blockcnt), counts, offsets, perm_token, perm_gate,
                        slot_pos, importance, st);
  if (e != hipSuccess) return device_status(e, "moe_forward (route)");
  e = moe::launch_ffn(dims->tokens, dims->k, dims->d_model, dims->d_hidden, dims->n_experts,
                      to_dt(dims->act_dtype), x, offsets, perm_token, w1, b1, w2, b2, expert_out,
                      at<int32_t>(ws, L.ffn_blocks), st);
  if (e != hipSuccess) return device_status(e, "moe_forward (expert_ffn)");
  e = moe::launch_combine(dims->tokens, dims->k, dims->d_model, to_dt(dims->act_dtype), expert_out,
                          slot_pos, topk_gate, y, st);
  if (e != hipSuccess) return device_status(e, "moe_forward (combine)");
  if (opts->train)
    e = moe::launch_load(g, topk_idx, thresh, at<float>(ws, L.load_partial), load, st);
  else
    e = moe::launch_counts_to_load(counts, dims->n_experts, load, st);
  if (e != hipSuccess) return device_status(e, "moe_forward (load)");
  e = moe::launch_cv2_losses(importance, load, dims->n_experts, opts->w_importance, opts->w_load,
                             losses, st);
  return device_status(e, "moe_forward (losses)");
}

}  // extern "C"
