// Host-side launch wrappers shared between the kernel translation units and
// the C ABI. Plain pointers and sizes only; every wrapper enqueues on the
// given stream and returns the launch status.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

enum Dt { kF32 = 0, kBF16 = 1 };

// Gate kernel geometry: 8 waves of 16 token rows each; the 32x32-tile kernel
// for bf16 gates runs 8 waves of 32 rows.
constexpr int kGateRows = 128;
constexpr int kGate32Rows = 256;
constexpr int kGate32Chunk = 16;  // experts per chunk of the 32x32-tile kernel
// Routing: tokens per block of the counting sort.
constexpr int kRouteTokens = 256;

struct GateLaunch {
  const void* x;
  const void* w_gate;
  const void* w_noise;
  const float* bias;  // may be null
  const float* eps;   // null when !train
  int64_t tokens;
  int d, n, k;
  Dt x_dt, w_dt;
  int train;
  float noise_floor;
  // Secondary gating of a hierarchical layer (all null for a flat gate): the
  // rows are the routed rows of a primary route, tiled per group by
  // launch_group_plan; `tokens` is then the number of routed rows, `n` the
  // experts per group, and w_gate / w_noise / bias hold every group's block.
  const int32_t* units = nullptr;      // [1 + 2 * max_units]
  const int32_t* seg_off = nullptr;    // [groups + 1] primary route offsets
  const int32_t* row_token = nullptr;  // [tokens] x row of each routed row
  const int32_t* row_slot = nullptr;   // [tokens] eps / output row of each routed row
  int64_t max_units = 0;
  // Flat gating of a small batch: each row tile's expert sweep split into
  // `ranges` consecutive ranges of chunks, one workgroup each (set by the
  // launchers from gate_ranges).
  int ranges = 1;
  // 1: the gates are the softmax over all n logits at the selected experts
  // (the selection is the same); 0: the softmax over the kept k.
  int gate_order = 0;
};

// The gradient pass of the gate (flat bf16 gate in training mode, the 32x32
// kernel): for every (token, expert) pair, taken as unselected, d loss / d
// clean logit and d loss / d noise pre-activation through the Load term
// (threshold thresh [row][0], the k-th logit; dload [n] = d loss / d Load)
// into dcu [n / 16][B][32]: for expert block q and token t, the 16 clean
// gradients of experts 16 q .. 16 q + 15, then their 16 noise gradients.
bool gate_pair_grads_supported(const GateLaunch& g);
hipError_t launch_gate_pair_grads(const GateLaunch& g, const float* thresh, const float* dload,
                                  float* dcu, hipStream_t s);

// Batchwise gating's scores: H of every (token, expert) pair, written
// expert-major to scores [n][sld], sld >= B (same arithmetic as launch_gate's H).
hipError_t launch_scores(const GateLaunch& g, float* scores, int64_t sld, hipStream_t s);

// Noisy top-k gating: writes topk_idx [B,k], topk_gate [B,k], thresh [B,2].
// cand (gate_cand_bytes(g) bytes, or null) lets a small flat batch split
// its expert sweep.
hipError_t launch_gate(const GateLaunch& g, int32_t* topk_idx, float* topk_gate, float* thresh,
                       hipStream_t s, void* cand = nullptr);

// Load (eq 10) with train = 1: recomputes the logits, evaluates P for every
// (token, expert) against the row's k-th logit and writes per-block column sums
// partial [blocks][n]; corrects the selected pairs to the (k+1)-th threshold
// from the routed rows (offsets / perm_token of the route of this selection)
// into corr (corr_bytes of the pairs over n experts); then reduces both into
// load [n].
int gate_blocks(int64_t tokens);
// The selected pairs' corrections are summed over slices of at most
// kCorrSliceRows routed rows of one expert, one workgroup each, so that an
// expert with many rows is spread over many workgroups. The corr region of
// corr_bytes(pairs, n) bytes holds one float per slice (at most
// corr_slices_max(pairs, n) slices), then each expert's first slice [n + 1]
// (int32), then each slice's expert [corr_slices_max] (int32).
constexpr int kCorrSliceRows = 256;
int64_t corr_slices_max(int64_t pairs, int n);
size_t corr_bytes(int64_t pairs, int n);
hipError_t launch_load(const GateLaunch& g, const float* thresh, const int32_t* offsets,
                       const int32_t* perm_token, float* partial, float* corr, float* load,
                       hipStream_t s);
bool gate_supported(int d, Dt x_dt, Dt w_dt, int k);
// Expert ranges per row tile for flat gating of `g` (1: no split): a batch of
// fewer row tiles than half of 256 workgroups splits each tile's sweep over
// the experts into up to 256 / tiles ranges of at least two chunks. A
// selection split this way leaves each range's best k+1 (value, expert) of
// every row in a candidate buffer of gate_cand_bytes(g) bytes, merged by a
// second kernel; without that buffer launch_gate does not split.
int gate_ranges(const GateLaunch& g);
size_t gate_cand_bytes(const GateLaunch& g);

// Secondary (grouped) gating. Rows per work unit of the kernel that `g` runs
// on; the largest unit count for `rows` routed rows over `groups` groups;
// the unit list (units [1 + 2 * max_units], unit_start [groups + 1]) from the
// primary route's offsets; the Load pass, whose per-unit partial sums
// ([max_units][n]) plus the selected pairs' corrections (from the route of the
// leaves, leaf = group * n + expert, and the primary selection sel1
// that gives each token's rank of the group) are reduced per group into
// load [groups * n].
int gate_tile_rows(const GateLaunch& g);
int64_t gate_max_units(int64_t rows, int groups, int tile_rows);
hipError_t launch_group_plan(const int32_t* offsets, int groups, int tile_rows, int32_t* units,
                             int32_t* unit_start, hipStream_t s);
hipError_t launch_load_grouped(const GateLaunch& g, int groups, const int32_t* unit_start,
                               const float* thresh, const int32_t* leaf_offsets,
                               const int32_t* leaf_perm_token, const int32_t* sel1, int k1,
                               float* partial, float* corr, float* load, hipStream_t s);

// Routing.
int route_blocks(int64_t tokens);
// capacity > 0: pairs past the first `capacity` of their expert's segment
// get slot_pos -1 (the segments and counts are unchanged).
hipError_t launch_route(int64_t tokens, int k, int n, const int32_t* topk_idx,
                        const float* topk_gate, int32_t* blockcnt /* [n][route_blocks] */,
                        int32_t* counts, int32_t* offsets, int32_t* perm_token, float* perm_gate,
                        int32_t* slot_pos, float* importance, hipStream_t s, int capacity = 0);

// Expert FFN.
int ffn_rows_per_block(int d, Dt dt);
int64_t ffn_max_blocks(int64_t rows, int n, int d, Dt dt);
// Bytes of the expert-FFN workspace: the work-unit list (the count, then 16
// bytes per unit) and, for a batch of few units split over the hidden units
// (ffn_hsplit > 1 ranges), each unit's fp32 partial output rows.
size_t ffn_plan_bytes(int64_t rows, int n, int d, int h, Dt dt);
int ffn_hsplit(int64_t rows, int n, int d, int h, Dt dt);
bool ffn_supported(int d, int h, Dt dt);
// ev0 / ev1, when given, are recorded on s right before and after the FFN
// kernel (after its plan kernel); capacity > 0 computes only the first
// `capacity` rows of each segment. With seg_counts, expert e's segment is
// rows [e * seg_stride, e * seg_stride + seg_counts[e]) and offsets is unused;
// tokens * k is then the row count the workspace was sized for.
hipError_t launch_ffn(int64_t tokens, int k, int d, int h, int n, Dt dt, const void* x,
                      const int32_t* offsets, const int32_t* perm_token, const void* w1,
                      const void* b1, const void* w2, const void* b2, void* expert_out,
                      int32_t* blocks /* [2*max_blocks + 1] */, hipStream_t s,
                      hipEvent_t ev0 = nullptr, hipEvent_t ev1 = nullptr, int capacity = 0,
                      const int32_t* seg_counts = nullptr, int seg_stride = 0,
                      bool packed = false);
// packed: w1 and w2 are in the packed layout that launch_pack_weights writes.

// Copies a row-major matrix of `rows` rows (a multiple of 16) and row_bytes
// bytes per row (a multiple of 64) into the packed layout of the expert FFN's
// weight operands (16-row x 64-byte blocks, one kilobyte each, in the order
// the product's lanes read them). src and dst must not overlap.
hipError_t launch_pack_weights(const void* src, void* dst, int64_t rows, int64_t row_bytes,
                               hipStream_t s);

// Weighted sum.
hipError_t launch_combine(int64_t tokens, int k, int d, Dt dt, const void* expert_out,
                          const int32_t* slot_pos, const float* topk_gate, void* y,
                          hipStream_t s);

// Hierarchical layer: inverse of a route's slot_pos (perm_slot[slot_pos[q]] = q);
// leaves of each token from both levels (leaf r*k2 + j = sel1[r]*b + sel2[r][j],
// gate gate1[r]*gate2[r][j]); leaf Load = load1[i] * load2[i*b + j] / rows1[i].
hipError_t launch_invert_slots(const int32_t* slot_pos, int64_t npairs, int32_t* perm_slot,
                               hipStream_t s);
hipError_t launch_hier_leaves(int64_t tokens, int k1, int k2, int b, const int32_t* sel1,
                              const float* gate1, const int32_t* sel2, const float* gate2,
                              int32_t* leaf_idx, float* leaf_gate, hipStream_t s);
hipError_t launch_hier_leaf_load(int a, int b, const float* load1, const float* load2,
                                 const int32_t* rows1, float* load, hipStream_t s);

// Batchwise gating: every expert takes the rows of the batch with the largest
// scores H (above its threshold, if given), at most m; each token's gates are
// the softmax of the scores of the experts that took it. Slots e*m .. e*m +
// counts[e] - 1 hold expert e's rows in token order. B <= 65536.
struct BatchwiseLaunch {
  GateLaunch gate;           // x, gate weights, noise; k unused
  int m = 0;
  const float* threshold = nullptr;  // [n] or null (no threshold)
  int h = 0;
  Dt act_dt = kBF16;
  const void *w1 = nullptr, *b1 = nullptr, *w2 = nullptr, *b2 = nullptr;
  bool packed = false;  // w1, w2 in the packed layout of launch_pack_weights
  float w_importance = 0.f, w_load = 0.f;
  // outputs
  void* y = nullptr;
  int32_t* counts = nullptr;     // [n]
  int32_t* sel_token = nullptr;  // [n*m]
  float* sel_score = nullptr;    // [n*m]
  float* sel_gate = nullptr;     // [n*m]
  float* importance = nullptr;   // [n]
  float* load = nullptr;         // [n]
  float* losses = nullptr;       // [3]
  // workspace (batchwise_carve)
  float* scores = nullptr;       // [n][score_ld], score_ld = B rounded up to 4
  int32_t* tok_cnt = nullptr;    // [B]
  int32_t* tok_off = nullptr;    // [B + 1]
  int32_t* tok_list = nullptr;   // [n*m]
  int32_t* tok_sorted = nullptr; // [n*m]
  int32_t* ffn_blocks = nullptr;
  void* expert_out = nullptr;    // [n*m][d]
};
size_t batchwise_ws_bytes(int64_t tokens, int n, int m, int d, int h, Dt act_dt);
void batchwise_carve(BatchwiseLaunch& b, void* ws, int d, int h, Dt act_dt);
hipError_t launch_batchwise(const BatchwiseLaunch& b, hipStream_t s, hipEvent_t ev0 = nullptr,
                            hipEvent_t ev1 = nullptr);

// Backward pass: gradients of sum dy . y + aux_scale (w_importance CV^2(Imp) +
// w_load CV^2(Load)) for x and every parameter (fp32), from the forward's
// selection (topk_idx / topk_gate), thresholds, Importance and Load, with the
// hidden activations recomputed. backward_ws_bytes sizes its workspace.
struct BackwardLaunch {
  int64_t tokens = 0;
  int d = 0, h = 0, n = 0, k = 0;
  Dt act_dt = kBF16, gate_dt = kBF16;  // experts share the activations' type
  int train = 1;
  float noise_floor = 0.f, w_importance = 0.f, w_load = 0.f, aux_scale = 1.f;
  const void *x = nullptr, *w_gate = nullptr, *w_noise = nullptr;
  const float* gate_bias = nullptr;
  const float* eps = nullptr;
  const void *w1 = nullptr, *b1 = nullptr, *w2 = nullptr, *b2 = nullptr;
  const int32_t* topk_idx = nullptr;
  const float *topk_gate = nullptr, *thresh = nullptr, *importance = nullptr, *load = nullptr;
  const void* dy = nullptr;
  float *dx = nullptr, *dw_gate = nullptr, *dw_noise = nullptr, *dgate_bias = nullptr;
  float *dw1 = nullptr, *db1 = nullptr, *dw2 = nullptr, *db2 = nullptr;
};
size_t backward_ws_bytes(int64_t tokens, int n, int k, int d, int h, Dt act_dt);
hipError_t launch_backward(const BackwardLaunch& b, void* ws, hipStream_t s);

// Compute units of the current device (cached per device).
hipError_t device_cus(int* cus);

// Load as the hard count (train = 0) and the CV^2 losses.
hipError_t launch_counts_to_load(const int32_t* counts, int n, float* load, hipStream_t s);
hipError_t launch_offsets_to_load(const int32_t* offsets, int n, float* load, hipStream_t s);
hipError_t launch_cv2_losses(const float* importance, const float* load, int n, float w_imp,
                             float w_load, float* losses, hipStream_t s);

}  // namespace moe
