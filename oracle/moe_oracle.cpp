// Oracle: a plain, slow CPU definition of the sparsely-gated MoE forward pass.
//
// TEST INFRASTRUCTURE ONLY. Nothing on the product path may call, link or load
// this file; only the tests, the smoke check and the benchmark's CPU-baseline
// leg use it. It shares no code with the HIP path.
//
// Source of every formula: "Mixture of Experts: Outrageously Large Neural
// Networks" (intuitivepapers.ai explainer of Shazeer et al., 2017), sections
// "How a mixture-of-experts layer works" (eq 1), "Noisy top-k gating"
// (eqs 2-5), "Why experts collapse, and the balancing losses" (eqs 6-7 and the
// coefficient of variation), "A differentiable count of examples" (eqs 8-11)
// and "Hierarchical MoE" (eq 12). Each function below evaluates one of those
// definitions directly: per token, the logits of eq 4, the kept set and
// softmax of eqs 3 and 5, the weighted expert sum of eq 1, P of eq 9; per
// batch, the sums of eqs 6 and 10 and the CV^2 of eqs 7 and 11.
//
// Arithmetic: every sum and transcendental in double precision. Inputs are the
// same rounded fp32 or bf16 values the GPU reads, widened exactly. Loops are
// plain; OpenMP splits only independent rows or experts, and every reduction
// over rows runs in a fixed block order, so results do not depend on the
// thread count.
//
// Readings where the pages are open (each also listed in the design notes):
//  * noise std = Softplus(x.W_noise) + noise_floor; the explainer's code
//    adds a floor of 0.01, eq 4 has none, so the floor is a parameter.
//  * Selection order: larger noisy logit first, equal logits -> lower expert
//    index first. The selection is decided on the logits rounded to fp32 (the
//    precision the GPU decides in) when decide_fp32 != 0; every value that is
//    returned (gates, thresholds, P) is computed from the fp64 logits.
//  * Threshold of eq 8: (k+1)-th largest logit if expert i is in the top k,
//    k-th largest otherwise; with k == n there is no (k+1)-th and P = 1.
//  * With train == 0 the noise is off, H = clean, and P(x, i) is the hard
//    indicator [i in top k] (the sigma -> 0 limit of eq 9).
//  * CV^2 uses the population variance (the worked example divides the sum of
//    squared deviations by the number of experts); CV^2 = 0 when n == 1 or
//    the mean is 0.
//  * An optional gate bias is added to the clean logit (so it enters H and the
//    numerator of eq 9 alike).
//  * Experts: E_i(x) = ReLU(x.W1_i + b1_i).W2_i + b2_i with optional biases.
//  * Hierarchical MoE (eq 12 is missing from the page; its prose is followed):
//    the primary gate picks k1 of a groups; for the r-th picked group i the
//    secondary gate of group i picks k2 of its b experts, with noise row
//    eps2[t][r][:]; leaf i*b + j gets gate G1_i * G2_ij, so each token uses
//    k1*k2 leaves. The pages give no balancing losses for the hierarchy; the
//    ones here are: leaf Importance = sum over tokens of the leaf gates; leaf
//    Load = Load1_i * Load2_ij / |X_i| (0 when |X_i| = 0), where Load1 is the
//    primary gate's Load over the batch, Load2_i the secondary gate's Load
//    over the rows X_i routed to group i; both reduce to the flat losses
//    when a = 1 or b = 1. Pinned at their limits only: those reductions, the
//    dense mixture's gate sums, and the hard leaf counts that the leaf Load
//    becomes at train = 0 and when the noise scale vanishes; between them the
//    product form is a reading, as no page defines the hierarchy's losses.
//
// Weight layouts: w_gate/w_noise [n][d] (row i = expert i), w1 [n][h][d]
// (row j = hidden unit j), w2 [n][d][h] (row c = output unit c). Hierarchical:
// primary gate [a][d], secondary gates [a][b][d], leaves as experts [a*b].
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <limits>
#include <numeric>
#include <vector>

#include <omp.h>

namespace {

constexpr int kF32 = 0;
constexpr int kBF16 = 1;
constexpr int64_t kRowBlock = 256;  // fixed reduction blocks over rows

inline double widen(const void* p, int64_t i, int dt) {
  if (dt == kF32) return (double)((const float*)p)[i];
  uint32_t u = (uint32_t)((const uint16_t*)p)[i] << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return (double)f;
}

// Widen a contiguous run [off, off+len) into dst.
void widen_run(const void* p, int64_t off, int64_t len, int dt, double* dst) {
  for (int64_t i = 0; i < len; ++i) dst[i] = widen(p, off + i, dt);
}

// Softplus(u) = log(1 + e^u), evaluated in the form that cannot overflow.
inline double softplus(double u) { return std::max(u, 0.0) + std::log1p(std::exp(-std::fabs(u))); }

// Standard normal CDF.
inline double Phi(double z) { return 0.5 * std::erfc(-z / std::sqrt(2.0)); }

struct GateArgs {
  int d, n, k;
  const void* x;
  int x_dt;
  const void* wg;
  const void* wn;
  int w_dt;
  const float* bg;   // [n] or null
  const float* eps;  // [B][n], or null when train == 0
  int64_t eps_row_stride;
  int train;
  double floor;
  int decide_fp32;
};

// Per-row gate state.
struct RowGate {
  std::vector<double> clean, sigma, H;
  std::vector<int> order;  // all n experts, best first
  std::vector<int> in_top; // 1 if expert is one of the k selected
  double vk = 0, vk1 = 0;  // k-th and (k+1)-th largest logits
  std::vector<double> gate;  // [k] in rank order
  explicit RowGate(int n) : clean(n), sigma(n), H(n), order(n), in_top(n) {}
};

// Eq 4 (noisy logits), then the keep-top-k of eqs 3/5 and the softmax over
// the kept logits, for token t.
void gate_row(const GateArgs& g, int64_t t, RowGate& r, std::vector<double>& xrow,
              std::vector<double>& wrow) {
  const int d = g.d, n = g.n, k = g.k;
  widen_run(g.x, t * (int64_t)d, d, g.x_dt, xrow.data());
  for (int i = 0; i < n; ++i) {
    // clean logit (x . W_g)_i (+ bias)
    widen_run(g.wg, (int64_t)i * d, d, g.w_dt, wrow.data());
    double c = 0.0;
    for (int j = 0; j < d; ++j) c += xrow[j] * wrow[j];
    if (g.bg) c += (double)g.bg[i];
    r.clean[i] = c;
    if (g.train) {
      widen_run(g.wn, (int64_t)i * d, d, g.w_dt, wrow.data());
      double u = 0.0;
      for (int j = 0; j < d; ++j) u += xrow[j] * wrow[j];
      double s = softplus(u) + g.floor;
      r.sigma[i] = s;
      r.H[i] = c + (double)g.eps[t * g.eps_row_stride + i] * s;
    } else {
      r.sigma[i] = 0.0;
      r.H[i] = c;
    }
  }
  // Rank the experts by noisy logit, larger first, ties to the lower index.
  std::iota(r.order.begin(), r.order.end(), 0);
  if (g.decide_fp32) {
    std::vector<float> key(n);
    for (int i = 0; i < n; ++i) key[i] = (float)r.H[i];
    std::stable_sort(r.order.begin(), r.order.end(), [&](int a, int b) { return key[a] > key[b]; });
  } else {
    std::stable_sort(r.order.begin(), r.order.end(), [&](int a, int b) { return r.H[a] > r.H[b]; });
  }
  std::fill(r.in_top.begin(), r.in_top.end(), 0);
  for (int j = 0; j < k; ++j) r.in_top[r.order[j]] = 1;
  r.vk = r.H[r.order[k - 1]];
  r.vk1 = (k < n) ? r.H[r.order[k]] : -std::numeric_limits<double>::infinity();
  // softmax over the kept logits (the others are -inf and get gate 0)
  r.gate.assign(k, 0.0);
  const double top = r.H[r.order[0]];
  double z = 0.0;
  for (int j = 0; j < k; ++j) {
    r.gate[j] = std::exp(r.H[r.order[j]] - top);
    z += r.gate[j];
  }
  for (int j = 0; j < k; ++j) r.gate[j] /= z;
}

// P(x, i) of eq 9: the probability that expert i is among the k largest
// logits under a fresh draw of its own noise, the other experts' noise held
// fixed (eq 8). The logit it has to beat is the k-th largest of the other
// experts' logits: v_{k+1} when i itself is one of the k kept, v_k otherwise.
inline double p_eq9(const GateArgs& g, const RowGate& r, int i) {
  if (!g.train) return r.in_top[i] ? 1.0 : 0.0;
  const double to_beat = r.in_top[i] ? r.vk1 : r.vk;
  return Phi((r.clean[i] - to_beat) / r.sigma[i]);
}

// E_i(x) for one token row: ReLU(W1_i x + b1_i), then W2_i . hidden + b2_i.
void expert_apply(int d, int h, const double* xrow, const void* w1, const void* b1,
                  const void* w2, const void* b2, int e_dt, int64_t e, double* out,
                  std::vector<double>& hid, std::vector<double>& wrow) {
  for (int j = 0; j < h; ++j) {
    widen_run(w1, (e * h + j) * (int64_t)d, d, e_dt, wrow.data());
    double a = 0.0;
    for (int c = 0; c < d; ++c) a += xrow[c] * wrow[c];
    if (b1) a += widen(b1, e * h + j, e_dt);
    hid[j] = a > 0.0 ? a : 0.0;
  }
  for (int c = 0; c < d; ++c) {
    widen_run(w2, (e * d + c) * (int64_t)h, h, e_dt, wrow.data());
    double a = 0.0;
    for (int j = 0; j < h; ++j) a += hid[j] * wrow[j];
    if (b2) a += widen(b2, e * d + c, e_dt);
    out[c] = a;
  }
}

// Squared coefficient of variation with the population variance.
double cv2(int n, const double* v) {
  if (n <= 1) return 0.0;
  double mean = 0.0;
  for (int i = 0; i < n; ++i) mean += v[i];
  mean /= n;
  if (mean == 0.0) return 0.0;
  double var = 0.0;
  for (int i = 0; i < n; ++i) var += (v[i] - mean) * (v[i] - mean);
  var /= n;
  return var / (mean * mean);
}

// ---------------------------------------------------------------------------
// Backward pass ("Implementation notes", the paragraph on which parameters
// receive gradients; "Noisy top-k gating", the k >= 2 paragraph; "Why experts
// collapse, and the balancing losses"; "A differentiable count of examples").
// Reading: the selection (which experts are kept) and the thresholds of eq 9
// (the k-th / (k+1)-th largest noisy logits, values the selection produces)
// are constants; gradients flow through the kept gates' softmax into their
// noisy logits, through the numerator (clean logit) and the denominator
// (noise scale) of eq 9, and through each kept expert's output.
// ---------------------------------------------------------------------------

// d CV^2(v) / d v_i for the population-variance CV^2: with mean m and
// variance V, (2 / (n m^2)) ((v_i - m) - V / m); 0 when n == 1 or m == 0
// (where CV^2 is defined as 0).
void cv2_grad(int n, const double* v, double* g) {
  if (n <= 1) {
    for (int i = 0; i < n; ++i) g[i] = 0.0;
    return;
  }
  double m = 0.0;
  for (int i = 0; i < n; ++i) m += v[i];
  m /= n;
  if (m == 0.0) {
    for (int i = 0; i < n; ++i) g[i] = 0.0;
    return;
  }
  double V = 0.0;
  for (int i = 0; i < n; ++i) V += (v[i] - m) * (v[i] - m);
  V /= n;
  for (int i = 0; i < n; ++i) g[i] = 2.0 / (n * m * m) * ((v[i] - m) - V / m);
}

// Backward of the softmax over the kept logits: gates g (k of them, summing
// to 1) and the gradient dg with respect to each gate give the gradient with
// respect to each kept logit, g_j (dg_j - sum_l g_l dg_l). Its diagonal is
// g_j (1 - g_j), the derivative of a gate by its own logit.
void kept_softmax_grad(int k, const double* g, const double* dg, double* dH) {
  double s = 0.0;
  for (int l = 0; l < k; ++l) s += g[l] * dg[l];
  for (int j = 0; j < k; ++j) dH[j] = g[j] * (dg[j] - s);
}

// Derivatives of eq 9's P = Phi((c - thr) / sigma) by the clean logit c and by
// the noise scale sigma (thr fixed): phi(z) / sigma and -phi(z) z / sigma,
// z = (c - thr) / sigma. With no threshold (thr = -inf, k == n) P is 1 and
// both are 0.
void p_eq9_grad(double c, double thr, double sigma, double* dc, double* dsigma) {
  if (std::isinf(thr)) {
    *dc = *dsigma = 0.0;
    return;
  }
  const double z = (c - thr) / sigma;
  const double ph = std::exp(-0.5 * z * z) / std::sqrt(2.0 * M_PI);
  *dc = ph / sigma;
  *dsigma = -ph * z / sigma;
}

// d Softplus(u) / du, the logistic function, in a form that cannot overflow.
inline double softplus_grad(double u) {
  return u >= 0.0 ? 1.0 / (1.0 + std::exp(-u)) : std::exp(u) / (1.0 + std::exp(u));
}

GateArgs make_args(int d, int n, int k, const void* x, int x_dt, const void* wg, const void* wn,
                   int w_dt, const float* bg, const float* eps, int train, double floor,
                   int decide_fp32) {
  GateArgs g;
  g.d = d; g.n = n; g.k = k; g.x = x; g.x_dt = x_dt; g.wg = wg; g.wn = wn; g.w_dt = w_dt;
  g.bg = bg; g.eps = eps; g.eps_row_stride = n; g.train = train; g.floor = floor;
  g.decide_fp32 = decide_fp32;
  return g;
}

bool bad_args(int64_t B, int d, int n, int k, int train, const void* eps) {
  return B < 0 || d < 1 || n < 1 || k < 1 || k > n || (train && !eps);
}

// Replaces the row's selection by a given set of k experts (in the given slot
// order) -- used to evaluate everything downstream of a selection another
// implementation made on a near-tie row. The order statistics v_k, v_{k+1} of
// the row's logits do not depend on the selection and are kept.
bool force_selection(RowGate& r, const int32_t* sel, int k, int n) {
  std::fill(r.in_top.begin(), r.in_top.end(), 0);
  for (int j = 0; j < k; ++j) {
    if (sel[j] < 0 || sel[j] >= n || r.in_top[sel[j]]) return false;
    r.in_top[sel[j]] = 1;
  }
  double top = r.H[sel[0]];
  for (int j = 1; j < k; ++j) top = std::max(top, r.H[sel[j]]);
  double z = 0.0;
  for (int j = 0; j < k; ++j) {
    r.order[j] = sel[j];
    r.gate[j] = std::exp(r.H[sel[j]] - top);
    z += r.gate[j];
  }
  for (int j = 0; j < k; ++j) r.gate[j] /= z;
  return true;
}

size_t dt_size(int dt) { return dt == kF32 ? 4 : 2; }

// Hierarchical MoE: both gate levels of one token.
struct HierArgs {
  GateArgs g1;         // primary gate over the a groups
  GateArgs g2;         // secondary gate template (weights of group 0, eps rank 0)
  int a, b, k1, k2;
  size_t w2_group;     // bytes of one group's [b][d] secondary gate weights
};

struct HierRow {
  RowGate r1;
  std::vector<RowGate> r2;  // [k1], the secondary gate of the r-th picked group
  HierRow(int a, int b, int k1) : r1(a), r2(k1, RowGate(b)) {}
};

HierArgs make_hier(int d, int a, int b, int k1, int k2, const void* x, int x_dt,
                   const void* wg1, const void* wn1, const void* wg2, const void* wn2, int w_dt,
                   const float* eps1, const float* eps2, int train, double floor,
                   int decide_fp32) {
  HierArgs h;
  h.g1 = make_args(d, a, k1, x, x_dt, wg1, wn1, w_dt, nullptr, eps1, train, floor, decide_fp32);
  h.g2 = make_args(d, b, k2, x, x_dt, wg2, wn2, w_dt, nullptr, eps2, train, floor, decide_fp32);
  h.g2.eps_row_stride = (int64_t)k1 * b;  // eps2 is [B][k1][b]
  h.a = a; h.b = b; h.k1 = k1; h.k2 = k2;
  h.w2_group = (size_t)b * d * dt_size(w_dt);
  return h;
}

// Primary gate of token t, then for each picked group (slot order r) the
// group's own gate with noise row eps2[t][r]. force1 [k1] / force2 [k1][k2]
// (either may be null) replace the selections.
bool hier_gate_row(const HierArgs& h, int64_t t, const int32_t* force1, const int32_t* force2,
                   HierRow& hr, std::vector<double>& xrow, std::vector<double>& wrow) {
  gate_row(h.g1, t, hr.r1, xrow, wrow);
  if (force1 && !force_selection(hr.r1, force1, h.k1, h.a)) return false;
  for (int r = 0; r < h.k1; ++r) {
    const int grp = hr.r1.order[r];
    GateArgs g2 = h.g2;
    g2.wg = (const char*)h.g2.wg + grp * h.w2_group;
    g2.wn = (const char*)h.g2.wn + grp * h.w2_group;
    if (g2.eps) g2.eps = h.g2.eps + (int64_t)r * h.b;
    gate_row(g2, t, hr.r2[r], xrow, wrow);
    if (force2 && !force_selection(hr.r2[r], force2 + r * h.k2, h.k2, h.b)) return false;
  }
  return true;
}

bool bad_hier(int64_t B, int d, int a, int b, int k1, int k2, int train, const void* eps1,
              const void* eps2) {
  return B < 0 || d < 1 || a < 1 || b < 1 || k1 < 1 || k1 > a || k2 < 1 || k2 > b ||
         (train && (!eps1 || !eps2));
}

}  // namespace

extern "C" {

int oracle_version(void) { return 1; }
int oracle_threads(void) { return omp_get_max_threads(); }
// Threads of the oracle's later parallel regions on the calling thread (the
// CPU baseline times it on one thread and on all host threads).
void oracle_set_threads(int n) { omp_set_num_threads(n > 0 ? n : 1); }

double oracle_softplus(double u) { return softplus(u); }
double oracle_phi(double z) { return Phi(z); }
double oracle_cv2(int n, const double* v) { return cv2(n, v); }

// Gating for a list of token rows (rows == null: rows 0..nrows-1).
// Outputs per listed row r (any may be null):
//   clean/sigma/H [nrows][n]; topk_idx [nrows][k] (rank order);
//   topk_gate [nrows][k]; thresh [nrows][2] = (k-th, (k+1)-th) largest logit.
int oracle_gate(int64_t nrows, const int64_t* rows, int d, int n, int k,
                const void* x, int x_dt, const void* wg, const void* wn, int w_dt,
                const float* bg, const float* eps, int train, double floor, int decide_fp32,
                double* clean, double* sigma, double* H,
                int32_t* topk_idx, double* topk_gate, double* thresh) {
  if (bad_args(nrows, d, n, k, train, eps)) return 1;
  const GateArgs g = make_args(d, n, k, x, x_dt, wg, wn, w_dt, bg, eps, train, floor, decide_fp32);
#pragma omp parallel
  {
    RowGate r(n);
    std::vector<double> xrow(d), wrow(d);
#pragma omp for schedule(dynamic, 16)
    for (int64_t q = 0; q < nrows; ++q) {
      const int64_t t = rows ? rows[q] : q;
      gate_row(g, t, r, xrow, wrow);
      if (clean) std::copy(r.clean.begin(), r.clean.end(), clean + q * n);
      if (sigma) std::copy(r.sigma.begin(), r.sigma.end(), sigma + q * n);
      if (H) std::copy(r.H.begin(), r.H.end(), H + q * n);
      for (int j = 0; j < k; ++j) {
        if (topk_idx) topk_idx[q * k + j] = r.order[j];
        if (topk_gate) topk_gate[q * k + j] = r.gate[j];
      }
      if (thresh) {
        thresh[q * 2 + 0] = r.vk;
        thresh[q * 2 + 1] = r.vk1;
      }
    }
  }
  return 0;
}

// Eqs 8-10 over the whole batch of B tokens: load[i] = sum_t P(x_t, i).
// Rows are summed in blocks of 256 in ascending order, then the blocks in
// ascending order.
int oracle_load(int64_t B, int d, int n, int k, const void* x, int x_dt, const void* wg,
                const void* wn, int w_dt, const float* bg, const float* eps, int train,
                double floor, int decide_fp32, double* load) {
  if (bad_args(B, d, n, k, train, eps)) return 1;
  const GateArgs g = make_args(d, n, k, x, x_dt, wg, wn, w_dt, bg, eps, train, floor, decide_fp32);
  const int64_t nblk = (B + kRowBlock - 1) / kRowBlock;
  std::vector<double> part((size_t)nblk * n, 0.0);
#pragma omp parallel
  {
    RowGate r(n);
    std::vector<double> xrow(d), wrow(d);
#pragma omp for schedule(dynamic, 1)
    for (int64_t b = 0; b < nblk; ++b) {
      double* acc = part.data() + b * n;
      for (int64_t t = b * kRowBlock; t < std::min(B, (b + 1) * kRowBlock); ++t) {
        gate_row(g, t, r, xrow, wrow);
        for (int i = 0; i < n; ++i) acc[i] += p_eq9(g, r, i);
      }
    }
  }
  for (int i = 0; i < n; ++i) load[i] = 0.0;
  for (int64_t b = 0; b < nblk; ++b)
    for (int i = 0; i < n; ++i) load[i] += part[b * n + i];
  return 0;
}

// Eq 1 for a list of token rows: y_t = sum over experts i in ascending index
// with G(x_t)_i > 0 of G(x_t)_i * E_i(x_t). y is [nrows][d].
int oracle_y_rows(int64_t nrows, const int64_t* rows, int d, int h, int n, int k,
                  const void* x, int x_dt, const void* wg, const void* wn, int w_dt,
                  const float* bg, const float* eps, int train, double floor, int decide_fp32,
                  const void* w1, const void* b1, const void* w2, const void* b2, int e_dt,
                  double* y) {
  if (bad_args(nrows, d, n, k, train, eps) || h < 1) return 1;
  const GateArgs g = make_args(d, n, k, x, x_dt, wg, wn, w_dt, bg, eps, train, floor, decide_fp32);
#pragma omp parallel
  {
    RowGate r(n);
    std::vector<double> xrow(d), wrow(std::max(d, h)), hid(h), eo(d);
#pragma omp for schedule(dynamic, 4)
    for (int64_t q = 0; q < nrows; ++q) {
      const int64_t t = rows ? rows[q] : q;
      gate_row(g, t, r, xrow, wrow);
      // dense gate row G(x_t), zero outside the top k
      std::vector<double> G(n, 0.0);
      for (int j = 0; j < k; ++j) G[r.order[j]] = r.gate[j];
      double* yr = y + q * d;
      for (int c = 0; c < d; ++c) yr[c] = 0.0;
      for (int i = 0; i < n; ++i) {
        if (G[i] == 0.0) continue;
        expert_apply(d, h, xrow.data(), w1, b1, w2, b2, e_dt, i, eo.data(), hid, wrow);
        for (int c = 0; c < d; ++c) yr[c] += G[i] * eo[c];
      }
    }
  }
  return 0;
}

// E_e(x_t) for a list of (token, expert) pairs; out is [npairs][d].
int oracle_expert_pairs(int64_t npairs, const int64_t* tokens, const int32_t* experts, int d,
                        int h, const void* x, int x_dt, const void* w1, const void* b1,
                        const void* w2, const void* b2, int e_dt, double* out) {
  if (npairs < 0 || d < 1 || h < 1) return 1;
#pragma omp parallel
  {
    std::vector<double> xrow(d), wrow(std::max(d, h)), hid(h);
#pragma omp for schedule(dynamic, 4)
    for (int64_t q = 0; q < npairs; ++q) {
      widen_run(x, tokens[q] * (int64_t)d, d, x_dt, xrow.data());
      expert_apply(d, h, xrow.data(), w1, b1, w2, b2, e_dt, experts[q], out + q * d, hid, wrow);
    }
  }
  return 0;
}

// Each expert's batch (eq 1 evaluates expert e only on the tokens whose gate
// for e is nonzero), in a fixed order: segment e lists the tokens that kept
// expert e, in ascending token order.
// Also Importance (eq 6): imp[e] = sum over those tokens of their gate.
//   counts [n], offsets [n+1], perm_token [B*k], perm_gate [B*k],
//   slot_pos [B*k] (slot_pos[t*k + j] = position of (t, j) in the permutation).
int oracle_route(int64_t B, int n, int k, const int32_t* topk_idx, const double* topk_gate,
                 int32_t* counts, int32_t* offsets, int32_t* perm_token, double* perm_gate,
                 int32_t* slot_pos, double* importance) {
  if (B < 0 || n < 1 || k < 1 || k > n) return 1;
  for (int64_t q = 0; q < B * k; ++q)
    if (topk_idx[q] < 0 || topk_idx[q] >= n) return 2;
  std::vector<int64_t> cnt(n, 0);
#pragma omp parallel for schedule(dynamic, 8)
  for (int e = 0; e < n; ++e) {
    int64_t c = 0;
    for (int64_t t = 0; t < B; ++t)
      for (int j = 0; j < k; ++j)
        if (topk_idx[t * k + j] == e) ++c;
    cnt[e] = c;
  }
  std::vector<int64_t> off(n + 1, 0);
  for (int e = 0; e < n; ++e) off[e + 1] = off[e] + cnt[e];
  for (int e = 0; e < n; ++e) {
    if (counts) counts[e] = (int32_t)cnt[e];
    if (offsets) offsets[e] = (int32_t)off[e];
  }
  if (offsets) offsets[n] = (int32_t)off[n];
#pragma omp parallel for schedule(dynamic, 8)
  for (int e = 0; e < n; ++e) {
    int64_t pos = off[e];
    double imp = 0.0;
    for (int64_t t = 0; t < B; ++t)
      for (int j = 0; j < k; ++j)
        if (topk_idx[t * k + j] == e) {
          if (perm_token) perm_token[pos] = (int32_t)t;
          if (perm_gate) perm_gate[pos] = topk_gate[t * k + j];
          if (slot_pos) slot_pos[t * k + j] = (int32_t)pos;
          imp += topk_gate[t * k + j];
          ++pos;
        }
    if (importance) importance[e] = imp;
  }
  return 0;
}

// The layer's forward pass on a batch of B tokens: eqs 3-5 per token, eq 1
// per token, eqs 6-7 and 9-11 over the batch.
// Outputs (any may be null except y):
//   y [B][d]; topk_idx/topk_gate [B][k]; thresh [B][2]; importance/load [n];
//   losses[3] = {CV^2(Importance), CV^2(Load), w_imp*CV^2(Imp) + w_load*CV^2(Load)}.
int oracle_forward(int64_t B, int d, int h, int n, int k, const void* x, int x_dt,
                   const void* wg, const void* wn, int w_dt, const float* bg, const float* eps,
                   int train, double floor, int decide_fp32, const void* w1, const void* b1,
                   const void* w2, const void* b2, int e_dt, double w_imp, double w_load,
                   double* y, int32_t* topk_idx_out, double* topk_gate_out, double* thresh_out,
                   double* importance, double* load, double* losses) {
  if (bad_args(B, d, n, k, train, eps) || h < 1 || !y) return 1;
  const GateArgs g = make_args(d, n, k, x, x_dt, wg, wn, w_dt, bg, eps, train, floor, decide_fp32);
  // Gating of every token (eqs 3-5) and its P(x_t, i) terms (eq 9).
  std::vector<int32_t> idx((size_t)B * k);
  std::vector<double> gate((size_t)B * k), thr((size_t)B * 2);
  std::vector<double> G((size_t)B * n, 0.0);
  const int64_t nblk = (B + kRowBlock - 1) / kRowBlock;
  std::vector<double> load_part((size_t)nblk * n, 0.0);
#pragma omp parallel
  {
    RowGate r(n);
    std::vector<double> xrow(d), wrow(d);
#pragma omp for schedule(dynamic, 1)
    for (int64_t b = 0; b < nblk; ++b) {
      for (int64_t t = b * kRowBlock; t < std::min(B, (b + 1) * kRowBlock); ++t) {
        gate_row(g, t, r, xrow, wrow);
        for (int j = 0; j < k; ++j) {
          idx[t * k + j] = r.order[j];
          gate[t * k + j] = r.gate[j];
          G[t * n + r.order[j]] = r.gate[j];
        }
        thr[t * 2] = r.vk;
        thr[t * 2 + 1] = r.vk1;
        // P(x_t, i) of eq 9, accumulated for eq 10 in this row block
        double* acc = load_part.data() + b * n;
        for (int i = 0; i < n; ++i) acc[i] += p_eq9(g, r, i);
      }
    }
  }
  // Eq 1 per token: y_t = sum of G(x_t)_i * E_i(x_t) over the experts with a
  // nonzero gate, in ascending expert index.
#pragma omp parallel
  {
    std::vector<double> xrow(d), wrow(std::max(d, h)), hid(h), eo(d);
#pragma omp for schedule(dynamic, 8)
    for (int64_t t = 0; t < B; ++t) {
      double* yr = y + t * d;
      for (int c = 0; c < d; ++c) yr[c] = 0.0;
      widen_run(x, t * (int64_t)d, d, x_dt, xrow.data());
      for (int i = 0; i < n; ++i) {
        const double gi = G[t * n + i];
        if (gi == 0.0) continue;
        expert_apply(d, h, xrow.data(), w1, b1, w2, b2, e_dt, i, eo.data(), hid, wrow);
        for (int c = 0; c < d; ++c) yr[c] += gi * eo[c];
      }
    }
  }
  // Importance (eq 6): column sums of G in ascending token order.
  std::vector<double> imp(n, 0.0), ld(n, 0.0);
  for (int64_t t = 0; t < B; ++t)
    for (int i = 0; i < n; ++i) imp[i] += G[t * n + i];
  // Load (eq 10): block partials in ascending block order.
  for (int64_t b = 0; b < nblk; ++b)
    for (int i = 0; i < n; ++i) ld[i] += load_part[b * n + i];
  const double cv_imp = cv2(n, imp.data());
  const double cv_load = cv2(n, ld.data());
  if (topk_idx_out) std::copy(idx.begin(), idx.end(), topk_idx_out);
  if (topk_gate_out) std::copy(gate.begin(), gate.end(), topk_gate_out);
  if (thresh_out) std::copy(thr.begin(), thr.end(), thresh_out);
  if (importance) std::copy(imp.begin(), imp.end(), importance);
  if (load) std::copy(ld.begin(), ld.end(), load);
  if (losses) {
    losses[0] = cv_imp;
    losses[1] = cv_load;
    losses[2] = w_imp * cv_imp + w_load * cv_load;  // eqs 7 and 11
  }
  return 0;
}

// Scalar objective of the backward pass's finite-difference check: with the
// selection fixed to force_idx [B][k] (rank order) and the thresholds of eq 9
// fixed to thresh_in [B][2] (the constants of the backward's reading), J =
// sum over t, c of dy[t][c] y[t][c] + aux_scale (w_imp CV^2(Importance) +
// w_load CV^2(Load)), y from eq 1 with the kept gates' softmax, Importance from
// eq 6 and Load from eqs 9-10 (hard counts when train == 0).
int oracle_objective(int64_t B, int d, int h, int n, int k, const void* x, int x_dt,
                     const void* wg, const void* wn, int w_dt, const float* bg, const float* eps,
                     int train, double floor, const void* w1, const void* b1, const void* w2,
                     const void* b2, int e_dt, double w_imp, double w_load, const double* dy,
                     double aux_scale, const int32_t* force_idx, const double* thresh_in,
                     double* J) {
  if (bad_args(B, d, n, k, train, eps) || h < 1 || !force_idx || !thresh_in || !dy || !J) return 1;
  const GateArgs g = make_args(d, n, k, x, x_dt, wg, wn, w_dt, bg, eps, train, floor, 1);
  std::vector<double> imp(n, 0.0), ld(n, 0.0);
  double task = 0.0;
  RowGate r(n);
  std::vector<double> xrow(d), wrow(std::max(d, h)), hid(h), eo(d);
  for (int64_t t = 0; t < B; ++t) {
    gate_row(g, t, r, xrow, wrow);
    if (!force_selection(r, force_idx + t * k, k, n)) return 3;
    r.vk = thresh_in[t * 2];
    r.vk1 = thresh_in[t * 2 + 1];
    for (int j = 0; j < k; ++j) {
      const int e = r.order[j];
      imp[e] += r.gate[j];
      expert_apply(d, h, xrow.data(), w1, b1, w2, b2, e_dt, e, eo.data(), hid, wrow);
      for (int c = 0; c < d; ++c) task += dy[t * d + c] * r.gate[j] * eo[c];
    }
    for (int i = 0; i < n; ++i) ld[i] += p_eq9(g, r, i);
  }
  *J = task + aux_scale * (w_imp * cv2(n, imp.data()) + w_load * cv2(n, ld.data()));
  return 0;
}

// Backward pass of the layer (reading in the comment above cv2_grad): the
// gradient of J = sum dy . y + aux_scale (w_imp CV^2(Importance) + w_load
// CV^2(Load)) with respect to the layer's input and parameters, the selection
// and the thresholds held fixed. force_idx [B][k] (null: the oracle's own
// selection) replaces the selection, as in oracle_gate's callers. Outputs
// (any may be null): dx [B][d]; dwg, dwn [n][d]; dbg [n]; dw1 [n][h][d];
// db1 [n][h]; dw2 [n][d][h]; db2 [n][d]. Sums over tokens run in ascending
// token order.
int oracle_backward(int64_t B, int d, int h, int n, int k, const void* x, int x_dt,
                    const void* wg, const void* wn, int w_dt, const float* bg, const float* eps,
                    int train, double floor, int decide_fp32, const void* w1, const void* b1,
                    const void* w2, const void* b2, int e_dt, double w_imp, double w_load,
                    const double* dy, double aux_scale, const int32_t* force_idx, double* dx,
                    double* dwg, double* dwn, double* dbg, double* dw1, double* db1, double* dw2,
                    double* db2) {
  if (bad_args(B, d, n, k, train, eps) || h < 1 || !dy) return 1;
  const GateArgs g = make_args(d, n, k, x, x_dt, wg, wn, w_dt, bg, eps, train, floor, decide_fp32);
  // Per token: the selection, gates and P terms (forward), then Importance and Load.
  std::vector<int32_t> sel((size_t)B * k);
  std::vector<double> gate((size_t)B * k), dgate((size_t)B * k), thr((size_t)B * 2);
  int bad = 0;
#pragma omp parallel
  {
    RowGate r(n);
    std::vector<double> xrow(d), wrow(std::max(d, h)), hid(h), eo(d);
#pragma omp for schedule(dynamic, 8) reduction(| : bad)
    for (int64_t t = 0; t < B; ++t) {
      gate_row(g, t, r, xrow, wrow);
      if (force_idx && !force_selection(r, force_idx + t * k, k, n)) {
        bad = 1;
        continue;
      }
      thr[t * 2] = r.vk;
      thr[t * 2 + 1] = r.vk1;
      for (int j = 0; j < k; ++j) {
        sel[t * k + j] = r.order[j];
        gate[t * k + j] = r.gate[j];
        // task part of dJ/dgate: dy_t . E_e(x_t)
        expert_apply(d, h, xrow.data(), w1, b1, w2, b2, e_dt, r.order[j], eo.data(), hid, wrow);
        double s = 0.0;
        for (int c = 0; c < d; ++c) s += dy[t * d + c] * eo[c];
        dgate[t * k + j] = s;
      }
    }
  }
  if (bad) return 3;
  std::vector<double> imp(n, 0.0), ld(n, 0.0), dimp(n), dld(n);
  for (int64_t t = 0; t < B; ++t)
    for (int j = 0; j < k; ++j) imp[sel[t * k + j]] += gate[t * k + j];
  if (train) {
    // Load (eq 10) with the same selection and thresholds, tokens in order
    RowGate r(n);
    std::vector<double> xrow(d), wrow(d);
    for (int64_t t = 0; t < B; ++t) {
      gate_row(g, t, r, xrow, wrow);
      force_selection(r, sel.data() + t * k, k, n);
      r.vk = thr[t * 2];
      r.vk1 = thr[t * 2 + 1];
      for (int i = 0; i < n; ++i) ld[i] += p_eq9(g, r, i);
    }
  }
  cv2_grad(n, imp.data(), dimp.data());
  cv2_grad(n, ld.data(), dld.data());
  for (int i = 0; i < n; ++i) {
    dimp[i] *= aux_scale * w_imp;
    dld[i] = train ? dld[i] * aux_scale * w_load : 0.0;  // hard counts carry no gradient
  }
  // Per (token, expert): gradients of the clean logit and of u = x . W_noise.
  std::vector<double> dC((size_t)B * n), dU((size_t)B * n);
#pragma omp parallel
  {
    RowGate r(n);
    std::vector<double> xrow(d), wrow(d), dg(k), dH(k);
#pragma omp for schedule(dynamic, 8)
    for (int64_t t = 0; t < B; ++t) {
      gate_row(g, t, r, xrow, wrow);
      force_selection(r, sel.data() + t * k, k, n);
      r.vk = thr[t * 2];
      r.vk1 = thr[t * 2 + 1];
      for (int j = 0; j < k; ++j) dg[j] = dgate[t * k + j] + dimp[sel[t * k + j]];
      kept_softmax_grad(k, gate.data() + t * k, dg.data(), dH.data());
      std::vector<double> dh_full(n, 0.0);
      for (int j = 0; j < k; ++j) dh_full[sel[t * k + j]] = dH[j];
      for (int i = 0; i < n; ++i) {
        double dc = dh_full[i];             // H = clean + eps * sigma: dH/dclean = 1
        double dsig = 0.0;
        if (train) {
          dsig = dh_full[i] * (double)g.eps[t * g.eps_row_stride + i];  // dH/dsigma = eps
          double pc, ps;
          p_eq9_grad(r.clean[i], r.in_top[i] ? r.vk1 : r.vk, r.sigma[i], &pc, &ps);
          dc += dld[i] * pc;
          dsig += dld[i] * ps;
        }
        dC[t * n + i] = dc;
        if (train) {
          // sigma = Softplus(u) + floor
          widen_run(g.wn, (int64_t)i * d, d, g.w_dt, wrow.data());
          double u = 0.0;
          for (int c = 0; c < d; ++c) u += xrow[c] * wrow[c];
          dU[t * n + i] = dsig * softplus_grad(u);
        } else {
          dU[t * n + i] = 0.0;
        }
      }
    }
  }
  // Gate parameters: dW_g[i] = sum_t dC[t][i] x_t, dW_noise likewise, db_g = sum_t dC.
#pragma omp parallel
  {
    std::vector<double> xrow(d);
#pragma omp for schedule(static)
    for (int i = 0; i < n; ++i) {
      std::vector<double> ag(d, 0.0), an(d, 0.0);
      double ab = 0.0;
      for (int64_t t = 0; t < B; ++t) {
        widen_run(x, t * (int64_t)d, d, x_dt, xrow.data());
        const double dc = dC[t * n + i], du = dU[t * n + i];
        for (int c = 0; c < d; ++c) {
          ag[c] += dc * xrow[c];
          an[c] += du * xrow[c];
        }
        ab += dc;
      }
      for (int c = 0; c < d; ++c) {
        if (dwg) dwg[(int64_t)i * d + c] = ag[c];
        if (dwn) dwn[(int64_t)i * d + c] = an[c];
      }
      if (dbg) dbg[i] = ab;
    }
  }
  // Experts: each from its routed rows only, scaled by their gates.
  // E(x) = ReLU(x.W1 + b1).W2 + b2 with dE = gate * dy_t.
  if (dw1 || db1 || dw2 || db2) {
#pragma omp parallel
    {
      std::vector<double> xrow(d), wrow(std::max(d, h)), pre(h), hid(h), dO(d), dA(h);
#pragma omp for schedule(dynamic, 1)
      for (int e = 0; e < n; ++e) {
        std::vector<double> gw1((size_t)h * d, 0.0), gb1(h, 0.0), gw2((size_t)d * h, 0.0),
            gb2(d, 0.0);
        for (int64_t t = 0; t < B; ++t) {
          int j = -1;
          for (int q = 0; q < k; ++q)
            if (sel[t * k + q] == e) j = q;
          if (j < 0) continue;
          widen_run(x, t * (int64_t)d, d, x_dt, xrow.data());
          for (int a = 0; a < h; ++a) {
            widen_run(w1, ((int64_t)e * h + a) * d, d, e_dt, wrow.data());
            double v = 0.0;
            for (int c = 0; c < d; ++c) v += xrow[c] * wrow[c];
            if (b1) v += widen(b1, (int64_t)e * h + a, e_dt);
            pre[a] = v;
            hid[a] = v > 0.0 ? v : 0.0;
          }
          for (int c = 0; c < d; ++c) dO[c] = gate[t * k + j] * dy[t * d + c];
          for (int a = 0; a < h; ++a) dA[a] = 0.0;
          for (int c = 0; c < d; ++c) {
            widen_run(w2, ((int64_t)e * d + c) * h, h, e_dt, wrow.data());
            for (int a = 0; a < h; ++a) {
              gw2[(size_t)c * h + a] += dO[c] * hid[a];
              dA[a] += dO[c] * wrow[a];
            }
            gb2[c] += dO[c];
          }
          for (int a = 0; a < h; ++a) {
            const double da = pre[a] > 0.0 ? dA[a] : 0.0;
            gb1[a] += da;
            for (int c = 0; c < d; ++c) gw1[(size_t)a * d + c] += da * xrow[c];
          }
        }
        if (dw1) std::copy(gw1.begin(), gw1.end(), dw1 + (int64_t)e * h * d);
        if (db1) std::copy(gb1.begin(), gb1.end(), db1 + (int64_t)e * h);
        if (dw2) std::copy(gw2.begin(), gw2.end(), dw2 + (int64_t)e * d * h);
        if (db2) std::copy(gb2.begin(), gb2.end(), db2 + (int64_t)e * d);
      }
    }
  }
  // The input: through the gate logits and through each kept expert.
  if (dx) {
#pragma omp parallel
    {
      std::vector<double> xrow(d), wrow(std::max(d, h)), pre(h), dA(h), acc(d);
#pragma omp for schedule(dynamic, 8)
      for (int64_t t = 0; t < B; ++t) {
        widen_run(x, t * (int64_t)d, d, x_dt, xrow.data());
        for (int c = 0; c < d; ++c) acc[c] = 0.0;
        for (int i = 0; i < n; ++i) {
          widen_run(g.wg, (int64_t)i * d, d, g.w_dt, wrow.data());
          for (int c = 0; c < d; ++c) acc[c] += dC[t * n + i] * wrow[c];
          if (train) {
            widen_run(g.wn, (int64_t)i * d, d, g.w_dt, wrow.data());
            for (int c = 0; c < d; ++c) acc[c] += dU[t * n + i] * wrow[c];
          }
        }
        for (int j = 0; j < k; ++j) {
          const int e = sel[t * k + j];
          for (int a = 0; a < h; ++a) {
            widen_run(w1, ((int64_t)e * h + a) * d, d, e_dt, wrow.data());
            double v = 0.0;
            for (int c = 0; c < d; ++c) v += xrow[c] * wrow[c];
            if (b1) v += widen(b1, (int64_t)e * h + a, e_dt);
            pre[a] = v;
            dA[a] = 0.0;
          }
          for (int c = 0; c < d; ++c) {
            widen_run(w2, ((int64_t)e * d + c) * h, h, e_dt, wrow.data());
            const double dO = gate[t * k + j] * dy[t * d + c];
            for (int a = 0; a < h; ++a) dA[a] += dO * wrow[a];
          }
          for (int a = 0; a < h; ++a) {
            if (pre[a] <= 0.0) continue;
            widen_run(w1, ((int64_t)e * h + a) * d, d, e_dt, wrow.data());
            for (int c = 0; c < d; ++c) acc[c] += dA[a] * wrow[c];
          }
        }
        for (int c = 0; c < d; ++c) dx[t * d + c] = acc[c];
      }
    }
  }
  return 0;
}

// The same gradients for a few experts and tokens, for batches too large for
// oracle_backward. One pass over all tokens gives the selection (or the forced
// one), gates, thresholds, Importance and Load (eqs 6, 8-10; Load summed in
// fixed blocks of rows) and the clean logits and noise pre-activations of the
// gate-sampled experts; the kept gates' gradients (the task part dy . E and the
// Importance part, through the kept softmax) are formed only for the tokens
// that need them. Outputs (any may be null):
//   gate experts ge[q] (q < ng): dwg [ng][d], dwn [ng][d], dbg [ng]
//   experts ee[q] (q < ne): dw1 [ne][h][d], db1 [ne][h], dw2 [ne][d][h], db2 [ne][d]
//   tokens tt[q] (q < nt): dx [nt][d]
int oracle_backward_sampled(int64_t B, int d, int h, int n, int k, const void* x, int x_dt,
                            const void* wg, const void* wn, int w_dt, const float* bg,
                            const float* eps, int train, double floor, int decide_fp32,
                            const void* w1, const void* b1, const void* w2, const void* b2,
                            int e_dt, double w_imp, double w_load, const double* dy,
                            double aux_scale, const int32_t* force_idx, int ng, const int32_t* ge,
                            double* dwg, double* dwn, double* dbg, int ne, const int32_t* ee,
                            double* dw1, double* db1, double* dw2, double* db2, int nt,
                            const int64_t* tt, double* dx) {
  if (bad_args(B, d, n, k, train, eps) || h < 1 || !dy || ng < 0 || ne < 0 || nt < 0) return 1;
  for (int q = 0; q < ng; ++q)
    if (ge[q] < 0 || ge[q] >= n) return 1;
  for (int q = 0; q < ne; ++q)
    if (ee[q] < 0 || ee[q] >= n) return 1;
  for (int q = 0; q < nt; ++q)
    if (tt[q] < 0 || tt[q] >= B) return 1;
  const GateArgs g = make_args(d, n, k, x, x_dt, wg, wn, w_dt, bg, eps, train, floor, decide_fp32);
  std::vector<int32_t> sel((size_t)B * k);
  std::vector<double> gate((size_t)B * k), thr((size_t)B * 2);
  std::vector<double> gc((size_t)B * ng), gu((size_t)B * ng);  // clean logit, u of gate experts
  const int64_t nblk = (B + kRowBlock - 1) / kRowBlock;
  std::vector<double> ldblk((size_t)nblk * n, 0.0);
  int bad = 0;
#pragma omp parallel
  {
    RowGate r(n);
    std::vector<double> xrow(d), wrow(d);
#pragma omp for schedule(dynamic, 1) reduction(| : bad)
    for (int64_t blk = 0; blk < nblk; ++blk) {
      double* lb = ldblk.data() + blk * n;
      for (int64_t t = blk * kRowBlock; t < std::min(B, (blk + 1) * kRowBlock); ++t) {
        gate_row(g, t, r, xrow, wrow);
        if (force_idx && !force_selection(r, force_idx + t * k, k, n)) {
          bad = 1;
          continue;
        }
        thr[t * 2] = r.vk;
        thr[t * 2 + 1] = r.vk1;
        for (int j = 0; j < k; ++j) {
          sel[t * k + j] = r.order[j];
          gate[t * k + j] = r.gate[j];
        }
        if (train)
          for (int i = 0; i < n; ++i) lb[i] += p_eq9(g, r, i);
        for (int q = 0; q < ng; ++q) {
          const int i = ge[q];
          gc[t * ng + q] = r.clean[i];
          double u = 0.0;
          if (train) {
            widen_run(g.wn, (int64_t)i * d, d, g.w_dt, wrow.data());
            for (int c = 0; c < d; ++c) u += xrow[c] * wrow[c];
          }
          gu[t * ng + q] = u;
        }
      }
    }
  }
  if (bad) return 3;
  std::vector<double> imp(n, 0.0), ld(n, 0.0), dimp(n), dld(n);
  for (int64_t t = 0; t < B; ++t)
    for (int j = 0; j < k; ++j) imp[sel[t * k + j]] += gate[t * k + j];
  for (int64_t blk = 0; blk < nblk; ++blk)
    for (int i = 0; i < n; ++i) ld[i] += ldblk[blk * n + i];
  cv2_grad(n, imp.data(), dimp.data());
  cv2_grad(n, ld.data(), dld.data());
  for (int i = 0; i < n; ++i) {
    dimp[i] *= aux_scale * w_imp;
    dld[i] = train ? dld[i] * aux_scale * w_load : 0.0;
  }
  // The tokens whose kept gates' gradients are needed: the sampled tokens and
  // every token that keeps a gate-sampled expert.
  std::vector<char> need(B, 0);
  for (int q = 0; q < nt; ++q) need[tt[q]] = 1;
  if (ng > 0) {
    std::vector<char> isg(n, 0);
    for (int q = 0; q < ng; ++q) isg[ge[q]] = 1;
    for (int64_t t = 0; t < B; ++t)
      for (int j = 0; j < k; ++j)
        if (isg[sel[t * k + j]]) need[t] = 1;
  }
  std::vector<double> dHk((size_t)B * k, 0.0);
#pragma omp parallel
  {
    std::vector<double> xrow(d), wrow(std::max(d, h)), hid(h), eo(d), dg(k), dH(k);
#pragma omp for schedule(dynamic, 8)
    for (int64_t t = 0; t < B; ++t) {
      if (!need[t]) continue;
      widen_run(x, t * (int64_t)d, d, x_dt, xrow.data());
      for (int j = 0; j < k; ++j) {
        const int e = sel[t * k + j];
        expert_apply(d, h, xrow.data(), w1, b1, w2, b2, e_dt, e, eo.data(), hid, wrow);
        double sdy = 0.0;
        for (int c = 0; c < d; ++c) sdy += dy[t * d + c] * eo[c];
        dg[j] = sdy + dimp[e];
      }
      kept_softmax_grad(k, gate.data() + t * k, dg.data(), dH.data());
      for (int j = 0; j < k; ++j) dHk[t * k + j] = dH[j];
    }
  }
  // d (loss) / d (clean logit) and / d (u) of token t, expert i (clean c, u given)
  auto pair_grads = [&](int64_t t, int i, double c, double u, double* dc, double* du) {
    double dh = 0.0;
    bool kept = false;
    for (int j = 0; j < k; ++j)
      if (sel[t * k + j] == i) {
        kept = true;
        dh = dHk[t * k + j];
      }
    *dc = dh;
    *du = 0.0;
    if (!train) return;
    const double sigma = softplus(u) + floor;
    double pc, ps;
    p_eq9_grad(c, kept ? thr[t * 2 + 1] : thr[t * 2], sigma, &pc, &ps);
    *dc += dld[i] * pc;
    const double dsig = dh * (double)eps[t * n + i] + dld[i] * ps;
    *du = dsig * softplus_grad(u);
  };
  // Gate experts: dW_g[i] = sum_t dC[t][i] x_t, dW_noise[i] likewise, db_g[i] = sum_t dC[t][i].
#pragma omp parallel
  {
    std::vector<double> xrow(d);
#pragma omp for schedule(dynamic, 1)
    for (int q = 0; q < ng; ++q) {
      const int i = ge[q];
      std::vector<double> ag(d, 0.0), an(d, 0.0);
      double ab = 0.0;
      for (int64_t t = 0; t < B; ++t) {
        double dc, du;
        pair_grads(t, i, gc[t * ng + q], gu[t * ng + q], &dc, &du);
        widen_run(x, t * (int64_t)d, d, x_dt, xrow.data());
        for (int c = 0; c < d; ++c) {
          ag[c] += dc * xrow[c];
          an[c] += du * xrow[c];
        }
        ab += dc;
      }
      for (int c = 0; c < d; ++c) {
        if (dwg) dwg[(int64_t)q * d + c] = ag[c];
        if (dwn) dwn[(int64_t)q * d + c] = an[c];
      }
      if (dbg) dbg[q] = ab;
    }
  }
  // Sampled experts: each from its routed rows only, scaled by their gates.
#pragma omp parallel
  {
    std::vector<double> xrow(d), wrow(std::max(d, h)), pre(h), hid(h), dO(d), dA(h);
#pragma omp for schedule(dynamic, 1)
    for (int q = 0; q < ne; ++q) {
      const int e = ee[q];
      std::vector<double> gw1((size_t)h * d, 0.0), gb1(h, 0.0), gw2((size_t)d * h, 0.0), gb2(d, 0.0);
      for (int64_t t = 0; t < B; ++t) {
        int j = -1;
        for (int s2 = 0; s2 < k; ++s2)
          if (sel[t * k + s2] == e) j = s2;
        if (j < 0) continue;
        widen_run(x, t * (int64_t)d, d, x_dt, xrow.data());
        for (int a = 0; a < h; ++a) {
          widen_run(w1, ((int64_t)e * h + a) * d, d, e_dt, wrow.data());
          double v = 0.0;
          for (int c = 0; c < d; ++c) v += xrow[c] * wrow[c];
          if (b1) v += widen(b1, (int64_t)e * h + a, e_dt);
          pre[a] = v;
          hid[a] = v > 0.0 ? v : 0.0;
          dA[a] = 0.0;
        }
        for (int c = 0; c < d; ++c) dO[c] = gate[t * k + j] * dy[t * d + c];
        for (int c = 0; c < d; ++c) {
          widen_run(w2, ((int64_t)e * d + c) * h, h, e_dt, wrow.data());
          for (int a = 0; a < h; ++a) {
            gw2[(size_t)c * h + a] += dO[c] * hid[a];
            dA[a] += dO[c] * wrow[a];
          }
          gb2[c] += dO[c];
        }
        for (int a = 0; a < h; ++a) {
          const double da = pre[a] > 0.0 ? dA[a] : 0.0;
          gb1[a] += da;
          for (int c = 0; c < d; ++c) gw1[(size_t)a * d + c] += da * xrow[c];
        }
      }
      if (dw1) std::copy(gw1.begin(), gw1.end(), dw1 + (int64_t)q * h * d);
      if (db1) std::copy(gb1.begin(), gb1.end(), db1 + (int64_t)q * h);
      if (dw2) std::copy(gw2.begin(), gw2.end(), dw2 + (int64_t)q * d * h);
      if (db2) std::copy(gb2.begin(), gb2.end(), db2 + (int64_t)q * d);
    }
  }
  // Sampled tokens: dx through every expert's clean logit and u, and through
  // each kept expert.
  if (dx) {
#pragma omp parallel
    {
      RowGate r(n);
      std::vector<double> xrow(d), wrow(std::max(d, h)), pre(h), dA(h), acc(d), wgr(d), wnr(d);
#pragma omp for schedule(dynamic, 1)
      for (int q = 0; q < nt; ++q) {
        const int64_t t = tt[q];
        widen_run(x, t * (int64_t)d, d, x_dt, xrow.data());
        for (int c = 0; c < d; ++c) acc[c] = 0.0;
        for (int i = 0; i < n; ++i) {
          widen_run(g.wg, (int64_t)i * d, d, g.w_dt, wgr.data());
          double c0 = 0.0, u = 0.0;
          for (int c = 0; c < d; ++c) c0 += xrow[c] * wgr[c];
          if (g.bg) c0 += (double)g.bg[i];
          if (train) {
            widen_run(g.wn, (int64_t)i * d, d, g.w_dt, wnr.data());
            for (int c = 0; c < d; ++c) u += xrow[c] * wnr[c];
          }
          double dc, du;
          pair_grads(t, i, c0, u, &dc, &du);
          for (int c = 0; c < d; ++c) acc[c] += dc * wgr[c];
          if (train)
            for (int c = 0; c < d; ++c) acc[c] += du * wnr[c];
        }
        for (int j = 0; j < k; ++j) {
          const int e = sel[t * k + j];
          for (int a = 0; a < h; ++a) {
            widen_run(w1, ((int64_t)e * h + a) * d, d, e_dt, wrow.data());
            double v = 0.0;
            for (int c = 0; c < d; ++c) v += xrow[c] * wrow[c];
            if (b1) v += widen(b1, (int64_t)e * h + a, e_dt);
            pre[a] = v;
            dA[a] = 0.0;
          }
          for (int c = 0; c < d; ++c) {
            widen_run(w2, ((int64_t)e * d + c) * h, h, e_dt, wrow.data());
            const double dO = gate[t * k + j] * dy[t * d + c];
            for (int a = 0; a < h; ++a) dA[a] += dO * wrow[a];
          }
          for (int a = 0; a < h; ++a) {
            if (pre[a] <= 0.0) continue;
            widen_run(w1, ((int64_t)e * h + a) * d, d, e_dt, wrow.data());
            for (int c = 0; c < d; ++c) acc[c] += dA[a] * wrow[c];
          }
        }
        for (int c = 0; c < d; ++c) dx[(int64_t)q * d + c] = acc[c];
      }
    }
  }
  return 0;
}

// The backward's pieces on their own, for their pins.
void oracle_cv2_grad(int n, const double* v, double* g) { cv2_grad(n, v, g); }
void oracle_kept_softmax_grad(int k, const double* g, const double* dg, double* dH) {
  kept_softmax_grad(k, g, dg, dH);
}
void oracle_p_eq9_grad(double c, double thr, double sigma, double* dc, double* dsigma) {
  p_eq9_grad(c, thr, sigma, dc, dsigma);
}

// Hierarchical gating ("Hierarchical MoE") for a list of token rows (rows ==
// null: 0..nrows-1). force1 [nrows][k1] / force2 [nrows][k1][k2] may be null.
// Outputs per listed row q (any may be null):
//   sel1/gate1 [k1], thr1 [2], H1 [a]; sel2/gate2 [k1][k2] (expert index within
//   the group), thr2 [k1][2], H2 [k1][b]; leaf_idx/leaf_gate [k1*k2] in slot
//   order (r, j): leaf sel1[r]*b + sel2[r][j], gate gate1[r]*gate2[r][j].
int oracle_hier_gate(int64_t nrows, const int64_t* rows, int d, int a, int b, int k1, int k2,
                     const void* x, int x_dt, const void* wg1, const void* wn1, const void* wg2,
                     const void* wn2, int w_dt, const float* eps1, const float* eps2, int train,
                     double floor, int decide_fp32, const int32_t* force1, const int32_t* force2,
                     int32_t* sel1, double* gate1, double* thr1, double* H1, int32_t* sel2,
                     double* gate2, double* thr2, double* H2, int32_t* leaf_idx,
                     double* leaf_gate) {
  if (nrows < 0 || bad_hier(nrows, d, a, b, k1, k2, train, eps1, eps2)) return 1;
  const HierArgs h = make_hier(d, a, b, k1, k2, x, x_dt, wg1, wn1, wg2, wn2, w_dt, eps1, eps2,
                               train, floor, decide_fp32);
  const int K = k1 * k2;
  int bad = 0;
#pragma omp parallel
  {
    HierRow hr(a, b, k1);
    std::vector<double> xrow(d), wrow(d);
#pragma omp for schedule(dynamic, 16) reduction(| : bad)
    for (int64_t q = 0; q < nrows; ++q) {
      const int64_t t = rows ? rows[q] : q;
      if (!hier_gate_row(h, t, force1 ? force1 + q * k1 : nullptr,
                         force2 ? force2 + q * K : nullptr, hr, xrow, wrow)) {
        bad = 1;
        continue;
      }
      for (int r = 0; r < k1; ++r) {
        if (sel1) sel1[q * k1 + r] = hr.r1.order[r];
        if (gate1) gate1[q * k1 + r] = hr.r1.gate[r];
        const RowGate& g2 = hr.r2[r];
        for (int j = 0; j < k2; ++j) {
          const int64_t o = q * K + r * k2 + j;
          if (sel2) sel2[o] = g2.order[j];
          if (gate2) gate2[o] = g2.gate[j];
          if (leaf_idx) leaf_idx[o] = hr.r1.order[r] * b + g2.order[j];
          if (leaf_gate) leaf_gate[o] = hr.r1.gate[r] * g2.gate[j];
        }
        if (thr2) {
          thr2[(q * k1 + r) * 2] = g2.vk;
          thr2[(q * k1 + r) * 2 + 1] = g2.vk1;
        }
        if (H2) std::copy(g2.H.begin(), g2.H.end(), H2 + (q * k1 + r) * b);
      }
      if (thr1) {
        thr1[q * 2] = hr.r1.vk;
        thr1[q * 2 + 1] = hr.r1.vk1;
      }
      if (H1) std::copy(hr.r1.H.begin(), hr.r1.H.end(), H1 + q * a);
    }
  }
  return bad ? 3 : 0;
}

// The hierarchical layer's forward pass on a batch of B tokens (eq 12 read
// from the prose; losses as in the header). force1/force2 as in
// oracle_hier_gate (null: the oracle's own selections). Outputs (any may be
// null; with y null the experts are not evaluated and w1/w2 may be null),
// n = a*b leaves:
//   y [B][d]; leaf_idx/leaf_gate [B][k1*k2];
//   imp1/load1 [a] (primary gate's Importance and Load), rows1 [a] = |X_i|;
//   load2 [a*b] (secondary Load of group i over X_i, at i*b + j);
//   importance/load [n] (leaf); losses[3] = {CV^2(Imp), CV^2(Load), weighted sum}.
int oracle_hier_forward(int64_t B, int d, int h, int a, int b, int k1, int k2, const void* x,
                        int x_dt, const void* wg1, const void* wn1, const void* wg2,
                        const void* wn2, int w_dt, const float* eps1, const float* eps2,
                        int train, double floor, int decide_fp32, const int32_t* force1,
                        const int32_t* force2, const void* w1, const void* b1, const void* w2,
                        const void* b2, int e_dt, double w_imp, double w_load, double* y,
                        int32_t* leaf_idx, double* leaf_gate, double* imp1, double* load1,
                        double* rows1, double* load2, double* importance, double* load,
                        double* losses) {
  if (bad_hier(B, d, a, b, k1, k2, train, eps1, eps2) || (y && (h < 1 || !w1 || !w2))) return 1;
  const HierArgs ha = make_hier(d, a, b, k1, k2, x, x_dt, wg1, wn1, wg2, wn2, w_dt, eps1, eps2,
                                train, floor, decide_fp32);
  const int K = k1 * k2;
  const int n = a * b;
  std::vector<int32_t> idx((size_t)B * K);
  std::vector<double> gate((size_t)B * K), g1((size_t)B * k1);
  std::vector<int32_t> s1((size_t)B * k1);
  const int64_t nblk = (B + kRowBlock - 1) / kRowBlock;
  std::vector<double> l1_part((size_t)nblk * a, 0.0), l2_part((size_t)nblk * n, 0.0);
  int bad = 0;
#pragma omp parallel
  {
    HierRow hr(a, b, k1);
    std::vector<double> xrow(d), wrow(d);
#pragma omp for schedule(dynamic, 1) reduction(| : bad)
    for (int64_t blk = 0; blk < nblk; ++blk) {
      double* acc1 = l1_part.data() + blk * a;
      double* acc2 = l2_part.data() + blk * n;
      for (int64_t t = blk * kRowBlock; t < std::min(B, (blk + 1) * kRowBlock); ++t) {
        if (!hier_gate_row(ha, t, force1 ? force1 + t * k1 : nullptr,
                           force2 ? force2 + t * K : nullptr, hr, xrow, wrow)) {
          bad = 1;
          continue;
        }
        for (int i = 0; i < a; ++i) acc1[i] += p_eq9(ha.g1, hr.r1, i);
        for (int r = 0; r < k1; ++r) {
          const int grp = hr.r1.order[r];
          s1[t * k1 + r] = grp;
          g1[t * k1 + r] = hr.r1.gate[r];
          // the secondary gate of group grp sees this token as one of X_grp
          for (int j = 0; j < b; ++j) acc2[grp * b + j] += p_eq9(ha.g2, hr.r2[r], j);
          for (int j = 0; j < k2; ++j) {
            idx[t * K + r * k2 + j] = grp * b + hr.r2[r].order[j];
            gate[t * K + r * k2 + j] = hr.r1.gate[r] * hr.r2[r].gate[j];
          }
        }
      }
    }
  }
  if (bad) return 3;
  // eq 12: y_t = sum over the token's leaves, ascending leaf id, of gate * E_leaf(x_t)
#pragma omp parallel if (y != nullptr)
  if (y) {
    std::vector<double> xrow(d), wrow(std::max(d, h)), hid(h), eo(d);
    std::vector<std::pair<int32_t, double>> lv(K);
#pragma omp for schedule(dynamic, 4)
    for (int64_t t = 0; t < B; ++t) {
      for (int j = 0; j < K; ++j) lv[j] = {idx[t * K + j], gate[t * K + j]};
      std::sort(lv.begin(), lv.end());
      widen_run(x, t * (int64_t)d, d, x_dt, xrow.data());
      double* yr = y + t * d;
      for (int c = 0; c < d; ++c) yr[c] = 0.0;
      for (int j = 0; j < K; ++j) {
        expert_apply(d, h, xrow.data(), w1, b1, w2, b2, e_dt, lv[j].first, eo.data(), hid, wrow);
        for (int c = 0; c < d; ++c) yr[c] += lv[j].second * eo[c];
      }
    }
  }
  // batch sums in ascending token / block order
  std::vector<double> i1(a, 0.0), l1(a, 0.0), r1(a, 0.0), l2(n, 0.0), imp(n, 0.0), ld(n, 0.0);
  for (int64_t t = 0; t < B; ++t) {
    for (int r = 0; r < k1; ++r) {
      i1[s1[t * k1 + r]] += g1[t * k1 + r];
      r1[s1[t * k1 + r]] += 1.0;
    }
    for (int j = 0; j < K; ++j) imp[idx[t * K + j]] += gate[t * K + j];
  }
  for (int64_t blk = 0; blk < nblk; ++blk) {
    for (int i = 0; i < a; ++i) l1[i] += l1_part[blk * a + i];
    for (int e = 0; e < n; ++e) l2[e] += l2_part[blk * n + e];
  }
  for (int i = 0; i < a; ++i)
    for (int j = 0; j < b; ++j)
      ld[i * b + j] = r1[i] > 0.0 ? l1[i] * l2[i * b + j] / r1[i] : 0.0;
  const double cv_imp = cv2(n, imp.data());
  const double cv_load = cv2(n, ld.data());
  if (leaf_idx) std::copy(idx.begin(), idx.end(), leaf_idx);
  if (leaf_gate) std::copy(gate.begin(), gate.end(), leaf_gate);
  if (imp1) std::copy(i1.begin(), i1.end(), imp1);
  if (load1) std::copy(l1.begin(), l1.end(), load1);
  if (rows1) std::copy(r1.begin(), r1.end(), rows1);
  if (load2) std::copy(l2.begin(), l2.end(), load2);
  if (importance) std::copy(imp.begin(), imp.end(), importance);
  if (load) std::copy(ld.begin(), ld.end(), load);
  if (losses) {
    losses[0] = cv_imp;
    losses[1] = cv_load;
    losses[2] = w_imp * cv_imp + w_load * cv_load;
  }
  return 0;
}

}  // extern "C"
