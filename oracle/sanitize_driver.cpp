// Test infrastructure: a stand-alone driver that runs every entry point of the
// oracle and of the seeded input generator on small inputs, for a build with
// AddressSanitizer and UndefinedBehaviorSanitizer (tests/test_sanitizers.py).
// It checks nothing of the method; the sanitizers check every access and
// every operation along the way, and the driver checks that each call
// accepts its arguments and leaves finite outputs. Exit status 0 on success.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <vector>

extern "C" {
int dg_normal(uint32_t seed, uint32_t tid, uint64_t offset, uint64_t count, double scale, int dtype,
              void* out);
void dg_f32_to_bf16(const float* in, uint16_t* out, uint64_t count);
int oracle_gate(int64_t, const int64_t*, int, int, int, const void*, int, const void*, const void*,
                int, const float*, const float*, int, double, int, double*, double*, double*,
                int32_t*, double*, double*);
int oracle_load(int64_t, int, int, int, const void*, int, const void*, const void*, int,
                const float*, const float*, int, double, int, double*);
int oracle_y_rows(int64_t, const int64_t*, int, int, int, int, const void*, int, const void*,
                  const void*, int, const float*, const float*, int, double, int, const void*,
                  const void*, const void*, const void*, int, double*);
int oracle_expert_pairs(int64_t, const int64_t*, const int32_t*, int, int, const void*, int,
                        const void*, const void*, const void*, const void*, int, double*);
int oracle_route(int64_t, int, int, const int32_t*, const double*, int32_t*, int32_t*, int32_t*,
                 double*, int32_t*, double*);
int oracle_forward(int64_t, int, int, int, int, const void*, int, const void*, const void*, int,
                   const float*, const float*, int, double, int, const void*, const void*,
                   const void*, const void*, int, double, double, double*, int32_t*, double*,
                   double*, double*, double*, double*);
int oracle_objective(int64_t, int, int, int, int, const void*, int, const void*, const void*, int,
                     const float*, const float*, int, double, const void*, const void*,
                     const void*, const void*, int, double, double, const double*, double,
                     const int32_t*, const double*, double*);
int oracle_backward(int64_t, int, int, int, int, const void*, int, const void*, const void*, int,
                    const float*, const float*, int, double, int, const void*, const void*,
                    const void*, const void*, int, double, double, const double*, double,
                    const int32_t*, double*, double*, double*, double*, double*, double*, double*,
                    double*);
int oracle_backward_sampled(int64_t, int, int, int, int, const void*, int, const void*,
                            const void*, int, const float*, const float*, int, double, int,
                            const void*, const void*, const void*, const void*, int, double, double,
                            const double*, double, const int32_t*, int, const int32_t*, double*,
                            double*, double*, int, const int32_t*, double*, double*, double*,
                            double*, int, const int64_t*, double*);
int oracle_hier_gate(int64_t, const int64_t*, int, int, int, int, int, const void*, int,
                     const void*, const void*, const void*, const void*, int, const float*,
                     const float*, int, double, int, const int32_t*, const int32_t*, int32_t*,
                     double*, double*, double*, int32_t*, double*, double*, double*, int32_t*,
                     double*);
int oracle_hier_forward(int64_t, int, int, int, int, int, int, const void*, int, const void*,
                        const void*, const void*, const void*, int, const float*, const float*,
                        int, double, int, const int32_t*, const int32_t*, const void*,
                        const void*, const void*, const void*, int, double, double, double*,
                        int32_t*, double*, double*, double*, double*, double*, double*, double*,
                        double*);
void oracle_cv2_grad(int, const double*, double*);
void oracle_kept_softmax_grad(int, const double*, const double*, double*);
void oracle_p_eq9_grad(double, double, double, double*, double*);
}

namespace {

int failures = 0;

void expect(bool ok, const char* what) {
  if (!ok) {
    std::fprintf(stderr, "FAILED: %s\n", what);
    ++failures;
  }
}

bool finite(const std::vector<double>& v) {
  for (double x : v)
    if (!std::isfinite(x)) return false;
  return true;
}

std::vector<float> normals(uint32_t tid, size_t n, double scale) {
  std::vector<float> v(n);
  expect(dg_normal(7, tid, 0, n, scale, 0, v.data()) == 0, "dg_normal fp32");
  return v;
}

}  // namespace

int main() {
  // flat layer: B 37 tokens, d 16, h 24, n 7 experts, k 3; fp32 and bf16 storage
  const int64_t B = 37;
  const int d = 16, h = 24, n = 7, k = 3;
  std::vector<float> x = normals(1, B * d, 1.0), wg = normals(2, n * d, 0.25),
                     wn = normals(3, n * d, 0.25), eps = normals(4, B * n, 1.0),
                     w1 = normals(5, n * h * d, 0.25), b1 = normals(6, n * h, 0.1),
                     w2 = normals(7, n * d * h, 0.2), b2 = normals(8, n * d, 0.1),
                     bg = normals(9, n, 0.3);
  std::vector<uint16_t> xb(x.size()), w1b(w1.size()), w2b(w2.size()), b1b(b1.size()),
      b2b(b2.size());
  dg_f32_to_bf16(x.data(), xb.data(), x.size());
  dg_f32_to_bf16(w1.data(), w1b.data(), w1.size());
  dg_f32_to_bf16(w2.data(), w2b.data(), w2.size());
  dg_f32_to_bf16(b1.data(), b1b.data(), b1.size());
  dg_f32_to_bf16(b2.data(), b2b.data(), b2.size());
  std::vector<uint16_t> probe(5);
  expect(dg_normal(7, 1, 3, 5, 1.0, 1, probe.data()) == 0, "dg_normal bf16");

  for (int train = 0; train < 2; ++train) {
    std::vector<double> clean(B * n), sigma(B * n), H(B * n), gate(B * k), thr(B * 2);
    std::vector<int32_t> idx(B * k);
    expect(oracle_gate(B, nullptr, d, n, k, x.data(), 0, wg.data(), wn.data(), 0, bg.data(),
                       eps.data(), train, 0.01, 1, clean.data(), sigma.data(), H.data(),
                       idx.data(), gate.data(), thr.data()) == 0,
           "oracle_gate");
    expect(finite(gate) && finite(clean), "gate outputs finite");
    std::vector<int64_t> rows = {0, 5, 36};
    std::vector<double> yr(rows.size() * d);
    expect(oracle_y_rows((int64_t)rows.size(), rows.data(), d, h, n, k, xb.data(), 1, wg.data(),
                         wn.data(), 0, bg.data(), eps.data(), train, 0.01, 1, w1b.data(),
                         b1b.data(), w2b.data(), b2b.data(), 1, yr.data()) == 0,
           "oracle_y_rows bf16");
    std::vector<double> load(n);
    expect(oracle_load(B, d, n, k, x.data(), 0, wg.data(), wn.data(), 0, bg.data(), eps.data(),
                       train, 0.01, 1, load.data()) == 0,
           "oracle_load");
    std::vector<int32_t> counts(n), offsets(n + 1), perm(B * k), slot(B * k);
    std::vector<double> pgate(B * k), imp(n);
    expect(oracle_route(B, n, k, idx.data(), gate.data(), counts.data(), offsets.data(),
                        perm.data(), pgate.data(), slot.data(), imp.data()) == 0,
           "oracle_route");
    std::vector<int32_t> experts(B * k);
    for (int e = 0; e < n; ++e)
      for (int q = offsets[e]; q < offsets[e + 1]; ++q) experts[q] = e;
    std::vector<int64_t> tok(perm.begin(), perm.end());
    std::vector<double> eo(B * k * d);
    expect(oracle_expert_pairs(B * k, tok.data(), experts.data(), d, h, x.data(), 0, w1.data(),
                               b1.data(), w2.data(), b2.data(), 0, eo.data()) == 0,
           "oracle_expert_pairs");
    std::vector<double> y(B * d), gg(B * k), th(B * 2), im(n), ld(n), losses(3);
    std::vector<int32_t> ii(B * k);
    expect(oracle_forward(B, d, h, n, k, x.data(), 0, wg.data(), wn.data(), 0, bg.data(),
                          eps.data(), train, 0.01, 1, w1.data(), b1.data(), w2.data(), b2.data(),
                          0, 0.1, 0.1, y.data(), ii.data(), gg.data(), th.data(), im.data(),
                          ld.data(), losses.data()) == 0,
           "oracle_forward");
    expect(finite(y) && finite(losses), "forward outputs finite");
    std::vector<double> dy(B * d);
    for (size_t i = 0; i < dy.size(); ++i) dy[i] = std::sin(0.37 * i);
    double J = 0.0;
    expect(oracle_objective(B, d, h, n, k, x.data(), 0, wg.data(), wn.data(), 0, bg.data(),
                            eps.data(), train, 0.01, w1.data(), b1.data(), w2.data(), b2.data(),
                            0, 0.1, 0.1, dy.data(), 1.0, ii.data(), th.data(), &J) == 0,
           "oracle_objective");
    std::vector<double> dx(B * d), dwg(n * d), dwn(n * d), dbg(n), dw1(n * h * d), db1(n * h),
        dw2(n * d * h), db2(n * d);
    expect(oracle_backward(B, d, h, n, k, x.data(), 0, wg.data(), wn.data(), 0, bg.data(),
                           eps.data(), train, 0.01, 1, w1.data(), b1.data(), w2.data(), b2.data(),
                           0, 0.1, 0.1, dy.data(), 1.0, ii.data(), dx.data(), dwg.data(),
                           dwn.data(), dbg.data(), dw1.data(), db1.data(), dw2.data(),
                           db2.data()) == 0,
           "oracle_backward");
    expect(finite(dx) && finite(dwg) && finite(dw1) && finite(dw2), "backward outputs finite");
    // the sampled backward: two experts, three tokens (the last row included)
    const int32_t se[2] = {n - 1, 0};
    const int64_t st[3] = {B - 1, 0, B / 2};
    std::vector<double> sg(2 * d), sn(2 * d), sb(2), s1(2 * h * d), sb1(2 * h), s2(2 * d * h),
        sb2(2 * d), sx(3 * d);
    expect(oracle_backward_sampled(B, d, h, n, k, x.data(), 0, wg.data(), wn.data(), 0, bg.data(),
                                   eps.data(), train, 0.01, 1, w1.data(), b1.data(), w2.data(),
                                   b2.data(), 0, 0.1, 0.1, dy.data(), 1.0, ii.data(), 2, se,
                                   sg.data(), sn.data(), sb.data(), 2, se, s1.data(), sb1.data(),
                                   s2.data(), sb2.data(), 3, st, sx.data()) == 0,
           "oracle_backward_sampled");
    expect(finite(sg) && finite(s1) && finite(sx), "sampled backward outputs finite");
    const int32_t bad_e[1] = {n};
    expect(oracle_backward_sampled(B, d, h, n, k, x.data(), 0, wg.data(), wn.data(), 0, bg.data(),
                                   eps.data(), train, 0.01, 1, w1.data(), b1.data(), w2.data(),
                                   b2.data(), 0, 0.1, 0.1, dy.data(), 1.0, ii.data(), 1, bad_e,
                                   sg.data(), sn.data(), sb.data(), 0, nullptr, nullptr, nullptr,
                                   nullptr, nullptr, 0, nullptr, nullptr) == 1,
           "oracle_backward_sampled rejects an expert index out of range");
  }
  // k == n: no (k+1)-th logit
  {
    std::vector<double> load(n);
    expect(oracle_load(B, d, n, n, x.data(), 0, wg.data(), wn.data(), 0, nullptr, eps.data(), 1,
                       0.01, 1, load.data()) == 0,
           "oracle_load k == n");
  }
  // the backward's pieces
  {
    std::vector<double> v = {3.6, 2.4, 1.2, 0.8}, g(4), dH(2);
    oracle_cv2_grad(4, v.data(), g.data());
    const double gates[2] = {0.55, 0.45}, dg[2] = {1.0, 0.0};
    oracle_kept_softmax_grad(2, gates, dg, dH.data());
    double pc, ps;
    oracle_p_eq9_grad(1.0, 1.3, 0.5, &pc, &ps);
    oracle_p_eq9_grad(1.0, -INFINITY, 0.5, &pc, &ps);
    expect(pc == 0.0 && ps == 0.0, "p_eq9_grad without threshold");
  }
  // hierarchy: a 3 groups x b 4 experts, k1 2, k2 2
  {
    const int a = 3, b = 4, k1 = 2, k2 = 2, nl = a * b;
    std::vector<float> g1 = normals(20, a * d, 0.25), n1 = normals(21, a * d, 0.25),
                       g2 = normals(22, a * b * d, 0.25), n2 = normals(23, a * b * d, 0.25),
                       e1 = normals(24, B * a, 1.0), e2 = normals(25, B * k1 * b, 1.0),
                       hw1 = normals(26, nl * h * d, 0.25), hw2 = normals(27, nl * d * h, 0.2);
    std::vector<int32_t> sel1(B * k1), sel2(B * k1 * k2), leaf(B * k1 * k2);
    std::vector<double> gate1(B * k1), thr1(B * 2), H1(B * a), gate2(B * k1 * k2),
        thr2(B * k1 * 2), H2(B * k1 * b), lg(B * k1 * k2);
    expect(oracle_hier_gate(B, nullptr, d, a, b, k1, k2, x.data(), 0, g1.data(), n1.data(),
                            g2.data(), n2.data(), 0, e1.data(), e2.data(), 1, 0.01, 1, nullptr,
                            nullptr, sel1.data(), gate1.data(), thr1.data(), H1.data(),
                            sel2.data(), gate2.data(), thr2.data(), H2.data(), leaf.data(),
                            lg.data()) == 0,
           "oracle_hier_gate");
    std::vector<double> y(B * d), i1(a), l1(a), r1(a), l2(nl), imp(nl), ld(nl), losses(3);
    std::vector<int32_t> li(B * k1 * k2);
    std::vector<double> lgo(B * k1 * k2);
    for (int with_y = 0; with_y < 2; ++with_y)
      expect(oracle_hier_forward(B, d, h, a, b, k1, k2, x.data(), 0, g1.data(), n1.data(),
                                 g2.data(), n2.data(), 0, e1.data(), e2.data(), 1, 0.01, 1,
                                 nullptr, nullptr, with_y ? hw1.data() : nullptr, nullptr,
                                 with_y ? hw2.data() : nullptr, nullptr, 0, 0.1, 0.1,
                                 with_y ? y.data() : nullptr, li.data(), lgo.data(), i1.data(),
                                 l1.data(), r1.data(), l2.data(), imp.data(), ld.data(),
                                 losses.data()) == 0,
             "oracle_hier_forward");
  }
  // invalid arguments are rejected, not read
  {
    std::vector<double> load(n);
    expect(oracle_load(B, d, n, n + 1, x.data(), 0, wg.data(), wn.data(), 0, nullptr, eps.data(),
                       1, 0.01, 1, load.data()) != 0,
           "oracle_load rejects k > n");
  }
  if (failures) return 1;
  std::printf("sanitized oracle driver: ok\n");
  return 0;
}
