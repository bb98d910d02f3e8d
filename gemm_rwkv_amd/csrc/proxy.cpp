// RWKVQuant's weights-only coarse-to-fine proxy, on the host (RWKVQuant:
// Quantizing the RWKV Family with Proxy Guided Hybrid of Scalar and Vector
// Quantization -- Abstract of the index page; machine-review page,
// pith_extraction.key_machinery).  The weights are sorted and their adjacent
// gaps, divided by the mean gap, give
//   P_c = H(uniform gaps) - H(gaps) = (1/n) sum g log g     (0 log 0 = 0)
//   M_k = (1/n) sum (g - mean g)^k,   P_f = sum_{k=2..K} v_k |M_k|
// over the n = M - 1 normalised gaps g (H taken over g / sum g, natural log;
// the uniform gaps have H = log n, so the gap of the two entropies is the
// mean of g log g).  Sums are compensated (Neumaier) so that a tensor of 10^8
// weights keeps about 15 significant digits.
//
// Pure host code: it reads host memory and runs on the calling thread.
#include <math.h>

#include <algorithm>
#include <vector>

#include "rq.h"

namespace {

struct Sum {
  double s = 0.0, c = 0.0;
  void add(double x) {
    const double t = s + x;
    c += fabs(s) >= fabs(x) ? (s - t) + x : (x - t) + s;
    s = t;
  }
  double value() const { return s + c; }
};

}  // namespace

extern "C" int rq_proxy(const float* w, int64_t count, int K, const double* v, double* pc, double* pf,
                        double* moments) {
  if (!w || !pc || !pf) return RQ_ERR_NULL;
  if (count < 3 || K < 2 || K > RQ_PROXY_MAX_K) return RQ_ERR_SHAPE;
  for (int64_t i = 0; i < count; ++i)
    if (!isfinite(w[i])) return RQ_ERR_NONFINITE;
  std::vector<float> s(w, w + count);
  std::sort(s.begin(), s.end());
  const int64_t n = count - 1;
  // mean gap: the gaps telescope, but their sum is taken the way the gaps
  // are (each gap of two floats is exact in double)
  Sum gs;
  for (int64_t i = 0; i < n; ++i) gs.add((double)s[i + 1] - (double)s[i]);
  const double mean = gs.value() / (double)n;
  if (!(mean > 0.0)) return RQ_ERR_DEGENERATE;
  const double inv = 1.0 / mean;
  // normalised gaps: their mean (1 up to rounding) and sum g log g
  Sum gsum, glog;
  for (int64_t i = 0; i < n; ++i) {
    const double g = ((double)s[i + 1] - (double)s[i]) * inv;
    gsum.add(g);
    if (g > 0.0) glog.add(g * log(g));
  }
  const double gm = gsum.value() / (double)n;
  // P_c = log n - H with H = -sum (g/G) log(g/G), G = sum g = n gm
  const double G = gsum.value();
  *pc = log((double)n) + glog.value() / G - log(G);
  Sum mk[RQ_PROXY_MAX_K + 1];
  for (int64_t i = 0; i < n; ++i) {
    const double d = ((double)s[i + 1] - (double)s[i]) * inv - gm;
    double p = d;
    for (int k = 2; k <= K; ++k) {
      p *= d;
      mk[k].add(p);
    }
  }
  double f = 0.0;
  for (int k = 2; k <= K; ++k) {
    const double m = mk[k].value() / (double)n;
    double vk = 1.0;
    if (v) {
      vk = v[k - 2];
    } else {
      for (int j = 2; j <= k; ++j) vk /= (double)j;  // 1/k!
    }
    f += vk * fabs(m);
    if (moments) moments[k - 2] = m;
  }
  *pf = f;
  return RQ_OK;
}
