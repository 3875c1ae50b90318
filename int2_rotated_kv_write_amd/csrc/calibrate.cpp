// Offline calibration on the host, fp64: the calibration phase of the Spanish
// summary "Resumen Tecnico: OSCAR ...", section 2.2 A (steps 1-4), and the
// covariances of the Russian page, paragraph 2:
//   C_Q = (1/N) sum_n q_n^T q_n                   (query-aware key target)
//   C_S = (1/N) V^T S^T S V                       (score-aware value target)
//   U_Q, U_S = eigenbases (spectral decomposition)
//   clip = quantile of |calibration activations rotated by U H P|
// S is read as the causal softmax attention of each calibration query head.
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <thread>
#include <vector>

#include "../../include/oscar.h"

namespace {

constexpr int D = 128;

// Symmetric eigendecomposition by cyclic Jacobi rotations.  On return A is
// (numerically) diagonal with the eigenvalues and V holds the eigenvectors as
// columns.  Each rotation zeroes one off-diagonal entry a_pq.
void jacobi_eigen(std::vector<double>& A, std::vector<double>& V) {
  V.assign(D * D, 0.0);
  for (int i = 0; i < D; ++i) V[i * D + i] = 1.0;
  for (int sweep = 0; sweep < 100; ++sweep) {
    double off = 0.0, diag = 0.0;
    for (int i = 0; i < D; ++i)
      for (int j = 0; j < D; ++j) (i == j ? diag : off) += A[i * D + j] * A[i * D + j];
    if (off <= 1e-30 * diag) break;
    for (int p = 0; p < D - 1; ++p) {
      for (int q = p + 1; q < D; ++q) {
        const double apq = A[p * D + q];
        if (std::fabs(apq) < 1e-300) continue;
        const double app = A[p * D + p], aqq = A[q * D + q];
        // angle with tan(2 theta) = 2 apq / (aqq - app); t = tan(theta), smaller root
        const double tau = (aqq - app) / (2.0 * apq);
        const double t = (tau >= 0 ? 1.0 : -1.0) / (std::fabs(tau) + std::sqrt(1.0 + tau * tau));
        const double c = 1.0 / std::sqrt(1.0 + t * t), s = t * c;
        for (int k = 0; k < D; ++k) {   // columns p, q
          const double akp = A[k * D + p], akq = A[k * D + q];
          A[k * D + p] = c * akp - s * akq;
          A[k * D + q] = s * akp + c * akq;
        }
        for (int k = 0; k < D; ++k) {   // rows p, q
          const double apk = A[p * D + k], aqk = A[q * D + k];
          A[p * D + k] = c * apk - s * aqk;
          A[q * D + k] = s * apk + c * aqk;
        }
        A[p * D + q] = A[q * D + p] = 0.0;
        for (int k = 0; k < D; ++k) {
          const double vkp = V[k * D + p], vkq = V[k * D + q];
          V[k * D + p] = c * vkp - s * vkq;
          V[k * D + q] = s * vkp + c * vkq;
        }
      }
    }
  }
}

// Columns sorted by descending eigenvalue, each signed so that its entry of
// largest magnitude (first on ties) is positive.
void canonical_basis(const std::vector<double>& A, const std::vector<double>& V, std::vector<double>& U) {
  std::vector<int> order(D);
  for (int i = 0; i < D; ++i) order[i] = i;
  std::stable_sort(order.begin(), order.end(), [&](int a, int b) { return A[a * D + a] > A[b * D + b]; });
  U.assign(D * D, 0.0);
  for (int c = 0; c < D; ++c) {
    const int src = order[c];
    int arg = 0;
    double best = -1.0;
    for (int r = 0; r < D; ++r)
      if (std::fabs(V[r * D + src]) > best) {
        best = std::fabs(V[r * D + src]);
        arg = r;
      }
    const double sg = V[arg * D + src] < 0 ? -1.0 : 1.0;
    for (int r = 0; r < D; ++r) U[r * D + c] = sg * V[r * D + src];
  }
}

// Round to 8 significant bits, ties to even, directly from the double.
uint16_t to_bf16(double x) {
  if (x == 0.0) return std::signbit(x) ? 0x8000 : 0;
  int e;
  const double m = std::frexp(x, &e);            // x = m 2^e, 0.5 <= |m| < 1
  const double r = std::nearbyint(m * 256.0);    // default rounding: nearest even
  const float f = (float)std::ldexp(r / 256.0, e);
  uint32_t u;
  std::memcpy(&u, &f, 4);
  return (uint16_t)(u >> 16);
}

double from_bf16(uint16_t b) {
  const uint32_t u = (uint32_t)b << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}

int bitrev7(int x) {
  int r = 0;
  for (int b = 0; b < 7; ++b) r |= ((x >> b) & 1) << (6 - b);
  return r;
}

// |x U H P| for n rows of x, appended to out.  H applied as integer Sylvester
// butterflies followed by one division by sqrt(128).
void rotated_abs(const double* x, int n, const std::vector<double>& Ub, std::vector<double>& out) {
  std::vector<double> y(D), z(D);
  const double rs = std::sqrt((double)D);
  for (int i = 0; i < n; ++i) {
    const double* xi = x + (size_t)i * D;
    for (int j = 0; j < D; ++j) {
      double s = 0.0;
      for (int k = 0; k < D; ++k) s += xi[k] * Ub[k * D + j];
      y[j] = s;
    }
    for (int s = 1; s < D; s <<= 1)
      for (int a = 0; a < D; a += 2 * s)
        for (int k = a; k < a + s; ++k) {
          const double u = y[k], v = y[k + s];
          y[k] = u + v;
          y[k + s] = u - v;
        }
    for (int j = 0; j < D; ++j) z[j] = y[bitrev7(j)] / rs;
    for (int j = 0; j < D; ++j) out.push_back(std::fabs(z[j]));
  }
}

// Linear-interpolation quantile of an unsorted sample.
double quantile_linear(std::vector<double>& a, double q) {
  const size_t n = a.size();
  const double pos = q * (double)(n - 1);
  const size_t lo = (size_t)std::floor(pos);
  const double frac = pos - (double)lo;
  std::nth_element(a.begin(), a.begin() + lo, a.end());
  const double vlo = a[lo];
  if (lo + 1 >= n) return vlo;
  const double vhi = *std::min_element(a.begin() + lo + 1, a.end());
  return vlo + (vhi - vlo) * frac;
}

struct HeadJob {
  const double *q, *k, *v;   // q [G][N][D], k/v [N][D]
  int G, N;
  double sm_scale;
  std::vector<double> uq, us;   // fp64 eigenbases (columns)
};

void calibrate_head(HeadJob& job) {
  const int G = job.G, N = job.N;
  const double inv = 1.0 / ((double)G * N);
  // C_Q: pooled over the G query heads sharing this KV head
  std::vector<double> cq(D * D, 0.0);
  for (int s = 0; s < G * N; ++s) {
    const double* x = job.q + (size_t)s * D;
    for (int i = 0; i < D; ++i)
      for (int j = i; j < D; ++j) cq[i * D + j] += x[i] * x[j];
  }
  // C_S: outputs o_n = sum_{m<=n} softmax_m(sm_scale q_n . k_m) v_m
  std::vector<double> cs(D * D, 0.0), lg(N), o(D);
  for (int g = 0; g < G; ++g) {
    for (int n = 0; n < N; ++n) {
      const double* qn = job.q + ((size_t)g * N + n) * D;
      double mx = -INFINITY;
      for (int m = 0; m <= n; ++m) {
        const double* km = job.k + (size_t)m * D;
        double d = 0.0;
        for (int c = 0; c < D; ++c) d += qn[c] * km[c];
        lg[m] = job.sm_scale * d;
        mx = std::max(mx, lg[m]);
      }
      double tot = 0.0;
      std::fill(o.begin(), o.end(), 0.0);
      for (int m = 0; m <= n; ++m) {
        const double w = std::exp(lg[m] - mx);
        tot += w;
        const double* vm = job.v + (size_t)m * D;
        for (int c = 0; c < D; ++c) o[c] += w * vm[c];
      }
      for (int c = 0; c < D; ++c) o[c] /= tot;
      for (int i = 0; i < D; ++i)
        for (int j = i; j < D; ++j) cs[i * D + j] += o[i] * o[j];
    }
  }
  for (int i = 0; i < D; ++i)
    for (int j = i; j < D; ++j) {
      cq[i * D + j] *= inv;
      cs[i * D + j] *= inv;
      cq[j * D + i] = cq[i * D + j];
      cs[j * D + i] = cs[i * D + j];
    }
  std::vector<double> V;
  jacobi_eigen(cq, V);
  canonical_basis(cq, V, job.uq);
  jacobi_eigen(cs, V);
  canonical_basis(cs, V, job.us);
}

}  // namespace

extern "C" int oscar_calibrate_layer(int32_t num_kv_heads, int32_t gqa, int32_t num_samples, const double* q_cal,
                                     const double* k_cal, const double* v_cal, double sm_scale, double quantile,
                                     uint16_t* u_k_out, uint16_t* u_v_out, float* clip_k_out, float* clip_v_out,
                                     int32_t num_threads) {
  if (num_kv_heads < 1 || gqa < 1 || num_samples < 2 || !q_cal || !k_cal || !v_cal || !u_k_out || !u_v_out ||
      !clip_k_out || !clip_v_out || !(quantile >= 0.0 && quantile <= 1.0) || !std::isfinite(sm_scale))
    return OSCAR_EINVAL;
  const int H = num_kv_heads, G = gqa, N = num_samples;
  std::vector<HeadJob> jobs(H);
  for (int h = 0; h < H; ++h) {
    jobs[h].q = q_cal + (size_t)h * G * N * D;
    jobs[h].k = k_cal + (size_t)h * N * D;
    jobs[h].v = v_cal + (size_t)h * N * D;
    jobs[h].G = G;
    jobs[h].N = N;
    jobs[h].sm_scale = sm_scale;
  }
  int nt = num_threads > 0 ? num_threads : (int)std::thread::hardware_concurrency();
  nt = std::max(1, std::min(nt, H));
  {
    std::vector<std::thread> pool;
    for (int w = 0; w < nt; ++w)
      pool.emplace_back([&, w] {
        for (int h = w; h < H; h += nt) calibrate_head(jobs[h]);
      });
    for (auto& th : pool) th.join();
  }
  std::vector<double> rk, rv;
  rk.reserve((size_t)H * N * D);
  rv.reserve((size_t)H * N * D);
  for (int h = 0; h < H; ++h) {
    std::vector<double> ubk(D * D), ubv(D * D);
    for (int i = 0; i < D * D; ++i) {
      const uint16_t bk = to_bf16(jobs[h].uq[i]), bv = to_bf16(jobs[h].us[i]);
      u_k_out[(size_t)h * D * D + i] = bk;
      u_v_out[(size_t)h * D * D + i] = bv;
      ubk[i] = from_bf16(bk);
      ubv[i] = from_bf16(bv);
    }
    rotated_abs(jobs[h].k, N, ubk, rk);
    rotated_abs(jobs[h].v, N, ubv, rv);
  }
  *clip_k_out = (float)quantile_linear(rk, quantile);
  *clip_v_out = (float)quantile_linear(rv, quantile);
  return OSCAR_OK;
}

extern "C" int oscar_calibrate_clip(int32_t num_kv_heads, int32_t num_samples, const double* x_cal,
                                    const uint16_t* u, double quantile, float* clip_out) {
  if (num_kv_heads < 1 || num_samples < 1 || !x_cal || !u || !clip_out || !(quantile >= 0.0 && quantile <= 1.0))
    return OSCAR_EINVAL;
  const int H = num_kv_heads, N = num_samples;
  std::vector<double> r;
  r.reserve((size_t)H * N * D);
  for (int h = 0; h < H; ++h) {
    std::vector<double> ub(D * D);
    for (int i = 0; i < D * D; ++i) ub[i] = from_bf16(u[(size_t)h * D * D + i]);
    rotated_abs(x_cal + (size_t)h * N * D, N, ub, r);
  }
  *clip_out = (float)quantile_linear(r, quantile);
  return OSCAR_OK;
}
