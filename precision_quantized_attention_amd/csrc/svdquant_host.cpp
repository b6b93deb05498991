// Offline weight preparation of SVD-Quant in FP4 (host code): the rank-r bf16 factors of a
// weight matrix and its bf16 residual, the inputs of kq_svdquant_down / kq_gemm_mxfp4_svdquant.
//
// The NVIDIA blog "Optimizing FLUX.1 Kontext for Image Editing with Low-Precision Quantization",
// section "Workflow and Quantization", names SVD-Quant in FP4 and gives none of its steps; the
// reading is W ~ L_up L_down with the leading r singular triplets of W (L_up = U_r S_r,
// L_down = V_r^T) kept in bf16 and the residual R = W - L_up L_down sent to FP4.
//
// The leading singular triplets come from a randomized range finder (Halko, Martinsson and
// Tropp, "Finding structure with randomness", 2011): Y = W Omega for a fixed pseudo-random
// Gaussian Omega with p = r + 8 columns, q rounds of power iteration (Y <- W W^T Y, each product
// re-orthonormalized by two passes of modified Gram-Schmidt), Q = orth(Y), B = Q^T W (p x K),
// then the SVD of the small B by one-sided Jacobi rotations (Hestenes) on the columns of B^T:
// B^T J = V S with V's columns orthonormal, so W ~ (Q J) S V^T.  All arithmetic is float64;
// each factor value is rounded once to bf16 (nearest even), and R is W minus the product of
// the rounded factors, in float64, rounded once.

#include "../../include/kq.h"

#include <math.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <vector>

namespace {

double bf16_value(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

// Nearest bf16 (ties to even) of a finite double within bf16's normal range: keep 8
// significant bits of the frexp mantissa (rint rounds halves to even in the default mode).
uint16_t bf16_round(double x) {
  int e = 0;
  const double m = frexp(x, &e);
  const float y = (float)ldexp(rint(m * 256.0) / 256.0, e);   // exact in float
  uint32_t u;
  memcpy(&u, &y, 4);
  return (uint16_t)(u >> 16);
}

// Deterministic standard normals (splitmix64 + Box-Muller).
struct Normal {
  uint64_t s;
  double spare = 0.0;
  bool has = false;
  explicit Normal(uint64_t seed) : s(seed) {}
  double uniform() {
    uint64_t z = (s += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    z ^= z >> 31;
    return ((z >> 11) + 0.5) * (1.0 / 9007199254740992.0);   // (0, 1)
  }
  double next() {
    if (has) {
      has = false;
      return spare;
    }
    const double u = uniform(), v = uniform();
    const double r = sqrt(-2.0 * log(u)), t = 6.283185307179586 * v;
    spare = r * sin(t);
    has = true;
    return r * cos(t);
  }
};

// Columns of X (rows x cols, row-major) made orthonormal in place, two passes of modified
// Gram-Schmidt; a column that vanishes is replaced by zeros.
void orthonormalize(std::vector<double>& X, int64_t rows, int cols) {
  for (int pass = 0; pass < 2; ++pass) {
    for (int j = 0; j < cols; ++j) {
      for (int i = 0; i < j; ++i) {
        double d = 0.0;
        for (int64_t r = 0; r < rows; ++r) d += X[r * cols + i] * X[r * cols + j];
        for (int64_t r = 0; r < rows; ++r) X[r * cols + j] -= d * X[r * cols + i];
      }
      double n = 0.0;
      for (int64_t r = 0; r < rows; ++r) n += X[r * cols + j] * X[r * cols + j];
      n = sqrt(n);
      const double inv = n > 0.0 ? 1.0 / n : 0.0;
      for (int64_t r = 0; r < rows; ++r) X[r * cols + j] *= inv;
    }
  }
}

// Y (N x p) = W (N x K) X (K x p)
void mul_w(const std::vector<double>& W, int64_t N, int64_t K, const std::vector<double>& X,
           int p, std::vector<double>& Y) {
  Y.assign(N * p, 0.0);
  for (int64_t n = 0; n < N; ++n) {
    double* y = &Y[n * p];
    const double* w = &W[n * K];
    for (int64_t k = 0; k < K; ++k) {
      const double a = w[k];
      const double* x = &X[k * p];
      for (int j = 0; j < p; ++j) y[j] += a * x[j];
    }
  }
}

// Z (K x p) = W^T (K x N) Y (N x p)
void mul_wt(const std::vector<double>& W, int64_t N, int64_t K, const std::vector<double>& Y,
            int p, std::vector<double>& Z) {
  Z.assign(K * p, 0.0);
  for (int64_t n = 0; n < N; ++n) {
    const double* w = &W[n * K];
    const double* y = &Y[n * p];
    for (int64_t k = 0; k < K; ++k) {
      const double a = w[k];
      double* z = &Z[k * p];
      for (int j = 0; j < p; ++j) z[j] += a * y[j];
    }
  }
}

}  // namespace

extern "C" kq_status kq_svdquant_factorize(const uint16_t* w_bf16, int64_t N, int64_t K,
                                           int rank, uint16_t* l_up_bf16,
                                           uint16_t* l_down_bf16, uint16_t* residual_bf16) {
  if (w_bf16 == nullptr || l_up_bf16 == nullptr || l_down_bf16 == nullptr ||
      residual_bf16 == nullptr || N < 1 || K < 1 || rank < 1)
    return KQ_ERR_INVALID_ARG;
  const int64_t mn = std::min(N, K);
  if (rank > mn) return KQ_ERR_INVALID_ARG;
  if (N * K > ((int64_t)1 << 32)) return KQ_ERR_UNSUPPORTED;
  const int p = (int)std::min<int64_t>(rank + 8, mn);
  const int q = 4;                                   // power-iteration rounds

  std::vector<double> W(N * K);
  for (int64_t i = 0; i < N * K; ++i) {
    W[i] = bf16_value(w_bf16[i]);
    if (!isfinite(W[i])) return KQ_ERR_INVALID_ARG;
  }
  // range finder
  std::vector<double> Om(K * p), Y, Z;
  Normal rng(0x5EEDu + (uint64_t)N * 1315423911u + (uint64_t)K);
  for (auto& v : Om) v = rng.next();
  mul_w(W, N, K, Om, p, Y);
  orthonormalize(Y, N, p);
  for (int it = 0; it < q; ++it) {
    mul_wt(W, N, K, Y, p, Z);
    orthonormalize(Z, K, p);
    mul_w(W, N, K, Z, p, Y);
    orthonormalize(Y, N, p);
  }
  // Bt (K x p) = W^T Q
  std::vector<double> Bt;
  mul_wt(W, N, K, Y, p, Bt);
  // one-sided Jacobi on the columns of Bt; J (p x p) accumulates the rotations
  std::vector<double> J(p * p, 0.0);
  for (int i = 0; i < p; ++i) J[i * p + i] = 1.0;
  for (int sweep = 0; sweep < 60; ++sweep) {
    double off = 0.0;
    for (int i = 0; i < p - 1; ++i)
      for (int j = i + 1; j < p; ++j) {
        double a = 0.0, b = 0.0, g = 0.0;
        for (int64_t k = 0; k < K; ++k) {
          const double x = Bt[k * p + i], y = Bt[k * p + j];
          a += x * x;
          b += y * y;
          g += x * y;
        }
        if (g == 0.0 || fabs(g) <= 1e-15 * sqrt(a * b)) continue;
        off = std::max(off, fabs(g) / sqrt(a * b));
        const double zeta = (b - a) / (2.0 * g);
        const double t = (zeta >= 0 ? 1.0 : -1.0) / (fabs(zeta) + sqrt(1.0 + zeta * zeta));
        const double c = 1.0 / sqrt(1.0 + t * t), s = c * t;
        for (int64_t k = 0; k < K; ++k) {
          const double x = Bt[k * p + i], y = Bt[k * p + j];
          Bt[k * p + i] = c * x - s * y;
          Bt[k * p + j] = s * x + c * y;
        }
        for (int k = 0; k < p; ++k) {
          const double x = J[k * p + i], y = J[k * p + j];
          J[k * p + i] = c * x - s * y;
          J[k * p + j] = s * x + c * y;
        }
      }
    if (off <= 1e-15) break;
  }
  // singular values = column norms of Bt; order them
  std::vector<double> sv(p);
  for (int j = 0; j < p; ++j) {
    double n = 0.0;
    for (int64_t k = 0; k < K; ++k) n += Bt[k * p + j] * Bt[k * p + j];
    sv[j] = sqrt(n);
  }
  std::vector<int> order(p);
  for (int j = 0; j < p; ++j) order[j] = j;
  std::stable_sort(order.begin(), order.end(), [&](int x, int y) { return sv[x] > sv[y]; });
  // L_up = (Q J)_r S_r, L_down = V_r^T with V = Bt's columns / S
  std::vector<double> up(N * rank), down((int64_t)rank * K);
  for (int c = 0; c < rank; ++c) {
    const int j = order[c];
    const double s = sv[j];
    for (int64_t n = 0; n < N; ++n) {
      double u = 0.0;
      for (int i = 0; i < p; ++i) u += Y[n * p + i] * J[i * p + j];
      l_up_bf16[n * rank + c] = bf16_round(u * s);
      up[n * rank + c] = bf16_value(l_up_bf16[n * rank + c]);
    }
    const double inv = s > 0.0 ? 1.0 / s : 0.0;
    for (int64_t k = 0; k < K; ++k) {
      l_down_bf16[(int64_t)c * K + k] = bf16_round(Bt[k * p + j] * inv);
      down[(int64_t)c * K + k] = bf16_value(l_down_bf16[(int64_t)c * K + k]);
    }
  }
  // R = bf16(W - L_up L_down) with the rounded factors
  std::vector<double> row(K);
  for (int64_t n = 0; n < N; ++n) {
    for (int64_t k = 0; k < K; ++k) row[k] = W[n * K + k];
    for (int c = 0; c < rank; ++c) {
      const double u = up[n * rank + c];
      const double* d = &down[(int64_t)c * K];
      for (int64_t k = 0; k < K; ++k) row[k] -= u * d[k];
    }
    for (int64_t k = 0; k < K; ++k) residual_bf16[n * K + k] = bf16_round(row[k]);
  }
  return KQ_OK;
}
