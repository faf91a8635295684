// Cyclic Jacobi eigensolver for a real symmetric matrix, float64 (host).
//
// Used by qkv_psac_fit: PSAC keeps the eigenvectors of the largest eigenvalues
// of the history queries' second-moment matrix (QuantWM summary, "QuantWM",
// second technique).  The matrix is at most 128 x 128, once per history window,
// so a plain and robust method is preferred to a fast one.
//
// The method: sweep over all off-diagonal pairs (p, q) in row order; each plane
// rotation J(p, q, theta) with tan(2 theta) = 2 a_pq / (a_qq - a_pp) annihilates
// a_pq; A <- J^T A J and V <- V J.  The off-diagonal mass decreases
// monotonically and the iteration converges quadratically; it stops when the
// off-diagonal Frobenius norm is below 1e-15 of the matrix norm.  The rotation
// is formed from t = tan(theta), the smaller root of t^2 + 2 t cot(2 theta) - 1,
// and the updates use tau = s / (1 + c) for numerical stability (Rutishauser's
// formulation).
#include <algorithm>
#include <cmath>
#include <numeric>
#include <vector>

namespace qkv {

// a: n x n row-major (overwritten).  evals (n) descending, evecs n x n
// row-major with column i the eigenvector of evals[i].
void jacobi_eigh(int n, double* a, double* evals, double* evecs) {
  std::vector<double> v((size_t)n * n, 0.0);
  for (int i = 0; i < n; ++i) v[(size_t)i * n + i] = 1.0;
  auto A = [&](int i, int j) -> double& { return a[(size_t)i * n + j]; };
  auto V = [&](int i, int j) -> double& { return v[(size_t)i * n + j]; };
  double total = 0.0;
  for (int i = 0; i < n * n; ++i) total += a[i] * a[i];
  for (int sweep = 0; sweep < 60; ++sweep) {
    double off = 0.0;
    for (int p = 0; p < n; ++p)
      for (int q = p + 1; q < n; ++q) off += 2.0 * A(p, q) * A(p, q);
    if (off <= 1e-30 * total || off == 0.0) break;
    for (int p = 0; p < n - 1; ++p) {
      for (int q = p + 1; q < n; ++q) {
        const double apq = A(p, q);
        if (apq == 0.0) continue;
        const double theta = (A(q, q) - A(p, p)) / (2.0 * apq);
        double t = 1.0 / (std::fabs(theta) + std::sqrt(theta * theta + 1.0));
        if (theta < 0.0) t = -t;
        const double c = 1.0 / std::sqrt(t * t + 1.0);
        const double s = t * c;
        const double tau = s / (1.0 + c);
        A(p, p) -= t * apq;
        A(q, q) += t * apq;
        A(p, q) = 0.0;
        A(q, p) = 0.0;
        for (int r = 0; r < n; ++r) {
          if (r == p || r == q) continue;
          const double arp = A(r, p), arq = A(r, q);
          const double nrp = arp - s * (arq + tau * arp);
          const double nrq = arq + s * (arp - tau * arq);
          A(r, p) = nrp;
          A(p, r) = nrp;
          A(r, q) = nrq;
          A(q, r) = nrq;
        }
        for (int r = 0; r < n; ++r) {
          const double vrp = V(r, p), vrq = V(r, q);
          V(r, p) = vrp - s * (vrq + tau * vrp);
          V(r, q) = vrq + s * (vrp - tau * vrq);
        }
      }
    }
  }
  std::vector<int> order(n);
  std::iota(order.begin(), order.end(), 0);
  std::stable_sort(order.begin(), order.end(), [&](int x, int y) { return A(x, x) > A(y, y); });
  for (int i = 0; i < n; ++i) {
    evals[i] = A(order[i], order[i]);
    for (int r = 0; r < n; ++r) evecs[(size_t)r * n + i] = V(r, order[i]);
  }
}

}  // namespace qkv
