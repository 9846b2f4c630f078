// Sharing-pattern search by dynamic programming ([IC-SUMMARY] Appendix C,
// similarity-based pattern search).  Host code: the problem is a few thousand
// additions over an n_layers x n_layers matrix.
//
// Layers are numbered 0..N-1 and layer 0 is F.  An S layer l takes its index set
// from src(l), the nearest F layer before it, and contributes S[l, src(l)]; F
// layers contribute nothing.  With the F layers j < i adjacent in the pattern,
// the S layers between them add seg(j, i) = sum_{j<l<i} S[l, j], and the S
// layers after the last F layer i add seg(i, N).  So
//     dp[i][m] = max_{j<i} dp[j][m-1] + seg(j, i),   dp[0][1] = 0,
//     best     = max_i dp[i][M] + seg(i, N),
// and backtracking the argmax choices gives the pattern.  seg comes from per-
// column prefix sums.
#include <cmath>
#include <limits>
#include <vector>

#include "common.hpp"

namespace dsa_host {

bool pattern_search_dp(const double* S, int n, int M, char* pattern, double* score) {
  const double NEG = -std::numeric_limits<double>::infinity();
  // pre[j][x] = sum_{l=j+1}^{x} S[l, j] for x >= j (pre[j][j] = 0); seg(j, i) = pre[j][i-1].
  std::vector<double> pre((size_t)n * n, 0.0);
  for (int j = 0; j < n; ++j) {
    double acc = 0.0;
    for (int x = j + 1; x < n; ++x) {
      acc += S[(size_t)x * n + j];
      pre[(size_t)j * n + x] = acc;
    }
  }
  auto seg = [&](int j, int i) { return pre[(size_t)j * n + (i - 1)]; };   // j < i <= n
  std::vector<double> dp((size_t)n * (M + 1), NEG);
  std::vector<int> arg((size_t)n * (M + 1), -1);
  dp[0 * (M + 1) + 1] = 0.0;
  for (int m = 2; m <= M; ++m) {
    for (int i = m - 1; i < n; ++i) {
      double best = NEG;
      int bj = -1;
      for (int j = m - 2; j < i; ++j) {
        const double prev = dp[(size_t)j * (M + 1) + (m - 1)];
        if (prev == NEG) continue;
        const double v = prev + seg(j, i);
        if (v > best) {   // strict: the earliest predecessor wins a tie
          best = v;
          bj = j;
        }
      }
      dp[(size_t)i * (M + 1) + m] = best;
      arg[(size_t)i * (M + 1) + m] = bj;
    }
  }
  double best = NEG;
  int last = -1;
  for (int i = M - 1; i < n; ++i) {
    const double d = dp[(size_t)i * (M + 1) + M];
    if (d == NEG) continue;
    const double v = d + (i + 1 < n ? seg(i, n) : 0.0);
    if (v > best) {
      best = v;
      last = i;
    }
  }
  if (last < 0) return false;
  for (int l = 0; l < n; ++l) pattern[l] = 'S';
  pattern[n] = '\0';
  for (int i = last, m = M; i >= 0 && m >= 1; i = arg[(size_t)i * (M + 1) + m], --m) pattern[i] = 'F';
  if (score) *score = best;
  return pattern[0] == 'F';
}

}  // namespace dsa_host
