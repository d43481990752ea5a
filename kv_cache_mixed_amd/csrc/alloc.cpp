// alloc.cpp -- block-wise bit-width allocation under a memory budget (host).
//
// PM-KVQ page, Key design 2: every transformer block i gets one width b from a
// set of choices, minimising the summed sensitivity s[i][b] while the blocks'
// KV-cache bytes stay within the budget M (an integer program on the page,
// solved there with a general solver).  Here it is solved exactly by dynamic
// programming over the byte costs divided by their greatest common divisor:
//   f[i][u] = min_j ( s[i][j] + f[i+1][u - w[i][j]] ),  f[n][u] = 0,
// u the remaining budget in those units, w the block's cost at choice j.
// The minimum is the sum evaluated from the last block to the first (binary64,
// the order of the recursion); the allocation returned is the
// lexicographically smallest choice vector that reaches it.
#include <cmath>
#include <cstdint>
#include <limits>
#include <new>
#include <vector>

#include "kvq.h"

namespace {
int64_t gcd64(int64_t a, int64_t b) {
  while (b) {
    const int64_t t = a % b;
    a = b;
    b = t;
  }
  return a;
}
}  // namespace

extern "C" kvq_status kvq_allocate_bits(int32_t n_blocks, int32_t n_choices, const double* sens,
                                        const int64_t* bytes, int64_t budget_bytes, int32_t* choice,
                                        double* cost) {
  try {
    if (n_blocks < 1 || n_choices < 1 || n_choices > KVQ_ALLOC_MAX_CHOICES) return KVQ_EINVAL;
    if (!sens || !bytes || !choice || budget_bytes < 0) return KVQ_EINVAL;
    const int64_t nb = n_blocks, nc = n_choices;
    int64_t g = 0, min_total = 0, max_total = 0;
    for (int64_t i = 0; i < nb; i++) {
      int64_t mn = std::numeric_limits<int64_t>::max(), mx = 0;
      for (int64_t j = 0; j < nc; j++) {
        const int64_t w = bytes[i * nc + j];
        const double s = sens[i * nc + j];
        if (w <= 0 || !std::isfinite(s)) return KVQ_EINVAL;
        if (w > (int64_t)1 << 50) return KVQ_EUNSUPPORTED;
        g = gcd64(g, w);
        mn = w < mn ? w : mn;
        mx = w > mx ? w : mx;
      }
      min_total += mn;
      max_total += mx;
    }
    if (min_total > budget_bytes) return KVQ_EBUDGET;
    // budget beyond every block's largest choice changes nothing
    const int64_t cap = budget_bytes < max_total ? budget_bytes : max_total;
    const int64_t U = cap / g;
    if ((U + 1) * (nb + 1) > KVQ_ALLOC_MAX_STATES) return KVQ_EUNSUPPORTED;
    const double INF = std::numeric_limits<double>::infinity();
    std::vector<double> f((size_t)((nb + 1) * (U + 1)), INF);
    auto F = [&](int64_t i, int64_t u) -> double& { return f[(size_t)(i * (U + 1) + u)]; };
    for (int64_t u = 0; u <= U; u++) F(nb, u) = 0.0;
    for (int64_t i = nb - 1; i >= 0; i--)
      for (int64_t u = 0; u <= U; u++) {
        double best = INF;
        for (int64_t j = 0; j < nc; j++) {
          const int64_t w = bytes[i * nc + j] / g;
          if (w > u) continue;
          const double c = sens[i * nc + j] + F(i + 1, u - w);
          if (c < best) best = c;
        }
        F(i, u) = best;
      }
    // forward: the smallest choice index that keeps the optimum at each block
    int64_t u = U;
    for (int64_t i = 0; i < nb; i++) {
      int32_t pick = -1;
      for (int64_t j = 0; j < nc && pick < 0; j++) {
        const int64_t w = bytes[i * nc + j] / g;
        if (w <= u && sens[i * nc + j] + F(i + 1, u - w) == F(i, u)) pick = (int32_t)j;
      }
      if (pick < 0) return KVQ_EHIP;   // cannot happen: F(i, u) is reached by some choice
      choice[i] = pick;
      u -= bytes[i * nc + pick] / g;
    }
    if (cost) *cost = F(0, U);
    return KVQ_OK;
  } catch (const std::bad_alloc&) {
    return KVQ_EUNSUPPORTED;
  } catch (...) {
    return KVQ_EHIP;
  }
}
