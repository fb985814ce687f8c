// Host half: bitmap-aware row reordering of IE-BME local tiles, an offline
// step before the union-mask encoding.
//
// Source: "UnionSparse" page, section on bitmap-aware row reordering.  Per
// local tile (LT), rows are partitioned into groups of R_A; a group's cost is
// the number of union-mask entries it activates (grouped columns j at which
// any of its rows is kept in any of the C_A column partitions).  The subset
// DP F(S) = min over groups g of S holding S's smallest row of cost(g) +
// F(S - g) finds the least total; the optimal groups, canonicalised (rows
// ascending, groups in lexicographic order), are laid out partition-wise so
// that logical union row i holds group i.
//
// Ties: groups holding the smallest row are tried with their other rows in
// lexicographic order and the first minimum is kept, so the output is
// deterministic.  The DP is exponential in the LT height (the pages say so);
// LTs of up to kMaxRows rows are accepted.

#include <cstdint>
#include <cstring>
#include <vector>

#include "usw.h"
#include "usw_internal.h"
#include "usw_parallel.h"

namespace usw {
namespace {

constexpr int kMaxRows = 20;

// One LT's solver state, reused across the LTs a thread handles.  Memo
// entries are valid when their stamp equals the current LT's stamp, so no
// table is cleared between LTs.
struct Solver {
  int H = 0, r_a = 0, words = 0;
  std::vector<uint64_t> u;         // folded row bit sets, words per row
  std::vector<uint32_t> stamp;     // per subset
  std::vector<int32_t> best;       // F(S)
  std::vector<uint32_t> choice;    // the group chosen for S
  uint32_t cur = 0;

  explicit Solver(int h) : H(h), stamp(size_t(1) << h, 0), best(size_t(1) << h), choice(size_t(1) << h) {}

  int cost(uint32_t group) const {
    int c = 0;
    for (int w = 0; w < words; ++w) {
      uint64_t acc = 0;
      for (uint32_t g = group; g; g &= g - 1) acc |= u[static_cast<size_t>(__builtin_ctz(g)) * words + w];
      c += __builtin_popcountll(acc);
    }
    return c;
  }

  // Groups of r_a rows of S holding S's smallest row, other rows in
  // lexicographic order (recursive combination walk over the rows of S).
  int F(uint32_t S) {
    if (S == 0) return 0;
    if (stamp[S] == cur) return best[S];
    const int r0 = __builtin_ctz(S);
    const uint32_t rest = S & (S - 1);
    int rows[kMaxRows];
    int n = 0;
    for (uint32_t x = rest; x; x &= x - 1) rows[n++] = __builtin_ctz(x);
    int bestc = -1;
    uint32_t bestg = 0;
    int pick[kMaxRows];
    // Depth-first walk of the (r_a - 1)-combinations of rows[0..n).
    const int k = r_a - 1;
    int d = 0;
    pick[0] = -1;
    if (k == 0) {
      const uint32_t g = 1u << r0;
      bestc = cost(g) + F(S & ~g);
      bestg = g;
    } else {
      while (d >= 0) {
        ++pick[d];
        if (pick[d] > n - (k - d)) {
          --d;
          continue;
        }
        if (d + 1 < k) {
          pick[d + 1] = pick[d];
          ++d;
          continue;
        }
        uint32_t g = 1u << r0;
        for (int i = 0; i < k; ++i) g |= 1u << rows[pick[i]];
        const int c = cost(g) + F(S & ~g);
        if (bestc < 0 || c < bestc) {
          bestc = c;
          bestg = g;
        }
      }
    }
    stamp[S] = cur;
    best[S] = bestc;
    choice[S] = bestg;
    return bestc;
  }
};

}  // namespace
}  // namespace usw

using namespace usw;

extern "C" {

usw_status usw_union_reorder(const uint16_t* W, const uint8_t* mask, int32_t M, int32_t K, int32_t lt_m,
                             int32_t lt_k, int32_t r_a, int32_t c_a, int32_t* perm, int32_t* actives_before,
                             int32_t* actives_after) {
  if ((!W && !mask) || !perm) return USW_ERR_NULL_ARG;
  UnionGeometry g;
  usw_status st = make_union_geometry(M, K, lt_m, lt_k, r_a, c_a, &g);
  if (st) return st;
  if (lt_m > kMaxRows) return USW_ERR_UNSUPPORTED;
  const int H = static_cast<int>(lt_m), RA = static_cast<int>(r_a);
  const int64_t ak = g.ak, words = (ak + 63) / 64, G = g.am;
  parallel_for(g.nlt, [&](int64_t lo, int64_t hi) {
    Solver s(H);
    s.r_a = RA;
    s.words = static_cast<int>(words);
    s.u.assign(static_cast<size_t>(H * words), 0);
    for (int64_t t = lo; t < hi; ++t) {
      const int64_t ti = t / g.lc, tj = t % g.lc;
      std::fill(s.u.begin(), s.u.end(), 0);
      for (int r = 0; r < H; ++r)
        for (int64_t a = 0; a < g.c_a; ++a)
          for (int64_t j = 0; j < ak; ++j) {
            const int64_t idx = (ti * g.lt_m + r) * g.K + tj * g.lt_k + a * ak + j;
            const bool kept = mask ? mask[idx] != 0 : (W[idx] & 0x7FFFu) != 0;
            if (kept) s.u[static_cast<size_t>(r * words + j / 64)] |= 1ull << (j % 64);
          }
      if (++s.cur == 0) {   // stamp wrapped: invalidate every entry once
        std::fill(s.stamp.begin(), s.stamp.end(), 0);
        s.cur = 1;
      }
      const uint32_t all = (1u << H) - 1;
      const int total = s.F(all);
      // Groups in DP order hold increasing smallest rows, each ascending:
      // already the canonical order.
      std::vector<uint32_t> groups;
      for (uint32_t S = all; S; S &= ~s.choice[S]) groups.push_back(s.choice[S]);
      int32_t* out = perm + t * H;
      for (int p = 0; p < RA; ++p)
        for (size_t gi = 0; gi < groups.size(); ++gi) {
          uint32_t x = groups[gi];
          for (int q = 0; q < p; ++q) x &= x - 1;
          out[p * groups.size() + gi] = __builtin_ctz(x);
        }
      if (actives_after) actives_after[t] = total;
      if (actives_before) {
        int before = 0;
        for (int64_t i = 0; i < G; ++i) {
          uint32_t grp = 0;
          for (int p = 0; p < RA; ++p) grp |= 1u << (i + p * G);
          before += s.cost(grp);
        }
        actives_before[t] = before;
      }
    }
  });
  return USW_OK;
}

}  // extern "C"
