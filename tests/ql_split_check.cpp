// Exhaustive check of the codebook GEMM's work split (ql_split.h) on the CPU.
//
// For a launch of ntiles tiles of nst K stages on `cus` compute units it
// enumerates what every workgroup computes, exactly as the kernel derives it,
// and checks the invariants the kernel relies on:
//   1. every whole tile [0, n_dp) is computed by exactly one workgroup;
//   2. every (tail tile, K stage) is computed by exactly one piece;
//   3. a tail tile's piece that holds its last stage finishes it (role 2),
//      every other piece leaves a partial (role 1);
//   4. the finisher's contributor list is exactly the workgroups that left a
//      partial of that tile, at most 4, in descending index order;
//   5. a finisher waits only on workgroups with a lower index;
//   6. a workgroup leaves at most one partial (one slot per workgroup), and
//      computes it before any piece it finishes;
//   7. the grid fits the workspace's slots.
// Also simulates the workspace's launch-generation protocol (ql_epoch and
// friends): `ql_split_check protocol`.
// Usage: ql_split_check ntiles nst cus [slots [w100]]   (one case, the plan's choice)
//        ql_split_check sweep                      (a broad sweep: the plan, and
//                                                   the split forced on every tail)
// Prints "ok <cases>" or the first violated invariant, exit status 1.
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <utility>
#include <map>
#include <set>
#include <vector>

#include "ql_split.h"

using namespace oq;

static int fail(const char* what, int64_t ntiles, int nst, int cus, int64_t slots, long a = 0, long b = 0) {
  std::printf("FAIL %s: ntiles=%lld nst=%d cus=%d slots=%lld (%ld %ld)\n", what, (long long)ntiles, nst, cus,
              (long long)slots, a, b);
  return 1;
}

static int check_split(const QlSplit& p, int64_t ntiles, int nst, int cus, int64_t slots);

// the plan for a workspace of `slots` slots
static int check(int64_t ntiles, int nst, int cus, int64_t slots, int w100 = 100) {
  return check_split(ql_split_plan(ntiles, nst, cus, slots, w100), ntiles, nst, cus, slots);
}

static int check_split(const QlSplit& p, int64_t ntiles, int nst, int cus, int64_t slots) {
  if (p.grid <= 0 || p.grid > cus) return fail("grid", ntiles, nst, cus, slots, p.grid);
  if (p.n_dp + p.sk_tiles != ntiles) return fail("tile count", ntiles, nst, cus, slots, (long)p.n_dp, p.sk_tiles);
  if (p.sk_tiles > 0 && p.grid > slots) return fail("slots", ntiles, nst, cus, slots, p.grid);
  if (p.grid % p.classes != 0) return fail("classes", ntiles, nst, cus, slots, p.classes);
  // 1. whole tiles
  std::vector<int> dp(p.n_dp, 0);
  for (int b = 0; b < p.grid; ++b) {
    int64_t t0, tstep, tend;
    ql_dp_range(p, b, &t0, &tstep, &tend);
    if (tend > p.n_dp) return fail("dp range end", ntiles, nst, cus, slots, b, (long)tend);
    for (int64_t t = t0; t < tend; t += tstep) {
      if (t < 0) return fail("dp tile < 0", ntiles, nst, cus, slots, b, (long)t);
      ++dp[t];
    }
  }
  for (int64_t t = 0; t < p.n_dp; ++t)
    if (dp[t] != 1) return fail("whole tile not computed once", ntiles, nst, cus, slots, (long)t, dp[t]);
  if (p.sk_tiles == 0) return 0;
  // 2.-6. the split tail
  std::vector<std::vector<int>> cover(p.sk_tiles, std::vector<int>(nst, 0));
  std::map<int64_t, std::set<int>> producers;     // tail tile -> workgroups leaving a partial
  std::map<int64_t, int> finisher;                 // tail tile -> finishing workgroup
  std::map<int64_t, std::vector<int>> contrib;     // tail tile -> finisher's list
  for (int b = 0; b < p.grid; ++b) {
    const QlClass c = ql_class(p, b);
    if (c.x + p.classes * c.loc != b) return fail("class index", ntiles, nst, cus, slots, b);
    const int np = ql_npieces(p, c);
    if (np < 0 || np > 2) return fail("pieces", ntiles, nst, cus, slots, b, np);
    int partials = 0;
    bool finished = false;
    for (int k = 0; k < np; ++k) {
      int64_t tl;
      int s0, s1, role;
      ql_piece(p, c, k, &tl, &s0, &s1, &role);
      const int64_t t = c.tx0 + tl;   // index among the tail tiles
      if (t < c.tx0 || t >= c.tx1) return fail("piece outside the class's tiles", ntiles, nst, cus, slots, b, (long)t);
      if (!(0 <= s0 && s0 < s1 && s1 <= nst)) return fail("piece stages", ntiles, nst, cus, slots, s0, s1);
      for (int st = s0; st < s1; ++st) ++cover[t][st];
      if ((s1 == nst) != (role == 2)) return fail("role vs last stage", ntiles, nst, cus, slots, b, role);
      if (role == 1) {
        if (finished) return fail("partial after a finish", ntiles, nst, cus, slots, b);
        ++partials;
        producers[t].insert(b);
      } else {
        if (finisher.count(t)) return fail("two finishers", ntiles, nst, cus, slots, (long)t, b);
        finisher[t] = b;
        finished = true;
        int cw[4];
        const int n = ql_contributors(p, c, tl, cw);
        if (n < 0) return fail("more than 4 contributors", ntiles, nst, cus, slots, (long)t, b);
        contrib[t] = std::vector<int>(cw, cw + n);
        for (int i = 0; i < n; ++i) {
          if (cw[i] >= b) return fail("waits on a later workgroup", ntiles, nst, cus, slots, b, cw[i]);
          if (i > 0 && cw[i] >= cw[i - 1]) return fail("contributor order", ntiles, nst, cus, slots, cw[i - 1], cw[i]);
        }
      }
    }
    if (partials > 1) return fail("more than one partial per workgroup", ntiles, nst, cus, slots, b, partials);
  }
  for (int64_t t = 0; t < p.sk_tiles; ++t) {
    for (int st = 0; st < nst; ++st)
      if (cover[t][st] != 1) return fail("tail stage not computed once", ntiles, nst, cus, slots, (long)t, st);
    if (!finisher.count(t)) return fail("tail tile without a finisher", ntiles, nst, cus, slots, (long)t);
    const std::set<int> got(contrib[t].begin(), contrib[t].end());
    if (got != producers[t] || got.size() != contrib[t].size())
      return fail("contributors differ from producers", ntiles, nst, cus, slots, (long)t, (long)got.size());
  }
  return 0;
}

// ---- the launch-generation protocol of a workspace, simulated ------------------------
// A sequence of split launches on one zero-filled workspace, workgroups
// starting in a scrambled order.  Launch `poison` loses one producer's flag
// (its producer never publishes: a device that stopped dispatching); every
// finisher looks at its contributors' flags before and after this launch's
// producers publish.  Checks: epochs are never 0 and differ from the previous
// launch's; before publication no contributor flag is ready (flags left by
// earlier launches, including the poisoned one, never match); after it all
// are, except the lost one in the poisoned launch; the header is back to
// (next generation, 0 started) after each launch.  `gen0` starts the
// generation near the 32-bit wrap.
static int protocol(int64_t ntiles, int nst, int cus, uint32_t gen0, int launches, int poison) {
  const QlSplit p = ql_split_make(ntiles, nst, cus, true);
  if (p.sk_tiles == 0) return 0;
  uint64_t hdr = gen0;   // generation gen0, none started
  std::vector<uint32_t> flags(p.grid, 0u);
  uint32_t prev_epoch = 0;
  uint64_t rng = 0x9E3779B97F4A7C15ull ^ (uint64_t)ntiles;
  for (int L = 0; L < launches; ++L) {
    // starts, in a scrambled order: each reads the generation, then counts itself
    std::vector<int> order(p.grid);
    for (int b = 0; b < p.grid; ++b) order[b] = b;
    for (int i = p.grid - 1; i > 0; --i) {
      rng = rng * 6364136223846793005ull + 1442695040888963407ull;
      std::swap(order[i], order[(int)((rng >> 33) % (uint64_t)(i + 1))]);
    }
    std::vector<uint32_t> epoch(p.grid);
    for (int b : order) {
      const uint64_t old = hdr;   // the atomic add's result
      hdr += ql_hdr_start();
      const uint32_t g = ql_hdr_gen(old);
      epoch[b] = ql_epoch(g);
      if (ql_last_starter(ql_hdr_started(old), (uint32_t)p.grid)) hdr = ql_hdr_next(g);
    }
    const uint32_t ep = epoch[0];
    for (int b = 0; b < p.grid; ++b)
      if (epoch[b] != ep) return fail("epochs differ within a launch", ntiles, nst, cus, cus, L, b);
    if (ep == 0) return fail("epoch 0", ntiles, nst, cus, cus, L);
    if (L > 0 && ep == prev_epoch) return fail("epoch repeated", ntiles, nst, cus, cus, L);
    if (ql_hdr_started(hdr) != 0 || ql_hdr_gen(hdr) != ql_next_gen(ep - 1u))
      return fail("header after the starts", ntiles, nst, cus, cus, L);
    prev_epoch = ep;
    // producers and finishers of this launch
    std::vector<int> producers;
    std::vector<std::vector<int>> waits;   // per finisher, its contributors
    for (int b = 0; b < p.grid; ++b) {
      const QlClass c = ql_class(p, b);
      for (int k = 0; k < ql_npieces(p, c); ++k) {
        int64_t tl;
        int s0, s1, role;
        ql_piece(p, c, k, &tl, &s0, &s1, &role);
        if (role == 1) producers.push_back(b);
        if (role == 2) {
          int cw[4];
          const int n = ql_contributors(p, c, tl, cw);
          if (n > 0) waits.push_back(std::vector<int>(cw, cw + n));
        }
      }
    }
    for (const auto& w : waits)
      for (int c : w)
        if (ql_flag_ready(flags[c], ep)) return fail("stale flag ready before publication", ntiles, nst, cus, cus, L, c);
    const int lost = (L == poison && !producers.empty()) ? producers[producers.size() / 2] : -1;
    for (int b : producers)
      if (b != lost) flags[b] = ep;
    for (const auto& w : waits)
      for (int c : w)
        if (ql_flag_ready(flags[c], ep) != (c != lost))
          return fail("flag readiness after publication", ntiles, nst, cus, cus, L, c);
  }
  return 0;
}

int main(int argc, char** argv) {
  long cases = 0;
  if (argc >= 4) {
    const int64_t ntiles = std::atoll(argv[1]);
    const int nst = std::atoi(argv[2]), cus = std::atoi(argv[3]);
    const int64_t slots = argc >= 5 ? std::atoll(argv[4]) : cus;
    const int w100 = argc >= 6 ? std::atoi(argv[5]) : 100;
    if (check(ntiles, nst, cus, slots, w100)) return 1;
    const QlSplit p = ql_split_plan(ntiles, nst, cus, slots, w100);
    std::printf("ok 1 n_dp=%lld sk_tiles=%d grid=%d classes=%d lmin=%d\n", (long long)p.n_dp, p.sk_tiles, p.grid,
                p.classes, p.lmin);
    return 0;
  }
  if (argc == 2 && std::strcmp(argv[1], "protocol") == 0) {
    const uint32_t gens[] = {0u, 7u, 0xFFFFFFFCu};
    for (uint32_t g : gens)
      for (int64_t nt : {(int64_t)8, (int64_t)36, (int64_t)136 + 512, (int64_t)200, (int64_t)300})
        for (int nst : {4, 24, 96}) {
          if (protocol(nt, nst, 256, g, 6, 2)) return 1;
          if (protocol(nt, nst, 80, g, 6, 0)) return 1;
          cases += 2;
        }
    std::printf("ok %ld\n", cases);
    return 0;
  }
  if (argc == 2 && std::strcmp(argv[1], "sweep") == 0) {
    const int nsts[] = {1, 2, 3, 4, 5, 6, 7, 8, 12, 16, 24, 40, 48, 96, 192};
    const int cuss[] = {1, 7, 8, 80, 104, 248, 256, 304};
    for (int cus : cuss)
      for (int nst : nsts)
        for (int64_t nt = 1; nt <= 3 * cus + 9; ++nt) {
          for (int64_t slots : {(int64_t)0, (int64_t)cus, (int64_t)cus - 1})
            for (int w100 : {70, 100, 105}) {
              if (check(nt, nst, cus, slots, w100)) return 1;
              ++cases;
            }
          // the split mechanism on every tail, whatever the plan would choose
          if (nst >= 2 && nt % cus != 0) {
            if (check_split(ql_split_make(nt, nst, cus, true), nt, nst, cus, cus)) return 1;
            ++cases;
          }
        }
    std::printf("ok %ld\n", cases);
    return 0;
  }
  std::fprintf(stderr, "usage: ql_split_check ntiles nst cus [slots] | sweep\n");
  return 2;
}
