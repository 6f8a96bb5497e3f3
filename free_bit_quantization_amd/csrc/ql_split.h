// Work split of the codebook GEMM over its persistent workgroups.
//
// Shared by the host planner, the kernel and a CPU test of the arithmetic
// (which compiles this header with a host compiler), so the split can be
// checked exhaustively without a GPU: every (tile, K stage) of a launch is
// computed exactly once, each tile of the split tail is finished by the one
// workgroup that holds its last K stage, and that workgroup waits only on
// workgroups with a lower index.
//
// A launch covers ntiles output tiles of 256 x 256, each nst K stages long.
//  * Tiles [0, n_dp) are whole-tile work: a workgroup computes all nst stages
//    of a tile and writes its outputs.
//  * With a split, the last sk_tiles tiles (the tail: the last, partial round
//    when there are more tiles than workgroups, else every tile) are cut along
//    K.  Workgroup b belongs to class x = b % classes (classes = 8 when the
//    grid is a multiple of 8: under the hardware's round-robin dealing of
//    workgroups over the 8 XCDs a class then shares one XCD's L2; nothing
//    depends on that for correctness).  Class x takes tiles [R x / C,
//    R (x + 1) / C) of the R = sk_tiles tail tiles and cuts their S_x stages
//    into rk runs of consecutive stages, run l = [S_x l / rk, S_x (l + 1) / rk)
//    for the class's l-th workgroup.  Runs are at least lmin stages, so a tile
//    has at most 4 pieces besides the one that finishes it, and never longer
//    than a tile, so a run touches at most two tiles.
//  * A piece that holds a tile's last stage finishes that tile: it adds the
//    partial tiles the class's lower workgroups left for it, in a fixed order,
//    and writes the outputs.  Any other piece leaves its partial tile in its
//    workgroup's slot (one slot per workgroup: a run produces at most one
//    partial) and raises its workgroup's flag.
#ifndef OQ_QL_SPLIT_H_
#define OQ_QL_SPLIT_H_

#include <stdint.h>

#if defined(__HIP__)
#define OQ_HD __host__ __device__
#else
#define OQ_HD
#endif

namespace oq {

struct QlSplit {
  int64_t ntiles;    // output tiles of the launch
  int64_t n_dp;      // whole tiles [0, n_dp)
  int32_t sk_tiles;  // tail tiles split along K (0: no split)
  int32_t nst;       // K stages per tile
  int32_t lmin;      // shortest run (stages)
  int32_t grid;      // workgroups
  int32_t classes;   // workgroup classes (1 or 8)
};

// The split of a launch whose tail (the last ntiles % cus tiles) is cut along K
// when `split` holds (needs nst >= 2, so that a run of lmin stages never spans
// more than two tiles); otherwise whole tiles only.
OQ_HD inline QlSplit ql_split_make(int64_t ntiles, int32_t nst, int32_t cus, bool split) {
  QlSplit p;
  p.ntiles = ntiles;
  p.nst = nst;
  p.n_dp = ntiles;
  p.sk_tiles = 0;
  p.lmin = 0;
  p.classes = 1;
  p.grid = (int32_t)(ntiles < cus ? ntiles : cus);
  const int64_t full = ntiles / cus, rem = ntiles % cus;
  if (split && rem > 0 && nst >= 2) {
    p.grid = cus;
    p.n_dp = full * cus;
    p.sk_tiles = (int32_t)rem;
    p.lmin = (nst + 3) / 4 > 2 ? (nst + 3) / 4 : 2;
    p.classes = cus % 8 == 0 ? 8 : 1;
  }
  return p;
}

// When the split pays, as a cost model fitted to measurements on MI355X (256
// CUs; HIP events over whole-tile and split launches of the same shapes, one
// process, alternating order).  A whole-tile tail costs one tile time, nst
// stages; split, its rem tiles spread over the CUs cost rem / cus of that plus
// a fixed overhead (partial tiles written and read back at one CU's bandwidth,
// the finisher's wait, a second pipeline start) of about 15 stages of a 4-bit
// activation stage (128 K).  So split iff nst w (1 - rem / cus) > 15, with w
// a stage's cost relative to that one: 100 (percent) for activations of at
// most 4 bits, 70 for 8-bit (a 64-wide stage) and 105 for 6-bit (64-wide, pair
// tables with bank conflicts).  Measured gains behind it: 24 stages, tails of
// 36, 72, 32 and 28 tiles +35, +6, +12 and +8 %, 132 to 216 tiles -3 to -14 %
// (136 after two rounds: FLUX QKV, whole); 96 stages, 24 to 192 tiles +150 %
// to +3 %, 216 tiles -1 %; 8-bit activations, 48 stages, 48 tiles +45 %, 128
// tiles within 1 %, 144 and 192 tiles -1 and -4 %; 6-bit, 48 stages, 136
// tiles +8 % (FLUX QKV W6A6).
OQ_HD inline int32_t ql_stage_weight(int32_t bits_a) { return bits_a == 8 ? 70 : bits_a == 6 ? 105 : 100; }

OQ_HD inline bool ql_split_pays(int64_t rem, int32_t nst, int32_t cus, int32_t w100) {
  if (rem <= 0 || rem >= cus || nst < 4) return false;
  return (int64_t)nst * w100 * (cus - rem) > (int64_t)1500 * cus;
}

// The plan: split the tail when a workspace with at least `slots` partial-tile
// slots is available (slots >= the workgroup count) and the split pays.
OQ_HD inline QlSplit ql_split_plan(int64_t ntiles, int32_t nst, int32_t cus, int64_t slots, int32_t w100 = 100) {
  return ql_split_make(ntiles, nst, cus,
                       slots >= cus && ql_split_pays(cus > 0 ? ntiles % cus : 0, nst, cus, w100));
}

// ---- whole tiles -----------------------------------------------------------
// Workgroup b takes tiles t0, t0 + tstep, ... below tend.  With a grid that is a
// multiple of 8, class x owns a contiguous eighth of the whole tiles (so its
// workgroups work on neighbouring tiles of the grouped raster order).
OQ_HD inline void ql_dp_range(const QlSplit& p, int b, int64_t* t0, int64_t* tstep, int64_t* tend) {
  if ((p.grid & 7) == 0) {
    const int x = b & 7, loc = b >> 3, per = p.grid >> 3;
    const int64_t q = p.n_dp / 8, rem = p.n_dp % 8;
    const int64_t start = x * q + (x < rem ? x : rem);
    *tend = start + q + (x < rem ? 1 : 0);
    *t0 = start + loc;
    *tstep = per;
  } else {
    *t0 = b;
    *tstep = p.grid;
    *tend = p.n_dp;
  }
}

// ---- the split tail ----------------------------------------------------------
struct QlClass {
  int x, loc, nloc;   // class, index in the class, workgroups in the class
  int64_t tx0, tx1;   // the class's tail tiles (indices among the tail tiles)
  int64_t S;          // its K stages
  int rk;             // its runs
};

OQ_HD inline QlClass ql_class(const QlSplit& p, int b) {
  QlClass c;
  const int C = p.classes;
  c.x = b % C;
  c.loc = b / C;
  c.nloc = p.grid / C;
  c.tx0 = (int64_t)p.sk_tiles * c.x / C;
  c.tx1 = (int64_t)p.sk_tiles * (c.x + 1) / C;
  c.S = (c.tx1 - c.tx0) * p.nst;
  const int64_t rkx = p.lmin > 0 ? c.S / p.lmin : 0;
  c.rk = (int)(rkx < c.nloc ? rkx : c.nloc);
  return c;
}

// first stage of run l (class-local stage index)
OQ_HD inline int64_t ql_bnd(const QlClass& c, int l) { return c.rk > 0 ? c.S * l / c.rk : 0; }

// Number of pieces of the class's run of workgroup c.loc (0, 1 or 2).
OQ_HD inline int ql_npieces(const QlSplit& p, const QlClass& c) {
  if (p.sk_tiles == 0 || c.loc >= c.rk) return 0;
  const int64_t u0 = ql_bnd(c, c.loc), u1 = ql_bnd(c, c.loc + 1);
  if (u0 >= u1) return 0;
  return u0 / p.nst == (u1 - 1) / p.nst ? 1 : 2;
}

// Piece k of the run, in execution order: with two pieces the producing one
// (the head of the second tile) comes first, then the one that finishes the
// first tile.  tile = class-local tail tile index; stages [s0, s1);
// role 1 = leaves a partial, 2 = finishes the tile.
OQ_HD inline void ql_piece(const QlSplit& p, const QlClass& c, int k, int64_t* tile, int* s0, int* s1, int* role) {
  const int nst = p.nst;
  const int64_t u0 = ql_bnd(c, c.loc), u1 = ql_bnd(c, c.loc + 1);
  const int64_t tA = u0 / nst, tB = (u1 - 1) / nst;
  if (tA == tB) {
    *tile = tA;
    *s0 = (int)(u0 - tA * nst);
    *s1 = (int)(u1 - tA * nst);
    *role = u1 == (tA + 1) * nst ? 2 : 1;
  } else if (k == 0) {
    *tile = tB;
    *s0 = 0;
    *s1 = (int)(u1 - tB * nst);
    *role = 1;
  } else {
    *tile = tA;
    *s0 = (int)(u0 - tA * nst);
    *s1 = nst;
    *role = 2;
  }
}

// Contributors of the finishing piece of class-local tile `tile` held by
// workgroup c.loc: the workgroups (grid indices, descending class index) whose
// runs reach into the tile before it.  Returns their number, or -1 if there
// are more than 4 (which the run lengths rule out).
OQ_HD inline int ql_contributors(const QlSplit& p, const QlClass& c, int64_t tile, int out[4]) {
  const int64_t U = tile * p.nst;   // the tile's first stage
  int n = 0;
  for (int l = c.loc - 1; l >= 0 && ql_bnd(c, l + 1) > U; --l) {
    if (ql_bnd(c, l) == ql_bnd(c, l + 1)) continue;   // empty run
    if (n == 4) return -1;
    out[n++] = c.x + p.classes * l;
  }
  return n;
}

// ---- launch generations of a workspace ---------------------------------------------
// The header is one 64-bit word: its low half holds the generation g of the
// next launch (0 in a zero-filled workspace), its high half counts the
// workgroups of the current launch that have started.  Every workgroup adds
// ql_hdr_start() to the word when it starts, one atomic that also returns g;
// the launch tags its flags with ql_epoch(g); the workgroup whose increment
// makes the count reach the grid stores ql_hdr_next(g) (next generation, none
// started).  That store follows every increment of the launch in the word's
// order of modifications, so no workgroup of the launch sees the next
// generation, and no fence is needed.  Epochs are never 0, so a flag that
// was never written does not match, and consecutive launches on one
// workspace use different epochs, so a flag left by an earlier launch (one
// whose finisher gave up) does not match either: flags need no clearing.
OQ_HD constexpr uint32_t ql_epoch(uint32_t g) { return g + 1u; }
OQ_HD constexpr uint32_t ql_next_gen(uint32_t g) { return g + 1u < 0xFFFFFFFFu ? g + 1u : 0u; }
OQ_HD constexpr bool ql_last_starter(uint32_t started_before, uint32_t grid) { return started_before + 1u == grid; }
OQ_HD constexpr bool ql_flag_ready(uint32_t flag, uint32_t epoch) { return flag == epoch; }
OQ_HD constexpr uint64_t ql_hdr_start() { return 1ull << 32; }
OQ_HD constexpr uint32_t ql_hdr_gen(uint64_t h) { return (uint32_t)h; }
OQ_HD constexpr uint32_t ql_hdr_started(uint64_t h) { return (uint32_t)(h >> 32); }
OQ_HD constexpr uint64_t ql_hdr_next(uint32_t g) { return (uint64_t)ql_next_gen(g); }

// ---- workspace layout ----------------------------------------------------------
// [0, 256)            header: one 64-bit word (launch generation, workgroups started)
// [256, 256 + F)      one 32-bit flag per workgroup slot (F = slots * 4, rounded up to 256)
// [256 + F, ...)      slots of 256 x 256 fp32 partial tiles (256 KB each)
constexpr int64_t kQlSlotBytes = 256 * 256 * 4;

OQ_HD constexpr int64_t ql_ws_flags_offset() { return 256; }
OQ_HD constexpr int64_t ql_ws_slots_offset(int64_t slots) { return 256 + ((slots * 4 + 255) / 256) * 256; }
OQ_HD constexpr int64_t ql_ws_bytes(int64_t slots) { return ql_ws_slots_offset(slots) + slots * kQlSlotBytes; }

}  // namespace oq

#endif  // OQ_QL_SPLIT_H_
