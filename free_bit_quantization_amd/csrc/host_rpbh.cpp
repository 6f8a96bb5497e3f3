// Seeded RPBH rotation tables (host).
//
// Method: "OrbitQuant: data-agnostic quantization for image and video"
// (rcap.io summary), paragraph on the Randomized Permuted Block-Hadamard
// rotation and the offline pseudo-code line that builds rotation[d]: a
// uniform random permutation, random sign flips, block-diagonal
// Walsh-Hadamard blocks of size h.  Only the permutation and the signs are
// random, so only they are tabulated; the Hadamard blocks are applied by
// the kernels' butterflies.
//
// Generator: splitmix64 (Steele, Lea and Flood, OOPSLA 2014), Fisher-Yates
// with a 128-bit multiply-shift bound, then one draw per sign.
#include "oq_internal.h"

namespace oq {

namespace {
struct SplitMix64 {
  uint64_t s;
  uint64_t next() {
    s += 0x9E3779B97F4A7C15ull;
    uint64_t z = s;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
  }
};
}  // namespace

void build_rpbh_tables(int32_t d, uint64_t seed, int32_t* perm, int8_t* sign) {
  SplitMix64 g{seed};
  for (int32_t i = 0; i < d; ++i) perm[i] = i;
  for (int32_t i = d - 1; i >= 1; --i) {
    unsigned __int128 prod = (unsigned __int128)g.next() * (unsigned __int128)(uint64_t)(i + 1);
    int32_t j = (int32_t)(uint64_t)(prod >> 64);
    int32_t t = perm[i];
    perm[i] = perm[j];
    perm[j] = t;
  }
  for (int32_t i = 0; i < d; ++i) sign[i] = (g.next() >> 63) ? (int8_t)-1 : (int8_t)1;
}

// Block-RHT, the rotation-ablation variant (same page, ablation paragraph:
// RPBH without its leading permutation): identity permutation, and the signs
// drawn from the start of the same stream (no shuffle draws before them).
void build_block_rht_tables(int32_t d, uint64_t seed, int32_t* perm, int8_t* sign) {
  SplitMix64 g{seed};
  for (int32_t i = 0; i < d; ++i) perm[i] = i;
  for (int32_t i = 0; i < d; ++i) sign[i] = (g.next() >> 63) ? (int8_t)-1 : (int8_t)1;
}

}  // namespace oq
