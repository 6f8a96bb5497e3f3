// Rotate-and-quantize kernels for gfx950.
//
// Method: "OrbitQuant: data-agnostic quantization for image and video"
// (rcap.io summary), online pseudo-code: per token x_rot = x R^T with the
// RPBH rotation (permutation gather, sign flips, block Walsh-Hadamard of
// size h, O(d log h) with a fast Hadamard transform), s = ||x_rot||, and the
// nearest centroid of x_rot / (s + eps) in the codebook of dimension d.
// The offline weight step is the same transform applied to weight rows.
//
// Activation kernel (hot path), one token row per group of d/16 lanes,
// each lane owning 16 coordinates:
//   1. coalesced 16-byte loads of the row into LDS (double-buffered across
//      loop iterations) and the sum of squares: s = ||x|| = ||x_rot|| since R
//      is orthogonal; per-lane fp64 sums of the exact squares (the
//      wavefront mapping below: fp32 per lane), fp64 across lanes;
//   2. signed gather from LDS: lane holds y_r = sign[i_r] x[perm[i_r]]; the
//      16 LDS addresses and sign words are loop-invariant registers;
//   3. block FWHT: a 16-point in-register transform over the top 4 index
//      bits, an LDS transpose inside the wavefront, then the remaining
//      log2(h) - 4 butterfly stages in registers (h <= 16: one pass);
//   4. threshold search: a uniform grid over the threshold range whose cells
//      hold at most one threshold, so idx = base[cell] + (u > theta[cell]),
//      decided by the sign of one fma;
//   5. guard: a coordinate whose fp32 value lies within a certified rounding
//      bound of its threshold is recomputed in fp64 by the lanes holding its
//      Hadamard block (rare; the groups of a wavefront work side by side)
//      and compared with the fp64 threshold (fp32 value + fp32 residual)
//      before its index is set, so every index is the one exact arithmetic
//      gives, up to fp64 rounding.  Bound: each output of the m = log2 h
//      butterfly stages is a depth-m tree of +-sums of exact inputs, so its
//      error is at most gamma_m L1(block), gamma_m = m u / (1 - m u), u = 2^-24;
//      the guard uses (m + 1) u L1 / (sqrt(h) s) with L1 and s as computed
//      (their relative errors fit in the extra u), plus k u |theta| of the
//      threshold compared, for the scale c = 1 / (sqrt(h) (s + eps)) and
//      theta's rounding to fp32 (u), at |u| ~ |theta| (the second-order k u
//      times the radius fits in the butterflies' spare u L1): k = 6 where s comes from fp64 sums of the exact squares
//      (c rounded once from fp64), k = 4 J + 5 where the fast path sums 8 J
//      squares per lane in fp32 ((8 J + 1) u in s^2, (4 J + 3.5) u in c); the
//      recheck then takes s from fp64 squares of the staged row;
//   6. LSB-first packing of 2 / 4 / 8-bit indices, one 4 / 8 / 16-byte store.
//
// Rows of d = 1024 J coordinates (J <= 5 for bf16, <= 2 for fp32) with h = 64
// or 256 take a second mapping of the same steps, rq_wave_kernel: a wavefront
// owns whole tokens (16 J coordinates per lane), so no workgroup barrier is needed after
// the set-up and every wavefront keeps its own token row in flight.
//
// Weight kernel (offline): one workgroup per row, fp64 throughout.
#include <cmath>
#include <type_traits>

#include "oq_internal.h"

namespace oq {
namespace {

constexpr int kPad = 16;  // floats of padding after each Hadamard block in the transpose buffer

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint64_t u64x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ void wave_sync_lds() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}


// ---- cross-lane sums on DPP (VALU latency instead of an LDS round trip) -----
// Stages pair lane i with i^1, i^2 (quad_perm), 7-i within 8 (row_half_mirror)
// and 15-i within 16 (row_mirror); each stage adds symmetric pairs, so every
// lane of a group ends with the bitwise-same total.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ double dpp_d(double v) {
  const uint64_t b = (uint64_t)__double_as_longlong(v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)b, CTRL, 0xF, 0xF, false);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(b >> 32), CTRL, 0xF, 0xF, false);
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}
// all-reduce over aligned groups of G lanes, G a power of two <= 16
template <int G, typename F>
__device__ __forceinline__ F group_sum(F v) {
  if constexpr (G >= 2) { if constexpr (sizeof(F) == 4) v += dpp_f<0xB1>(v); else v += dpp_d<0xB1>(v); }
  if constexpr (G >= 4) { if constexpr (sizeof(F) == 4) v += dpp_f<0x4E>(v); else v += dpp_d<0x4E>(v); }
  if constexpr (G >= 8) { if constexpr (sizeof(F) == 4) v += dpp_f<0x141>(v); else v += dpp_d<0x141>(v); }
  if constexpr (G >= 16) { if constexpr (sizeof(F) == 4) v += dpp_f<0x140>(v); else v += dpp_d<0x140>(v); }
  return v;
}
__device__ __forceinline__ double readlane_d(double v, int lane) {
  const uint64_t b = (uint64_t)__double_as_longlong(v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)b, lane);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), lane);
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}
// sum over the whole wavefront, same value in every lane, fixed order
__device__ __forceinline__ double wave_sum_d(double v) {
  v = group_sum<16>(v);
  return (readlane_d(v, 0) + readlane_d(v, 16)) + (readlane_d(v, 32) + readlane_d(v, 48));
}

__host__ __device__ inline size_t align16(size_t v) { return (v + 15) & ~size_t(15); }

// Staged rows are padded by 16 coordinates after every 256: coordinate i of a
// row sits at lds_pos(i).  The gathers read, for a fixed element index, one
// run of 16 coordinates per 256-block; without the padding every block's run
// falls on the same LDS banks (a 256-coordinate block spans a whole number of
// bank rows), which is what an identity or block-diagonal permutation (a folded
// permutation, Block-RHT) would read.  With it the blocks of a wavefront use
// different banks.  Random permutations are unaffected.
// (The workgroup kernel pads only when its layout still fits the LDS: pad = 0
// or 1 below.)
__host__ __device__ constexpr int lds_pos(int i, int pad = 1) { return i + pad * 16 * (i >> 8); }
__host__ __device__ constexpr int lds_row(int d, int pad = 1) { return d + pad * 16 * ((d + 255) >> 8); }

// Packed indices of one 16-coordinate slot: index r occupies bits
// [r BITS, (r+1) BITS) of a little-endian stream held in 32-bit words (the
// row layout of the index arrays); 2 BITS bytes are stored.
template <int BITS>
struct Pack16 {
  static constexpr int NW = (16 * BITS + 31) / 32;
  uint32_t w[NW];
  __device__ __forceinline__ Pack16() {
#pragma unroll
    for (int k = 0; k < NW; ++k) w[k] = 0;
  }
  // r must be a compile-time constant after unrolling
  __device__ __forceinline__ void put(int r, uint32_t v) {
    const int pos = BITS * r, k = pos >> 5, sh = pos & 31;
    w[k] |= v << sh;
    if (sh + BITS > 32) w[k + 1] |= v >> (32 - sh);
  }
  // replace index r (any r): on two 64-bit halves with runtime shifts, so the
  // words stay in registers
  __device__ __forceinline__ void set(int r, uint32_t v) {
    const uint64_t m = (1ull << BITS) - 1;
    uint64_t lo = w[0], hi = 0;
    if constexpr (NW > 1) lo |= (uint64_t)w[1] << 32;
    if constexpr (NW > 2) hi = w[2];
    if constexpr (NW > 3) hi |= (uint64_t)w[3] << 32;
    const int pos = BITS * r;
    if (pos < 64) {
      lo = (lo & ~(m << pos)) | ((uint64_t)v << pos);
      if (pos + BITS > 64) hi = (hi & ~(m >> (64 - pos))) | ((uint64_t)v >> (64 - pos));
    } else {
      hi = (hi & ~(m << (pos - 64))) | ((uint64_t)v << (pos - 64));
    }
    w[0] = (uint32_t)lo;
    if constexpr (NW > 1) w[1] = (uint32_t)(lo >> 32);
    if constexpr (NW > 2) w[2] = (uint32_t)hi;
    if constexpr (NW > 3) w[3] = (uint32_t)(hi >> 32);
  }
  // index r (any r)
  __device__ __forceinline__ uint32_t get(int r) const {
    uint64_t lo = w[0], hi = 0;
    if constexpr (NW > 1) lo |= (uint64_t)w[1] << 32;
    if constexpr (NW > 2) hi = w[2];
    if constexpr (NW > 3) hi |= (uint64_t)w[3] << 32;
    const uint64_t m = (1ull << BITS) - 1;
    const int pos = BITS * r;
    uint64_t v;
    if (pos < 64) {
      v = lo >> pos;
      if (pos + BITS > 64) v |= hi << (64 - pos);
    } else {
      v = hi >> (pos - 64);
    }
    return (uint32_t)(v & m);
  }
  // p: first byte of the slot (2 BITS bytes; aligned to 2 BITS bytes' natural
  // unit).  Non-temporal: the indices are read by the next kernel, not this one
  // (2 % faster than plain stores on the FLUX QKV rows).
  __device__ __forceinline__ void store(uint8_t* p) const {
    if constexpr (BITS == 2) {
      __builtin_nontemporal_store(w[0], reinterpret_cast<uint32_t*>(p));
    } else if constexpr (BITS == 4) {
      typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
      __builtin_nontemporal_store(u32x2_t{w[0], w[1]}, reinterpret_cast<u32x2_t*>(p));
    } else if constexpr (BITS == 8) {
      __builtin_nontemporal_store(u32x4{w[0], w[1], w[2], w[3]}, reinterpret_cast<u32x4*>(p));
    } else if constexpr (BITS == 6) {   // 12 bytes, 4-byte aligned
      uint32_t* q = reinterpret_cast<uint32_t*>(p);
      q[0] = w[0]; q[1] = w[1]; q[2] = w[2];
    } else {                            // 3 bits: 6 bytes, 2-byte aligned
      static_assert(BITS == 3, "index widths 2, 3, 4, 6, 8");
      uint16_t* q = reinterpret_cast<uint16_t*>(p);
      q[0] = (uint16_t)w[0]; q[1] = (uint16_t)(w[0] >> 16); q[2] = (uint16_t)w[1];
    }
  }
};

struct RqLayout {
  size_t lut, thr, row, trans, red, total, row_stride;  // row_stride: bytes of one parity buffer
};

__host__ __device__ inline RqLayout rq_layout(int d, int log2h, int es, int tpw, int G, int pad) {
  RqLayout L;
  const int h = 1 << log2h;
  L.lut = 0;
  L.thr = align16(8 * (size_t)(G > 0 ? G : 1));
  L.row = L.thr + 2 * 256 * 4;   // thr, then thr_lo
  L.row_stride = align16((size_t)tpw * lds_row(d, pad) * es);
  L.trans = L.row + 2 * L.row_stride;
  const size_t trans_bytes = log2h > 4 ? (size_t)tpw * (d / h) * (h + kPad) * 4 : 0;
  L.red = L.trans + align16(trans_bytes);
  L.total = L.red + 2 * 16 * 8;
  return L;
}

// #{j < n : thr[j] < u} by binary search (thr ascending, n <= 255).
__device__ __forceinline__ int count_below_f64(const float* thr, int n, double u) {
  int lo = 0;
#pragma unroll
  for (int step = 128; step >= 1; step >>= 1)
    if (lo + step <= n && (double)thr[lo + step - 1] < u) lo += step;
  return lo;
}

// #{j : theta_j < u} against the fp64 thresholds theta_j = thr[j] + thr_lo[j]
// (the sum is exact in fp64: thr_lo lies below half an fp32 ulp of thr),
// walking from a guess (the fast path's index, at most a step or two away):
// the result is exact for any guess in [0, n], since the thresholds ascend
// strictly.
__device__ __forceinline__ int count_below_exact_from(const float* thr, const float* thr_lo, int n, double u,
                                                      int lo) {
  while (lo > 0 && (double)thr[lo - 1] + (double)thr_lo[lo - 1] >= u) --lo;
  while (lo < n && (double)thr[lo] + (double)thr_lo[lo] < u) ++lo;
  return lo;
}

template <int LOG2H, bool BF16, int BITS>
__global__ void __launch_bounds__(768) rq_act_kernel(const RqArgs a, const int NS, const int TPW, const int PAD) {
  constexpr int H = 1 << LOG2H;
  constexpr int ES = BF16 ? 2 : 4;
  constexpr bool TWO_PASS = LOG2H > 4;
  constexpr int BL = TWO_PASS ? H / 16 : 1;        // lanes per Hadamard block
  constexpr int BPL = TWO_PASS ? 1 : 16 / H;       // Hadamard blocks per lane (one pass)
  constexpr float kGam = (LOG2H + 1) * 5.9604644775390625e-8f;  // (m+1) 2^-24 > gamma_m (1 + 3e-5)
  constexpr float kRel = 6.0f * 5.9604644775390625e-8f;   // 6 ulp of |theta| >= 2x the scale (one rounding from fp64) + theta roundings

  const int d = a.d;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int tl = tid / NS;          // token within the workgroup iteration
  const int sl = tid - tl * NS;     // 16-coordinate slot within the token
  const int G = a.G;
  const int nthr = a.nthr;

  extern __shared__ __align__(16) unsigned char smem[];
  const RqLayout Ly = rq_layout(d, LOG2H, ES, TPW, G, PAD);
  int2* lut = reinterpret_cast<int2*>(smem + Ly.lut);
  float* thr = reinterpret_cast<float*>(smem + Ly.thr);
  double* red = reinterpret_cast<double*>(smem + Ly.red);

  // ---- thresholds and the search grid --------------------------------------
  // thresholds (fp32) and their fp64 residuals side by side: the recheck reads
  // both with per-lane indices, which LDS serves without a memory round trip
  for (int i = tid; i < 256; i += blockDim.x) {
    thr[i] = i < nthr ? a.thr[i] : INFINITY;
    thr[256 + i] = i < nthr ? a.thr_lo[i] : 0.f;
  }
  __syncthreads();
  if (G > 0) {
    const double w = 1.0 / a.g_invw;
    for (int c = tid; c < G; c += blockDim.x) {
      const double ulo = c == 0 ? -INFINITY : a.g_lo + (c - 0.02) * w - a.g_rmax;
      const double uhi = c == G - 1 ? INFINITY : a.g_lo + (c + 1.02) * w + a.g_rmax;
      const int base = count_below_f64(thr, nthr, ulo);
      const float th = (base < nthr && (double)thr[base] <= uhi) ? thr[base] : INFINITY;
      lut[c] = make_int2(__float_as_int(th), base);
    }
  }

  // ---- loop-invariant gather addresses and sign words ------------------------
  // pass-1 element r of this lane has row coordinate gin(r)
  auto gin = [&](int r) -> int {
    if (TWO_PASS) return (sl / BL) * H + r * BL + (sl % BL);
    return 16 * sl + r;
  };
  uint32_t addr[16];
  uint32_t sgn[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int gi = gin(r);
    const int src = min((unsigned)a.perm[gi], (unsigned)(d - 1));  // perm is a permutation of 0..d-1
    addr[r] = (uint32_t)(Ly.row + ((size_t)tl * lds_row(d, PAD) + lds_pos(src, PAD)) * ES);
    sgn[r] = a.sign[gi] < 0 ? 0x80000000u : 0u;
  }
  __syncthreads();

  const float inv_sqrt_h = (float)(1.0 / sqrt((double)H));
  const float og = (float)(-a.g_lo * a.g_invw);
  const int64_t ngroups = (a.T + TPW - 1) / TPW;

  // raw 16 coordinates of this lane's slot, prefetched one token ahead
  constexpr int NV = BF16 ? 2 : 4;
  u32x4 raw[NV];
  auto fetch = [&](int64_t grp) {
    int64_t tk = grp * TPW + tl;
    tk = tk < a.T ? tk : a.T - 1;
    const u32x4* src = reinterpret_cast<const u32x4*>(static_cast<const unsigned char*>(a.x) +
                                                      ((size_t)tk * d + 16 * sl) * ES);
#pragma unroll
    for (int k = 0; k < NV; ++k) raw[k] = src[k];
  };
  if ((int64_t)blockIdx.x < ngroups) fetch(blockIdx.x);

  int par = 0;
  for (int64_t g = blockIdx.x; g < ngroups; g += gridDim.x, par ^= 1) {
    const int64_t tok = g * TPW + tl;
    const bool valid = tok < a.T;
    const uint32_t paroff = par * (uint32_t)Ly.row_stride;

    // ---- 1. stage the prefetched coordinates [16 sl, 16 sl + 16), sum of squares
    double q0 = 0.0, q1 = 0.0, q2 = 0.0, q3 = 0.0;   // exact squares, fp64 sums
    {
      u32x4* rowdst = reinterpret_cast<u32x4*>(smem + Ly.row + paroff +
                                               ((size_t)tl * lds_row(d, PAD) + lds_pos(16 * sl, PAD)) * ES);
#pragma unroll
      for (int k = 0; k < NV; ++k) rowdst[k] = raw[k];
      if (BF16) {
#pragma unroll
        for (int k = 0; k < 2; ++k) {
#pragma unroll
          for (int q = 0; q < 4; q += 2) {
            const uint32_t w0 = raw[k][q], w1 = raw[k][q + 1];
            const float e0 = __uint_as_float(w0 << 16), e1 = __uint_as_float(w0 & 0xFFFF0000u);
            const float e2 = __uint_as_float(w1 << 16), e3 = __uint_as_float(w1 & 0xFFFF0000u);
            q0 = fma((double)e0, (double)e0, q0);
            q1 = fma((double)e1, (double)e1, q1);
            q2 = fma((double)e2, (double)e2, q2);
            q3 = fma((double)e3, (double)e3, q3);
          }
        }
      } else {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const float e0 = __uint_as_float(raw[k][0]), e1 = __uint_as_float(raw[k][1]);
          const float e2 = __uint_as_float(raw[k][2]), e3 = __uint_as_float(raw[k][3]);
          q0 = fma((double)e0, (double)e0, q0);
          q1 = fma((double)e1, (double)e1, q1);
          q2 = fma((double)e2, (double)e2, q2);
          q3 = fma((double)e3, (double)e3, q3);
        }
      }
    }
    // the next token's row is in flight while this one is processed
    if (g + gridDim.x < ngroups) fetch(g + gridDim.x);
    double ss = (q0 + q1) + (q2 + q3);
    if (NS >= 64) {
      ss = wave_sum_d(ss);
      if (lane == 0) red[par * 16 + wave] = ss;
    } else {
      // groups of NS lanes (a power of two below 64)
      if (NS >= 16) ss = group_sum<16>(ss);
      else if (NS == 8) ss = group_sum<8>(ss);
      else if (NS == 4) ss = group_sum<4>(ss);
      else if (NS == 2) ss = group_sum<2>(ss);
      if (NS == 32) ss += __shfl_xor(ss, 16);
    }
    __syncthreads();
    if (NS >= 64) {
      ss = 0.0;
      const int nw = NS >> 6;
      for (int w = 0; w < nw; ++w) ss += red[par * 16 + w];
    }
    const double s64 = sqrt(ss);
    const double c64 = 1.0 / (sqrt((double)H) * (s64 + OQ_EPS));
    const float c = (float)c64;
    const float cg = (float)(c64 * a.g_invw);

    // ---- 2. signed gather ------------------------------------------------------
    float y[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      uint32_t bits;
      if (BF16) bits = (uint32_t)(*reinterpret_cast<const uint16_t*>(smem + addr[r] + paroff)) << 16;
      else bits = *reinterpret_cast<const uint32_t*>(smem + addr[r] + paroff);
      y[r] = __uint_as_float(bits ^ sgn[r]);
    }
    float l1[BPL];
#pragma unroll
    for (int q = 0; q < BPL; ++q) {
      l1[q] = 0.f;
#pragma unroll
      for (int r = 0; r < 16 / BPL; ++r) l1[q] += fabsf(y[q * (16 / BPL) + r]);
    }

    // ---- 3. block FWHT -----------------------------------------------------------
#pragma unroll
    for (int st = 1; st < (TWO_PASS ? 16 : H); st <<= 1) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        if (!(r & st)) {
          const float p = y[r], q = y[r + st];
          y[r] = p + q;
          y[r + st] = p - q;
        }
      }
    }
    if (TWO_PASS) {
      // element i of the block lives at row i/16 (its pass-2 lane), column
      // chunk (i/4 % 4) ^ (row/4 % 4): the 16 lanes of a block then hit 64
      // distinct banks with their 16-byte reads
      float* tb = reinterpret_cast<float*>(smem + Ly.trans) + ((size_t)tl * (d / H) + sl / BL) * (H + kPad);
      const int t = sl % BL;
      auto swz = [](int i) { return (i & ~15) | ((((i >> 2) & 3) ^ ((i >> 6) & 3)) << 2) | (i & 3); };
#pragma unroll
      for (int r = 0; r < 16; ++r) tb[swz(r * BL + t)] = y[r];
      wave_sync_lds();
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(tb + swz(t * 16 + 4 * k));
        y[4 * k] = v.x; y[4 * k + 1] = v.y; y[4 * k + 2] = v.z; y[4 * k + 3] = v.w;
      }
#pragma unroll
      for (int st = 1; st < BL; st <<= 1) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          if (!(r & st)) {
            const float p = y[r], q = y[r + st];
            y[r] = p + q;
            y[r + st] = p - q;
          }
        }
      }
      l1[0] = group_sum<BL>(l1[0]);
    }

    // ---- 4./5. threshold search and guard ----------------------------------------
    // Guard radius: the butterfly term of the coordinate's block plus k u
    // |theta|, with max |theta| for up to 16 levels (one compare per
    // coordinate) and the compared threshold's own |theta| above; the grid path
    // notes only whether the lane has a near coordinate, and the flags are
    // recomputed when some lane does.
    Pack16<BITS> pk;
    uint32_t flags = 0;
    auto put = [&](int r, int idx) { pk.put(r, (uint32_t)idx); };
    // guard radius: the butterfly term of the coordinate's block plus k u
    // |theta| of the compared threshold, per coordinate, the flags kept as a
    // bitmask on the fast path (here a slot-wide max |theta| radius with an
    // any-lane test and recomputed flags measured slower: the workgroup's
    // wavefronts meet at the next token's barrier, so a recheck anywhere
    // delays all of them)
    auto radius = [&](int r, float th) {
      const float radb = kGam * l1[TWO_PASS ? 0 : r / (16 / BPL)] * c;
      return fmaf(fabsf(th), kRel, radb);
    };
    if (G > 0) {
      // two halves of 8: all LUT reads of a half are in flight together
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        int2 e[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const int ci = (int)__builtin_amdgcn_fmed3f(fmaf(y[8 * hf + q], cg, og), 0.0f, (float)(G - 1));
          e[q] = lut[ci];
        }
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const int r = 8 * hf + q;
          const float th = __int_as_float(e[q].x);
          const float dd = fmaf(y[r], c, -th);
          put(r, e[q].y + (dd > 0.f ? 1 : 0));
          flags |= (fabsf(dd) < radius(r, th) ? 1u : 0u) << r;
        }
      }
    } else {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float v = y[r];
        int lo = 0;
        for (int step = 128; step >= 1; step >>= 1)
          if (lo + step <= nthr && fmaf(v, c, -thr[lo + step - 1]) > 0.f) lo += step;
        bool near = false;
        if (lo > 0) {
          const float th = thr[lo - 1];
          near |= fabsf(fmaf(v, c, -th)) < radius(r, th);
        }
        if (lo < nthr) {
          const float th = thr[lo];
          near |= fabsf(fmaf(v, c, -th)) < radius(r, th);
        }
        put(r, lo);
        flags |= (near ? 1u : 0u) << r;
      }
    }
    if (!valid) flags = 0;

    // fp64 recheck of guarded coordinates.  An output of Hadamard block b
    // depends only on that block's inputs, which the GS lanes of the block
    // hold (an aligned group: GS = BL with two passes, 1 with one), so each
    // group rechecks its own lowest flagged output per round and the groups
    // of a wavefront run their rounds side by side.  The group sum adds the
    // same nonzero parts in the same order as a wavefront sum would.
    constexpr int GS = TWO_PASS ? BL : 1;
    static_assert(GS <= 16, "group sums span at most 16 lanes");
    while (true) {
      const uint64_t bal = __ballot(flags != 0);
      if (bal == 0) break;
      const int g0 = lane & ~(GS - 1);
      const uint32_t gbits = (uint32_t)(bal >> g0) & ((1u << GS) - 1u);
      const int L = gbits ? g0 + __ffs(gbits) - 1 : lane;   // this group's leader
      const uint32_t fl = __shfl(flags, L);
      const int slL = __shfl(sl, L);
      const int r = fl ? __ffs(fl) - 1 : 0;
      const int gi = 16 * slL + r;
      const int b = gi >> LOG2H;
      const int j = gi & (H - 1);
      double part = 0.0;
      if (gbits) {
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
          const int gk = gin(rr);
          if ((gk >> LOG2H) == b) {
            uint32_t bits;
            if (BF16) bits = (uint32_t)(*reinterpret_cast<const uint16_t*>(smem + addr[rr] + paroff)) << 16;
            else bits = *reinterpret_cast<const uint32_t*>(smem + addr[rr] + paroff);
            const double yv = (double)__uint_as_float(bits ^ sgn[rr]);
            part += (__popc(j & gk & (H - 1)) & 1) ? -yv : yv;
          }
        }
      }
      if constexpr (GS > 1) part = group_sum<GS>(part);
      if (gbits && lane == L) {
        const double u = part / (sqrt((double)H) * (s64 + OQ_EPS));
        pk.set(r, (uint32_t)count_below_exact_from(thr, thr + 256, nthr, u, (int)pk.get(r)));
        flags &= ~(1u << r);
      }
    }

    // ---- 6. stores ----------------------------------------------------------------
    if (valid) {
      const int64_t ob = tok * (int64_t)d + 16 * sl;  // first coordinate of this slot
      pk.store(a.x_idx + ob * BITS / 8);
      if (a.x_rot) {
        f32x4* xr = reinterpret_cast<f32x4*>(a.x_rot + ob);
#pragma unroll
        for (int k = 0; k < 4; ++k)
          xr[k] = f32x4{y[4 * k] * inv_sqrt_h, y[4 * k + 1] * inv_sqrt_h, y[4 * k + 2] * inv_sqrt_h,
                        y[4 * k + 3] * inv_sqrt_h};
      }
      if (sl == 0) a.s[tok] = (float)s64;
    }
  }
}

// ---- activations, one wavefront per token (d = 1024 J, J <= 5, h = 64 or 256) ----
// The same computation as rq_act_kernel with a different mapping: a
// wavefront owns whole tokens, lane l stages the 16-coordinate chunks
// l, l + 64, ... of the row (coalesced), the norm is a wavefront sum, and
// slot j of lane l holds the pass-1 elements of coordinates [1024 j,
// 1024 j + 1024) exactly as slot 64 j + l of rq_act_kernel.  No barrier is
// needed after the set-up, so each wavefront runs its tokens independently
// and a CU keeps one token row in flight per wavefront.  Sign flips are
// applied while staging (sign'_perm(i) = sign_i), and only the grid search is
// built here (the host uses rq_act_kernel when the grid is empty).
constexpr int kByteCells = 256;

// Grid cell of the cell coordinate xc (see rq_wave_kernel).
template <bool BYTE>
__device__ __forceinline__ int grid_cell(float xc, int G) {
  if constexpr (BYTE) return (int)__builtin_amdgcn_cvt_pk_u8_f32(xc, 0u, 0u);
  else return (int)__builtin_amdgcn_fmed3f(xc, 0.0f, (float)(G - 1));
}

struct RqwLayout {
  size_t thr, lut, mtab, atab, wave0, row_bytes, wave_bytes, total;
};

__host__ __device__ inline RqwLayout rqw_layout(int d, int log2h, int es, int G, int wpb) {
  RqwLayout L;
  const int h = 1 << log2h;
  L.thr = 0;              // thr, then thr_lo
  L.lut = 2 * 256 * 4;
  L.mtab = L.lut + align16(8 * (size_t)(G > kByteCells ? G : kByteCells));   // byte cell indices: 256 cells
  const size_t mwords = es == 2 ? (size_t)d / 2 : (size_t)d;   // sign masks of the source words
  L.atab = L.mtab + align16(4 * mwords);                          // gather offsets, 4 d bytes
  L.wave0 = L.atab + align16(4 * (size_t)d);
  L.row_bytes = align16((size_t)lds_row(d) * es);
  L.wave_bytes = L.row_bytes + align16((size_t)(1024 / h) * (h + kPad) * 4);
  L.total = L.wave0 + (size_t)wpb * L.wave_bytes;
  const size_t setup = L.wave0 + align16((size_t)d);   // sign' bytes over the wave buffers
  if (setup > L.total) L.total = setup;
  return L;
}

// MAXT: the workgroup size the kernel is built for, 768 (12 wavefronts, 3 per
// SIMD: at most 170 VGPRs) or 512 (8 wavefronts: 256).  With 768 the slots of a
// token run one after the other (a rolled loop) so that the live values fit
// without spilling; with 512 the slot loop is unrolled and its slots overlap.
template <int LOG2H, bool BF16, int BITS, int J, int MAXT>
__global__ void __launch_bounds__(MAXT) rq_wave_kernel(const RqArgs a, const int WPB) {
  constexpr int H = 1 << LOG2H;
  constexpr int ES = BF16 ? 2 : 4;
  constexpr int BL = H / 16;                       // lanes per Hadamard block (h >= 32: two passes)
  static_assert(LOG2H >= 5 && LOG2H <= 8, "two-pass block sizes only");
  constexpr float kGam = (LOG2H + 1) * 5.9604644775390625e-8f;  // (m+1) 2^-24 > gamma_m (1 + 3e-5)
  // the fast-path scale comes from per-lane fp32 sums of 8 J squares: relative
  // error (8 J + 1) u in ss, (4 J + 3.5) u in c; with theta's rounding, (4 J + 5) u
  constexpr float kRel = (4 * J + 5) * 5.9604644775390625e-8f;
  constexpr int NV = BF16 ? 2 : 4;                 // 16-byte loads per 16-coordinate chunk
  constexpr int MW = BF16 ? 8 : 16;                // sign-mask words per chunk
  constexpr int d = 1024 * J;
  // Up to 64 levels the host's grid has at most 256 cells (the plan takes this
  // kernel only then), so a cell index is one byte conversion: round to
  // nearest of the cell coordinate minus 1/2 (floor, or at an exact tie the
  // cell below, which reaches 0.02 of a cell past its edge), saturated to
  // [0, 255] (NaN gives 0); cells G .. 255 repeat cell G - 1, whose range is
  // open above.  With 8-bit codes: clamp to [0, G - 1], then truncate.
  constexpr bool kByteCell = BITS <= 6;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int G = a.G;
  const int nthr = a.nthr;
  const int64_t T = a.T;
  const int64_t nwaves = (int64_t)gridDim.x * WPB;
  // tokens of wavefront w of workgroup b: b + grid (w + WPB k), so that every
  // workgroup (CU) gets the same share of the tokens
  const int64_t gw = (int64_t)blockIdx.x + (int64_t)gridDim.x * wave;

  extern __shared__ __align__(16) unsigned char smem[];
  const RqwLayout Ly = rqw_layout(d, LOG2H, ES, G, WPB);
  float* thr = reinterpret_cast<float*>(smem + Ly.thr);
  int2* lut = reinterpret_cast<int2*>(smem + Ly.lut);
  uint32_t* mtab = reinterpret_cast<uint32_t*>(smem + Ly.mtab);
  unsigned char* wrow = smem + Ly.wave0 + (size_t)wave * Ly.wave_bytes;   // this wavefront's row
  float* wtr = reinterpret_cast<float*>(wrow + Ly.row_bytes);           // and transpose buffer

  // raw chunks l + 64 i of this wavefront's current token
  u32x4 raw[J][NV];
  auto fetch = [&](int64_t tok) {
    tok = tok < T ? tok : T - 1;
#pragma unroll
    for (int i = 0; i < J; ++i) {
      const u32x4* src = reinterpret_cast<const u32x4*>(static_cast<const unsigned char*>(a.x) +
                                                        ((size_t)tok * d + 16 * (lane + 64 * i)) * ES);
#pragma unroll
      for (int k = 0; k < NV; ++k) raw[i][k] = src[k];
    }
  };
  // ---- set-up: thresholds, grid, sign masks, gather addresses ---------------
  // The small set-up loads (perm, sign: cache-resident after the first
  // workgroup) are issued before the first token's row, so they do not queue
  // behind it; the row streams in while the tables are built.
  // pass-1 element r of slot j of lane l has coordinate gin(j, l, r); its row
  // offset perm(gin) * ES sits at atab[((4 j + r / 4) * 64 + l) * 4 + r % 4], so
  // a slot's 16 offsets are four conflict-free 16-byte reads per lane
  auto gin = [&](int j, int l, int r) { return 1024 * j + (l / BL) * H + r * BL + (l % BL); };
  // d <= 16 blockDim (checked by the plan): at most 16 entries per thread
  int pj[16], pa[16];
  int8_t sj[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const int i = tid + k * (int)blockDim.x;
    pj[k] = i < d ? (int)min((unsigned)a.perm[i], (unsigned)(d - 1)) : 0;  // perm is a permutation
    sj[k] = i < d ? a.sign[i] : 0;
    const int kk = i & 3, l = (i >> 2) & 63, jq = i >> 8;   // table entry i: ((4 j + q) * 64 + l) * 4 + kk
    pa[k] = i < d ? (int)min((unsigned)a.perm[gin(jq >> 2, l, 4 * (jq & 3) + kk)], (unsigned)(d - 1)) : 0;
  }
  // the kernel-argument tables too (blockDim >= 256 >= kHostGrid): every set-up
  // load is issued before the first token's row, so waiting for them does not
  // wait for the row, which streams in under the table build
  const float thr_i = tid < nthr ? a.thr[tid] : INFINITY;
  const float thr_lo_i = tid < nthr ? a.thr_lo[tid] : 0.f;   // fp64 residuals, read by the recheck
  const bool host_grid = G > 0 && G <= kHostGrid;
  int2 glut_i = make_int2(0, 0);
  if (host_grid) {
    const int c = tid < G ? tid : G - 1;
    glut_i = make_int2(a.glut[c][0], a.glut[c][1]);
  }
  __builtin_amdgcn_sched_barrier(0);
  if (gw < T) fetch(gw);
  __builtin_amdgcn_sched_barrier(0);

  if (tid < 256) {
    thr[tid] = thr_i;
    thr[256 + tid] = thr_lo_i;
  }
  int8_t* sp = reinterpret_cast<int8_t*>(smem + Ly.wave0);   // sign' scratch over the wave buffers
  uint32_t* atab = reinterpret_cast<uint32_t*>(smem + Ly.atab);
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const int i = tid + k * (int)blockDim.x;
    if (i < d) {
      sp[pj[k]] = sj[k];
      atab[i] = (uint32_t)lds_pos(pa[k]) * ES;
    }
  }
  __syncthreads();
  const int ncell = kByteCell && G < kByteCells ? kByteCells : G;   // cells G .. ncell - 1 repeat cell G - 1
  if (host_grid) {
    // built on the host; thread c holds cell min(c, G - 1)
    if (tid < ncell) lut[tid] = glut_i;
  } else if (G > 0) {
    const double w = 1.0 / a.g_invw;
    for (int c = tid; c < ncell; c += blockDim.x) {
      const int cc = c < G ? c : G - 1;
      const double ulo = cc == 0 ? -INFINITY : a.g_lo + (cc - 0.02) * w - a.g_rmax;
      const double uhi = cc == G - 1 ? INFINITY : a.g_lo + (cc + 1.02) * w + a.g_rmax;
      const int base = count_below_f64(thr, nthr, ulo);
      const float th = (base < nthr && (double)thr[base] <= uhi) ? thr[base] : INFINITY;
      lut[c] = make_int2(__float_as_int(th), base);
    }
  }
  for (int i = tid; i < d / (16 / MW); i += blockDim.x) {
    uint32_t m;
    if (BF16) m = (sp[2 * i] < 0 ? 0x8000u : 0u) | (sp[2 * i + 1] < 0 ? 0x80000000u : 0u);
    else m = sp[i] < 0 ? 0x80000000u : 0u;
    mtab[i] = m;
  }
  __syncthreads();  // tables complete, sign scratch consumed

  const float inv_sqrt_h = (float)(1.0 / sqrt((double)H));
  const float kSqrtH = (float)sqrt((double)H);
  const float og = (float)(-a.g_lo * a.g_invw) - (kByteCell ? 0.5f : 0.0f);
  const float ginvw = (float)a.g_invw;

  for (int64_t tok = gw; tok < T; tok += nwaves) {
    // ---- 1. signed staging of the row, sum of squares --------------------------
    float q0 = 0.f, q1 = 0.f;
#pragma unroll
    for (int i = 0; i < J; ++i) {
      const int k = lane + 64 * i;   // chunk: coordinates [16 k, 16 k + 16)
      const u32x4* mk = reinterpret_cast<const u32x4*>(mtab + k * MW);
      u32x4* dst = reinterpret_cast<u32x4*>(wrow + (size_t)lds_pos(16 * k) * ES);
#pragma unroll
      for (int v = 0; v < NV; ++v) {
        const u32x4 m = mk[v];
        u32x4 w = raw[i][v];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if (BF16) {
            const float e0 = __uint_as_float(w[q] << 16), e1 = __uint_as_float(w[q] & 0xFFFF0000u);
            q0 = fmaf(e0, e0, q0);
            q1 = fmaf(e1, e1, q1);
          } else {
            const float e = __uint_as_float(w[q]);
            if (q & 1) q1 = fmaf(e, e, q1);
            else q0 = fmaf(e, e, q0);
          }
        }
        dst[v] = w ^ m;
      }
    }
    // registers free again: the next token's row is in flight from here on
    if (tok + nwaves < T) fetch(tok + nwaves);
    const double ss = wave_sum_d((double)(q0 + q1));
    // fp32 scale for the fast path (its error is inside the guard's kRel)
    const float s32 = sqrtf((float)ss);
    const float c = 1.0f / (kSqrtH * (s32 + (float)OQ_EPS));
    const float cg = c * ginvw;
    wave_sync_lds();  // the staged row is visible to every lane

    const uint32_t rowbase = (uint32_t)(Ly.wave0 + (size_t)wave * Ly.wave_bytes);
    double inv64 = 0.0;   // 1 / (sqrt(h) (s + eps)) from the exact norm, once a slot needs it
    auto slot = [&](const int j) {
      // ---- 2. gather ---------------------------------------------------------------
      uint32_t addr[16];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const u32x4 o = reinterpret_cast<const u32x4*>(atab)[(4 * j + q) * 64 + lane];
#pragma unroll
        for (int k = 0; k < 4; ++k) addr[4 * q + k] = rowbase + o[k];
      }
      float y[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        if (BF16) y[r] = __uint_as_float((uint32_t)(*reinterpret_cast<const uint16_t*>(smem + addr[r])) << 16);
        else y[r] = *reinterpret_cast<const float*>(smem + addr[r]);
      }
      float l1 = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) l1 += fabsf(y[r]);

      // ---- 3. block FWHT: 16 points in registers, transpose, log2(h) - 4 stages --
#pragma unroll
      for (int st = 1; st < 16; st <<= 1) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          if (!(r & st)) {
            const float p = y[r], q = y[r + st];
            y[r] = p + q;
            y[r + st] = p - q;
          }
        }
      }
      {
        float* tb = wtr + (size_t)(lane / BL) * (H + kPad);
        const int t = lane % BL;
        auto swz = [](int i) { return (i & ~15) | ((((i >> 2) & 3) ^ ((i >> 6) & 3)) << 2) | (i & 3); };
#pragma unroll
        for (int r = 0; r < 16; ++r) tb[swz(r * BL + t)] = y[r];
        wave_sync_lds();
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const f32x4 v = *reinterpret_cast<const f32x4*>(tb + swz(t * 16 + 4 * k));
          y[4 * k] = v.x; y[4 * k + 1] = v.y; y[4 * k + 2] = v.z; y[4 * k + 3] = v.w;
        }
        wave_sync_lds();  // reads done before the next slot overwrites the buffer
      }
#pragma unroll
      for (int st = 1; st < BL; st <<= 1) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          if (!(r & st)) {
            const float p = y[r], q = y[r + st];
            y[r] = p + q;
            y[r + st] = p - q;
          }
        }
      }
      l1 = group_sum<BL>(l1);

      // ---- 4./5. grid search and guard --------------------------------------------
      // The guard radius: the butterfly term of this slot's block plus k u |theta|
      // of the threshold compared.  Up to 16 levels one radius covers the slot
      // (|theta| <= max |theta|: a wider band, hardly more rechecks at these
      // widths, one compare per coordinate); with more levels each compare uses
      // its own threshold's term, which keeps the band narrow where rechecks are
      // frequent.  The fast path only notes whether some coordinate of the lane
      // is near (a lane mask); the recheck recomputes which.
      const float radb = kGam * l1 * c;
      const float rad_slot = fmaf(a.thr_absmax, kRel, radb);
      constexpr bool kSlotRadius = BITS <= 4;
      auto radius = [&](float th) { return kSlotRadius ? rad_slot : fmaf(fabsf(th), kRel, radb); };
      Pack16<BITS> pw;
      bool near = false;
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        int2 e[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          e[q] = lut[grid_cell<kByteCell>(fmaf(y[8 * hf + q], cg, og), G)];
        }
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const int r = 8 * hf + q;
          const float th = __int_as_float(e[q].x);
          const float dd = fmaf(y[r], c, -th);
          const uint32_t idx = (uint32_t)e[q].y + (dd > 0.f ? 1u : 0u);
          pw.put(r, idx);
          near |= fabsf(dd) < radius(th);
        }
      }

      // fp64 recheck of guarded coordinates (rare).  The BL lanes of a Hadamard
      // block hold its inputs (pass 1) and its outputs (pass 2), so each group
      // of BL lanes recomputes one of its flagged coordinates per round, all
      // groups at once, with an fp64 sum over the group.
      if (__ballot(near) != 0) {
        // which coordinates: the fast path's test again, per coordinate
        uint32_t flags = 0;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float th = __int_as_float(lut[grid_cell<kByteCell>(fmaf(y[r], cg, og), G)].x);
          flags |= (fabsf(fmaf(y[r], c, -th)) < radius(th) ? 1u : 0u) << r;
        }
        // the norm again, exactly: fp64 squares of the staged row (sign flips do
        // not change them); the fast path's fp32 partials are only certified.
        // Once per token (8-bit codebooks flag ~2 coordinates per token).
        if (inv64 == 0.0) {
          double sx = 0.0;
#pragma unroll
          for (int i = 0; i < J; ++i) {
            const u32x4* src = reinterpret_cast<const u32x4*>(wrow + (size_t)lds_pos(16 * (lane + 64 * i)) * ES);
#pragma unroll
            for (int v = 0; v < NV; ++v) {
              const u32x4 w = src[v];
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                if (BF16) {
                  const double e0 = __uint_as_float(w[q] << 16), e1 = __uint_as_float(w[q] & 0xFFFF0000u);
                  sx = fma(e0, e0, sx);
                  sx = fma(e1, e1, sx);
                } else {
                  const double e = __uint_as_float(w[q]);
                  sx = fma(e, e, sx);
                }
              }
            }
          }
          sx = wave_sum_d(sx);
          inv64 = 1.0 / (sqrt((double)H) * (sqrt(sx) + OQ_EPS));
        }
        const int g0 = lane & ~(BL - 1);   // first lane of this lane's block group
        // the gather addresses again (not kept live through the transform)
        uint32_t raddr[16];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const u32x4 o = reinterpret_cast<const u32x4*>(atab)[(4 * j + q) * 64 + lane];
#pragma unroll
          for (int k = 0; k < 4; ++k) raddr[4 * q + k] = rowbase + o[k];
        }
        while (true) {
          const uint64_t bal = __ballot(flags != 0);
          if (bal == 0) break;
          const uint32_t gm = (uint32_t)(bal >> g0) & ((1u << BL) - 1u);   // flagged lanes of the group
          const int L = gm ? g0 + __ffs(gm) - 1 : lane;                    // owner of this round's coordinate
          const uint32_t fl = __shfl(flags, L);
          const int r = gm ? __ffs(fl) - 1 : 0;
          const int gi = 1024 * j + 16 * L + r;   // coordinate of pass-2 element r of lane L
          const int b = gi >> LOG2H;
          const int jj = gi & (H - 1);
          double part = 0.0;
#pragma unroll
          for (int rr = 0; rr < 16; ++rr) {
            const int gk = gin(j, lane, rr);
            if (gm && (gk >> LOG2H) == b) {
              double yv;
              if (BF16) yv = (double)__uint_as_float((uint32_t)(*reinterpret_cast<const uint16_t*>(smem + raddr[rr])) << 16);
              else yv = (double)*reinterpret_cast<const float*>(smem + raddr[rr]);
              part += (__popc(jj & gk & (H - 1)) & 1) ? -yv : yv;
            }
          }
          part = group_sum<BL>(part);
          if (gm && lane == L) {
            const double u = part * inv64;
            // u is exact to fp64 rounding; its cell holds the only threshold near it
            const double cf = fmin(fmax(floor((u - a.g_lo) * a.g_invw), 0.0), (double)(G - 1));
            const int2 e = lut[(int)cf];
            // against the fp64 threshold (thr + thr_lo), not its fp32 rounding
            const double th = e.x == __float_as_int(INFINITY)
                                  ? (double)INFINITY
                                  : (double)__int_as_float(e.x) + (double)thr[256 + e.y];
            const uint32_t nidx = (uint32_t)e.y + (th < u ? 1u : 0u);
            pw.set(r, nidx);
            flags &= ~(1u << r);
          }
        }
      }

      // ---- 6. stores ----------------------------------------------------------------
      const int64_t ob = tok * (int64_t)d + 1024 * j + 16 * lane;  // first coordinate of this slot
      pw.store(a.x_idx + ob * BITS / 8);
      if (a.x_rot) {
        f32x4* xr = reinterpret_cast<f32x4*>(a.x_rot + ob);
#pragma unroll
        for (int k = 0; k < 4; ++k)
          xr[k] = f32x4{y[4 * k] * inv_sqrt_h, y[4 * k + 1] * inv_sqrt_h, y[4 * k + 2] * inv_sqrt_h,
                        y[4 * k + 3] * inv_sqrt_h};
      }
    };
    if constexpr (MAXT > 512) {
#pragma unroll 1
      for (int j = 0; j < J; ++j) slot(j);
    } else {
#pragma unroll
      for (int j = 0; j < J; ++j) slot(j);
    }
    if (lane == 0) a.s[tok] = s32;
    wave_sync_lds();  // every lane's gathers are done before the next row is staged
  }
}

// ---- weights: one workgroup per row, fp64 -----------------------------------
template <bool BF16, int BITS>
__global__ void __launch_bounds__(256) wq_kernel(const WqArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  double* buf = reinterpret_cast<double*>(smem);
  double* thr = buf + a.d;
  double* red = thr + 256;
  const int d = a.d, h = a.h, tid = threadIdx.x, nt = blockDim.x;
  const int64_t o = blockIdx.x;
  for (int i = tid; i < a.nthr; i += nt) thr[i] = a.thr[i];
  for (int i = tid; i < d; i += nt) {
    const int p = min((unsigned)a.perm[i], (unsigned)(d - 1));
    double v;
    if (BF16) v = (double)__uint_as_float((uint32_t)static_cast<const uint16_t*>(a.W)[o * d + p] << 16);
    else v = (double)static_cast<const float*>(a.W)[o * d + p];
    buf[i] = a.sign[i] < 0 ? -v : v;
  }
  __syncthreads();
  for (int st = 1; st < h; st <<= 1) {
    for (int p = tid; p < d / 2; p += nt) {
      const int i = (p / st) * (2 * st) + (p % st);
      const double x0 = buf[i], x1 = buf[i + st];
      buf[i] = x0 + x1;
      buf[i + st] = x0 - x1;
    }
    __syncthreads();
  }
  const double sh = sqrt((double)h);
  double part = 0.0;
  for (int i = tid; i < d; i += nt) {
    const double v = buf[i] / sh;
    buf[i] = v;
    part += v * v;
  }
  for (int off = 32; off >= 1; off >>= 1) part += __shfl_xor(part, off);
  if ((tid & 63) == 0) red[tid >> 6] = part;
  __syncthreads();
  double ss = 0.0;
  for (int w = 0; w < nt / 64; ++w) ss += red[w];
  const double n = sqrt(ss);
  const double den = n + OQ_EPS;
  // groups of 8 indices = BITS bytes of the row's little-endian bit stream
  // (d * BITS is a whole number of bytes, so a last short group ends on a byte)
  const size_t row_bytes = (size_t)d * BITS / 8;
  for (int q = tid; q < (d + 7) / 8; q += nt) {
    uint64_t v = 0;
    const int cnt = min(8, d - 8 * q);
    for (int k = 0; k < cnt; ++k) {
      const double u = buf[8 * q + k] / den;
      int lo = 0;
      for (int step = 128; step >= 1; step >>= 1)
        if (lo + step <= a.nthr && thr[lo + step - 1] < u) lo += step;
      v |= (uint64_t)lo << (k * BITS);
    }
    uint8_t* dst = a.w_idx + o * row_bytes + (size_t)q * BITS;
    for (int b = 0; b < cnt * BITS / 8; ++b) dst[b] = (uint8_t)(v >> (8 * b));
  }
  if (tid == 0) a.w_norm[o] = (float)n;
}

// Allow up to the 160 KB of LDS of a gfx950 CU (set on every launch: the
// attribute belongs to the kernel and device, and the call is cheap, so no
// host-side memo is kept).
template <typename K>
hipError_t allow_lds(K kernel) {
  return hipFuncSetAttribute(reinterpret_cast<const void*>(kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                             160 * 1024);
}

hipError_t device_cus(int* cus) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  return hipDeviceGetAttribute(cus, hipDeviceAttributeMultiprocessorCount, dev);
}

// Persistent grid: as many workgroups as are resident at once (capped by the
// plan's own count), each looping over tokens.
template <typename K>
hipError_t resident_grid(K kernel, const RqPlan& p, int* grid) {
  int per_cu = 0, cus = 0;
  hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, p.threads, p.lds);
  if (e != hipSuccess) return e;
  if ((e = device_cus(&cus)) != hipSuccess) return e;
  const int64_t resident = (int64_t)(per_cu > 0 ? per_cu : 1) * cus;
  *grid = (int)(p.grid < resident ? p.grid : resident);
  return hipSuccess;
}

template <int LOG2H, bool BF16, int BITS>
hipError_t rq_go(const RqArgs& a, const RqPlan& p, hipStream_t st) {
  auto kern = rq_act_kernel<LOG2H, BF16, BITS>;
  hipError_t e = allow_lds(kern);
  int grid = 0;
  if (e == hipSuccess) e = resident_grid(kern, p, &grid);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(p.threads), p.lds, st, a, p.ns, p.tpw, p.pad);
  return hipGetLastError();
}

template <int LOG2H, bool BF16>
hipError_t rq_dispatch_bits(const RqArgs& a, int bits, const RqPlan& p, hipStream_t st) {
  switch (bits) {
    case 2: return rq_go<LOG2H, BF16, 2>(a, p, st);
    case 3: return rq_go<LOG2H, BF16, 3>(a, p, st);
    case 4: return rq_go<LOG2H, BF16, 4>(a, p, st);
    case 6: return rq_go<LOG2H, BF16, 6>(a, p, st);
    case 8: return rq_go<LOG2H, BF16, 8>(a, p, st);
    default: return hipErrorInvalidValue;
  }
}

template <bool BF16, int BITS>
hipError_t wq_go(const WqArgs& a, size_t lds, hipStream_t st) {
  hipError_t e = allow_lds(&wq_kernel<BF16, BITS>);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((wq_kernel<BF16, BITS>), dim3(a.d_out), dim3(256), lds, st, a);
  return hipGetLastError();
}

template <bool BF16>
hipError_t rq_dispatch(const RqArgs& a, int bits, const RqPlan& p, hipStream_t st) {
  switch (a.log2h) {
    case 1: return rq_dispatch_bits<1, BF16>(a, bits, p, st);
    case 2: return rq_dispatch_bits<2, BF16>(a, bits, p, st);
    case 3: return rq_dispatch_bits<3, BF16>(a, bits, p, st);
    case 4: return rq_dispatch_bits<4, BF16>(a, bits, p, st);
    case 5: return rq_dispatch_bits<5, BF16>(a, bits, p, st);
    case 6: return rq_dispatch_bits<6, BF16>(a, bits, p, st);
    case 7: return rq_dispatch_bits<7, BF16>(a, bits, p, st);
    case 8: return rq_dispatch_bits<8, BF16>(a, bits, p, st);
    default: return hipErrorInvalidValue;
  }
}

template <int LOG2H, bool BF16, int BITS, int J, int MAXT>
hipError_t rqw_go(const RqArgs& a, const RqPlan& p, hipStream_t st) {
  if (p.threads > MAXT) return hipErrorInvalidValue;
  auto kern = rq_wave_kernel<LOG2H, BF16, BITS, J, MAXT>;
  hipError_t e = allow_lds(kern);
  int grid = 0;
  if (e == hipSuccess) e = resident_grid(kern, p, &grid);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(p.threads), p.lds, st, a, p.wpb);
  return hipGetLastError();
}

template <int LOG2H, bool BF16, int BITS>
hipError_t rqw_dispatch_j(const RqArgs& a, const RqPlan& p, hipStream_t st) {
  // 12 wavefronts (J <= 3, from 3072 tokens on) or 8
  const bool big = p.threads > 512;
  switch (p.wave_j) {
    case 1: return big ? rqw_go<LOG2H, BF16, BITS, 1, 768>(a, p, st) : rqw_go<LOG2H, BF16, BITS, 1, 512>(a, p, st);
    case 2: return big ? rqw_go<LOG2H, BF16, BITS, 2, 768>(a, p, st) : rqw_go<LOG2H, BF16, BITS, 2, 512>(a, p, st);
    case 3:
      if constexpr (BF16)
        return big ? rqw_go<LOG2H, BF16, BITS, 3, 768>(a, p, st) : rqw_go<LOG2H, BF16, BITS, 3, 512>(a, p, st);
      else return hipErrorInvalidValue;
    case 4:
      if constexpr (BF16) return rqw_go<LOG2H, BF16, BITS, 4, 512>(a, p, st);
      else return hipErrorInvalidValue;
    case 5:
      if constexpr (BF16) return rqw_go<LOG2H, BF16, BITS, 5, 512>(a, p, st);
      else return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
  }
}

template <bool BF16>
hipError_t rqw_dispatch(const RqArgs& a, int bits, const RqPlan& p, hipStream_t st) {
  auto by_bits = [&](auto lg) -> hipError_t {
    constexpr int LG = decltype(lg)::value;
    switch (bits) {
      case 2: return rqw_dispatch_j<LG, BF16, 2>(a, p, st);
      case 3: return rqw_dispatch_j<LG, BF16, 3>(a, p, st);
      case 4: return rqw_dispatch_j<LG, BF16, 4>(a, p, st);
      case 6: return rqw_dispatch_j<LG, BF16, 6>(a, p, st);
      case 8: return rqw_dispatch_j<LG, BF16, 8>(a, p, st);
      default: return hipErrorInvalidValue;
    }
  };
  switch (a.log2h) {
    case 6: return by_bits(std::integral_constant<int, 6>{});
    case 8: return by_bits(std::integral_constant<int, 8>{});
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

bool rq_plan(int32_t d, int32_t log2h, bool bf16, int32_t bits, int64_t T, int G, RqPlan* p) {
  if (log2h < 1 || log2h > 8 || d % 16 != 0 || d % (1 << log2h) != 0) return false;
  const int ns = d / 16;
  p->wave_j = 0;
  p->wpb = 0;
  p->pad = 1;
  // one wavefront per token: d = 1024 J with J <= 5 (bf16) or J <= 2 (fp32: the
  // prefetched row takes twice the registers), h in {64, 256}, grid search
  if (ns % 64 == 0 && ns / 64 <= (bf16 ? 5 : 2) && (log2h == 6 || log2h == 8) && G > 0 &&
      (bits > 6 || G <= kByteCells)) {
    const int J = ns / 64;
    const int es = bf16 ? 2 : 4;
    // J <= 3: 768 threads, 3 wavefronts per SIMD; J = 4, 5: 512 threads (the
    // kernels' register budgets); fewer if the row buffers exceed the LDS.
    // Below 3072 tokens 8 wavefronts per workgroup spread the tokens over more
    // CUs (measured ~1 us faster at 256-1024 tokens, slower from 4608 on).
    int wpb = J <= 3 && T >= 3072 ? 12 : 8;
    while (wpb > 4 && rqw_layout(d, log2h, es, G, wpb).total > 160 * 1024) wpb -= 4;
    const RqwLayout L = rqw_layout(d, log2h, es, G, wpb);
    // the set-up gives each thread at most 16 of the d table entries: 64 wpb >= d / 16
    if (L.total <= 160 * 1024 && 64 * wpb * 16 >= d) {
      p->ns = ns;
      p->tpw = 1;
      p->wave_j = J;
      p->wpb = wpb;
      p->threads = 64 * wpb;
      p->lds = L.total;
      const int64_t groups = (T + wpb - 1) / wpb;
      p->grid = (int)(groups < (1 << 30) ? (groups > 0 ? groups : 1) : (1 << 30));
      return true;
    }
  }
  int tpw;
  if (ns % 64 == 0 && ns <= 768) tpw = 1;
  else if (ns < 64 && (ns & (ns - 1)) == 0) tpw = 256 / ns;
  else return false;
  p->ns = ns;
  p->tpw = tpw;
  p->threads = ns * tpw;
  p->pad = 1;
  if (rq_layout(d, log2h, bf16 ? 2 : 4, tpw, G, 1).total > 160 * 1024) p->pad = 0;   // pad only if it fits
  const RqLayout L = rq_layout(d, log2h, bf16 ? 2 : 4, tpw, G, p->pad);
  p->lds = L.total;
  if (p->lds > 160 * 1024) return false;
  const int64_t groups = (T + tpw - 1) / tpw;
  p->grid = (int)(groups < (1 << 30) ? (groups > 0 ? groups : 1) : (1 << 30));  // capped at launch by residency
  return true;
}

hipError_t rq_launch(const RqArgs& a, bool bf16, int bits, const RqPlan& p, hipStream_t st) {
  if (p.wave_j > 0) return bf16 ? rqw_dispatch<true>(a, bits, p, st) : rqw_dispatch<false>(a, bits, p, st);
  return bf16 ? rq_dispatch<true>(a, bits, p, st) : rq_dispatch<false>(a, bits, p, st);
}

hipError_t wq_launch(const WqArgs& a, bool bf16, int bits, hipStream_t st) {
  const size_t lds = (size_t)a.d * 8 + 256 * 8 + 4 * 8;
  if (bf16) {
    switch (bits) {
      case 2: return wq_go<true, 2>(a, lds, st);
      case 3: return wq_go<true, 3>(a, lds, st);
      case 4: return wq_go<true, 4>(a, lds, st);
      case 6: return wq_go<true, 6>(a, lds, st);
      case 8: return wq_go<true, 8>(a, lds, st);
    }
  } else {
    switch (bits) {
      case 2: return wq_go<false, 2>(a, lds, st);
      case 3: return wq_go<false, 3>(a, lds, st);
      case 4: return wq_go<false, 4>(a, lds, st);
      case 6: return wq_go<false, 6>(a, lds, st);
      case 8: return wq_go<false, 8>(a, lds, st);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace oq
