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
//      is orthogonal; per-lane fp32 partials, fp64 across lanes;
//   2. signed gather from LDS: lane holds y_r = sign[i_r] x[perm[i_r]]; the
//      16 LDS addresses and sign words are loop-invariant registers;
//   3. block FWHT: a 16-point in-register transform over the top 4 index
//      bits, an LDS transpose inside the wavefront, then the remaining
//      log2(h) - 4 butterfly stages in registers (h <= 16: one pass);
//   4. threshold search: a uniform grid over the threshold range whose cells
//      hold at most one threshold, so idx = base[cell] + (u > theta[cell]),
//      decided by the sign of one fma;
//   5. guard: a coordinate whose fp32 value lies within a certified rounding
//      bound of its threshold (2 (log2 h + 1) 2^-24 L1(block) / (sqrt(h) s)
//      for the butterflies, plus 16 ulp of |theta| for s and the scaling) is
//      recomputed in fp64 by the wavefront (rare) before its index is set;
//   6. LSB-first packing of 2 / 4 / 8-bit indices, one 4 / 8 / 16-byte store.
//
// Weight kernel (offline): one workgroup per row, fp64 throughout.
#include <cmath>

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

struct RqLayout {
  size_t lut, thr, row, trans, red, total, row_stride;  // row_stride: bytes of one parity buffer
};

__host__ __device__ inline RqLayout rq_layout(int d, int log2h, int es, int tpw, int G) {
  RqLayout L;
  const int h = 1 << log2h;
  L.lut = 0;
  L.thr = align16(8 * (size_t)(G > 0 ? G : 1));
  L.row = L.thr + 256 * 4;
  L.row_stride = align16((size_t)tpw * d * es);
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

template <int LOG2H, bool BF16, int BITS>
__global__ void __launch_bounds__(768) rq_act_kernel(const RqArgs a, const int NS, const int TPW) {
  constexpr int H = 1 << LOG2H;
  constexpr int ES = BF16 ? 2 : 4;
  constexpr bool TWO_PASS = LOG2H > 4;
  constexpr int BL = TWO_PASS ? H / 16 : 1;        // lanes per Hadamard block
  constexpr int BPL = TWO_PASS ? 1 : 16 / H;       // Hadamard blocks per lane (one pass)
  constexpr float kGam = 2.0f * (LOG2H + 1) * 5.9604644775390625e-8f;  // 2 (m+1) 2^-24
  constexpr float kRel = 16.0f * 5.9604644775390625e-8f;               // 16 ulp of |theta|

  const int d = a.d;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int tl = tid / NS;          // token within the workgroup iteration
  const int sl = tid - tl * NS;     // 16-coordinate slot within the token
  const int G = a.G;
  const int nthr = a.nthr;

  extern __shared__ __align__(16) unsigned char smem[];
  const RqLayout Ly = rq_layout(d, LOG2H, ES, TPW, G);
  int2* lut = reinterpret_cast<int2*>(smem + Ly.lut);
  float* thr = reinterpret_cast<float*>(smem + Ly.thr);
  double* red = reinterpret_cast<double*>(smem + Ly.red);

  // ---- thresholds and the search grid --------------------------------------
  for (int i = tid; i < 256; i += blockDim.x) thr[i] = i < nthr ? a.thr[i] : INFINITY;
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
    addr[r] = (uint32_t)(Ly.row + ((size_t)tl * d + src) * ES);
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
    float q0 = 0.f, q1 = 0.f, q2 = 0.f, q3 = 0.f;
    {
      u32x4* rowdst = reinterpret_cast<u32x4*>(smem + Ly.row + paroff + ((size_t)tl * d + 16 * sl) * ES);
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
            q0 = fmaf(e0, e0, q0);
            q1 = fmaf(e1, e1, q1);
            q2 = fmaf(e2, e2, q2);
            q3 = fmaf(e3, e3, q3);
          }
        }
      } else {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const float e0 = __uint_as_float(raw[k][0]), e1 = __uint_as_float(raw[k][1]);
          const float e2 = __uint_as_float(raw[k][2]), e3 = __uint_as_float(raw[k][3]);
          q0 = fmaf(e0, e0, q0);
          q1 = fmaf(e1, e1, q1);
          q2 = fmaf(e2, e2, q2);
          q3 = fmaf(e3, e3, q3);
        }
      }
    }
    // the next token's row is in flight while this one is processed
    if (g + gridDim.x < ngroups) fetch(g + gridDim.x);
    double ss = (double)((q0 + q1) + (q2 + q3));
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
    uint64_t pk0 = 0, pk1 = 0;  // packed indices (pk1 only for 8-bit)
    uint32_t flags = 0;
    auto put = [&](int r, int idx) {
      if (BITS == 8) {
        if (r < 8) pk0 |= (uint64_t)idx << (8 * r);
        else pk1 |= (uint64_t)idx << (8 * (r - 8));
      } else {
        pk0 |= (uint64_t)idx << (BITS * r);
      }
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
          const float radb = kGam * l1[TWO_PASS ? 0 : r / (16 / BPL)] * c;
          const float th = __int_as_float(e[q].x);
          const float dd = fmaf(y[r], c, -th);
          put(r, e[q].y + (dd > 0.f ? 1 : 0));
          flags |= (fabsf(dd) < fmaf(fabsf(th), kRel, radb) ? 1u : 0u) << r;
        }
      }
    } else {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float v = y[r];
        const float radb = kGam * l1[TWO_PASS ? 0 : r / (16 / BPL)] * c;
        int lo = 0;
        for (int step = 128; step >= 1; step >>= 1)
          if (lo + step <= nthr && fmaf(v, c, -thr[lo + step - 1]) > 0.f) lo += step;
        bool near = false;
        if (lo > 0) {
          const float th = thr[lo - 1];
          near |= fabsf(fmaf(v, c, -th)) < fmaf(fabsf(th), kRel, radb);
        }
        if (lo < nthr) {
          const float th = thr[lo];
          near |= fabsf(fmaf(v, c, -th)) < fmaf(fabsf(th), kRel, radb);
        }
        put(r, lo);
        flags |= (near ? 1u : 0u) << r;
      }
    }
    if (!valid) flags = 0;

    // fp64 recheck of guarded coordinates, by the whole wavefront
    while (true) {
      const uint64_t bal = __ballot(flags != 0);
      if (bal == 0) break;
      const int L = __ffsll((unsigned long long)bal) - 1;
      const uint32_t fl = __shfl(flags, L);
      const int r = __ffs(fl) - 1;
      const int slL = __shfl(sl, L);
      const int tlL = __shfl(tl, L);
      const int gi = 16 * slL + r;
      const int b = gi >> LOG2H;
      const int j = gi & (H - 1);
      double part = 0.0;
      if (tl == tlL) {
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
      part = wave_sum_d(part);
      if (lane == L) {
        const double u = part / (sqrt((double)H) * (s64 + OQ_EPS));
        const uint64_t nidx = (uint64_t)count_below_f64(thr, nthr, u);
        constexpr uint64_t mask = (1ull << BITS) - 1;
        if (BITS == 8) {
          if (r < 8) pk0 = (pk0 & ~(mask << (8 * r))) | (nidx << (8 * r));
          else pk1 = (pk1 & ~(mask << (8 * (r - 8)))) | (nidx << (8 * (r - 8)));
        } else {
          pk0 = (pk0 & ~(mask << (BITS * r))) | (nidx << (BITS * r));
        }
        flags &= ~(1u << r);
      }
    }

    // ---- 6. stores ----------------------------------------------------------------
    if (valid) {
      const int64_t ob = tok * (int64_t)d + 16 * sl;  // first coordinate of this slot
      if (BITS == 4) *reinterpret_cast<uint64_t*>(a.x_idx + ob / 2) = pk0;
      else if (BITS == 2) *reinterpret_cast<uint32_t*>(a.x_idx + ob / 4) = (uint32_t)pk0;
      else *reinterpret_cast<u64x2*>(a.x_idx + ob) = u64x2{pk0, pk1};
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
  constexpr int PER = 8 / BITS;
  for (int q = tid; q < d / PER; q += nt) {
    uint32_t byte = 0;
    for (int k = 0; k < PER; ++k) {
      const double u = buf[q * PER + k] / den;
      int lo = 0;
      for (int step = 128; step >= 1; step >>= 1)
        if (lo + step <= a.nthr && thr[lo + step - 1] < u) lo += step;
      byte |= (uint32_t)lo << (k * BITS);
    }
    a.w_idx[o * (d / PER) + q] = (uint8_t)byte;
  }
  if (tid == 0) a.w_norm[o] = (float)n;
}

// Allow up to the 160 KB of LDS of a gfx950 CU (once per kernel instantiation).
template <typename K>
hipError_t allow_lds(K kernel, bool& done) {
  if (done) return hipSuccess;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
  if (e == hipSuccess) done = true;
  return e;
}

int device_cus() {
  static int cus = 0;
  if (cus == 0) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      cus = 256;
  }
  return cus;
}

template <int LOG2H, bool BF16, int BITS>
hipError_t rq_go(const RqArgs& a, const RqPlan& p, hipStream_t st) {
  static bool attr = false;
  hipError_t e = allow_lds(&rq_act_kernel<LOG2H, BF16, BITS>, attr);
  if (e != hipSuccess) return e;
  // persistent grid: as many workgroups as are resident at once, each looping over tokens
  int per_cu = 0;
  e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, rq_act_kernel<LOG2H, BF16, BITS>, p.threads, p.lds);
  if (e != hipSuccess) return e;
  const int64_t resident = (int64_t)(per_cu > 0 ? per_cu : 1) * device_cus();
  const int grid = (int)(p.grid < resident ? p.grid : resident);
  hipLaunchKernelGGL((rq_act_kernel<LOG2H, BF16, BITS>), dim3(grid), dim3(p.threads), p.lds, st, a, p.ns, p.tpw);
  return hipGetLastError();
}

template <int LOG2H, bool BF16>
hipError_t rq_dispatch_bits(const RqArgs& a, int bits, const RqPlan& p, hipStream_t st) {
  switch (bits) {
    case 2: return rq_go<LOG2H, BF16, 2>(a, p, st);
    case 4: return rq_go<LOG2H, BF16, 4>(a, p, st);
    case 8: return rq_go<LOG2H, BF16, 8>(a, p, st);
    default: return hipErrorInvalidValue;
  }
}

template <bool BF16, int BITS>
hipError_t wq_go(const WqArgs& a, size_t lds, hipStream_t st) {
  static bool attr = false;
  hipError_t e = allow_lds(&wq_kernel<BF16, BITS>, attr);
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

}  // namespace

bool rq_plan(int32_t d, int32_t log2h, bool bf16, int64_t T, int G, RqPlan* p) {
  if (log2h < 1 || log2h > 8 || d % 16 != 0 || d % (1 << log2h) != 0) return false;
  const int ns = d / 16;
  int tpw;
  if (ns % 64 == 0 && ns <= 768) tpw = 1;
  else if (ns < 64 && (ns & (ns - 1)) == 0) tpw = 256 / ns;
  else return false;
  p->ns = ns;
  p->tpw = tpw;
  p->threads = ns * tpw;
  const RqLayout L = rq_layout(d, log2h, bf16 ? 2 : 4, tpw, G);
  p->lds = L.total;
  if (p->lds > 160 * 1024) return false;
  const int64_t groups = (T + tpw - 1) / tpw;
  p->grid = (int)(groups < (1 << 30) ? (groups > 0 ? groups : 1) : (1 << 30));  // capped at launch by residency
  return true;
}

hipError_t rq_launch(const RqArgs& a, bool bf16, int bits, const RqPlan& p, hipStream_t st) {
  return bf16 ? rq_dispatch<true>(a, bits, p, st) : rq_dispatch<false>(a, bits, p, st);
}

hipError_t wq_launch(const WqArgs& a, bool bf16, int bits, hipStream_t st) {
  const size_t lds = (size_t)a.d * 8 + 256 * 8 + 4 * 8;
  if (bf16) {
    switch (bits) {
      case 2: return wq_go<true, 2>(a, lds, st);
      case 4: return wq_go<true, 4>(a, lds, st);
      case 8: return wq_go<true, 8>(a, lds, st);
    }
  } else {
    switch (bits) {
      case 2: return wq_go<false, 2>(a, lds, st);
      case 4: return wq_go<false, 4>(a, lds, st);
      case 8: return wq_go<false, 8>(a, lds, st);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace oq
