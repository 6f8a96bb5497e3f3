// INT4 round-to-nearest weight-only linear (W4A16) for the AdaLN modulation
// projections, which stay outside the OrbitQuant codebooks: their
// timestep-dependent scale and shift cannot absorb the rotation, and the
// method keeps them at INT4 weight round-to-nearest ("OrbitQuant:
// data-agnostic quantization for image and video", rcap.io summary:
// deployment paragraph and AdaLN caveat; "FLUX.3 Image Klein OrbitQuant W4A8" model
// card, Components table).
//
// Scheme: symmetric signed codes q in [-8, 7]; one fp32 scale
// s = max|w| / 7 per output row and group of `group` input columns;
// q = clamp(rint(w / s), -8, 7) with the stored fp32 s (fp64 division);
// codes packed as two's-complement nibbles, code k in bits [4k, 4k + 4) of
// the row.  y[t][o] = sum_g s[o][g] sum_{k in g} q[o][k] x[t][k] (+ bias[o]).
//
// rtn_kernel  : the offline quantizer, one wavefront per (row, group), fp64.
// w4a_kernel  : the product.  The modulation input is one row per image of
//   the batch, so T is tiny and the kernel streams the packed weights once
//   from HBM (0.5 byte per weight): bound by HBM bandwidth.  A workgroup owns
//   32 output features and up to 16 tokens; its 8 wavefronts split d_in.  Codes are
//   decoded through a 256-entry LDS table (one byte = two codes -> two 16-bit
//   values) into the B operand of v_mfma_f32_16x16x32_{bf16,f16} (codes are
//   exact in both types), activations are the A operand as loaded, fp32
//   accumulation; each group's sum is scaled into a running total, and the 8
//   partial tiles are summed through LDS in a fixed order.

#include "oq_internal.h"

namespace oq {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 half8 __attribute__((ext_vector_type(8)));

constexpr int kWaves = 8;            // split of d_in inside a workgroup
constexpr int kThreads = 64 * kWaves;
constexpr int kFeat = 32;            // output features per workgroup (two MFMA tiles)
constexpr int kBatch = 3;            // 128-wide K chunks whose weights are loaded at once
constexpr int kRedStride = kFeat + 1;  // padded row of the reduction buffer
constexpr int kTabBytes = 1024;
constexpr int kRedBytes = kWaves * 16 * kRedStride * 4;
constexpr int kXLdsMax = 96 * 1024;  // staged activation rows

// ---- offline quantizer ---------------------------------------------------------
template <bool BF16>
__global__ void __launch_bounds__(256) rtn_kernel(const RtnArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t wid = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int ng = a.K / a.group;
  if (wid >= (int64_t)a.N * ng) return;   // whole wavefronts exit together
  const int64_t row = wid / ng;
  const int g = (int)(wid % ng);
  const int64_t base = row * a.K + (int64_t)g * a.group;
  auto ld = [&](int64_t i) -> double {
    if (BF16) return (double)__uint_as_float((uint32_t)static_cast<const uint16_t*>(a.W)[i] << 16);
    return (double)static_cast<const float*>(a.W)[i];
  };
  double m = 0.0;
  for (int k = lane; k < a.group; k += 64) m = fmax(m, fabs(ld(base + k)));
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) m = fmax(m, __shfl_xor(m, o));
  const float s = (float)(m / 7.0);
  const double sd = (double)s;
  // lane handles bytes (code pairs) lane, lane + 64, ...
  for (int b = lane; b < a.group / 2; b += 64) {
    uint32_t nib[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      int q = 0;
      if (sd > 0.0) q = (int)fmin(fmax(rint(ld(base + 2 * b + e) / sd), -8.0), 7.0);
      nib[e] = (uint32_t)q & 15u;
    }
    a.q[(base >> 1) + b] = (uint8_t)(nib[0] | (nib[1] << 4));
  }
  if (lane == 0) a.scale[row * ng + g] = s;
}

// ---- the product -------------------------------------------------------------------
template <bool BF16>
__device__ __forceinline__ f32x4 mfma(const u32x4 a, const u32x4 b, const f32x4 c) {
  if constexpr (BF16)
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                   0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, a), __builtin_bit_cast(half8, b), c, 0,
                                                  0, 0);
}

// The 8 codes of word w (code j in bits [4j, 4j+4)) as 8 16-bit values: one
// table entry per byte holds the values of its low and high nibble.
__device__ __forceinline__ u32x4 decode8(const uint32_t* tab, uint32_t w) {
  return u32x4{tab[w & 0xFFu], tab[(w >> 8) & 0xFFu], tab[(w >> 16) & 0xFFu], tab[w >> 24]};
}

// v_mfma_f32_16x16x32: lane l holds A[l % 16][8 (l / 16) .. +8], B[8 (l / 16) .. +8][l % 16]
// and D[4 (l / 16) .. +4][l % 16].  A = activations (rows = tokens), B = decoded
// codes (columns = output features).  Lane (l % 16, j = l / 16) loads the 16
// bytes (32 codes) k = 128 c + 32 j + [0, 32) of its feature for 128-wide chunk
// c; MFMA step s takes codes 8 s .. 8 s + 7 of them and the activations of the
// same 8 k, so each step sums a permutation of 32 columns of chunk c.
//
// A workgroup owns kFeat = 32 features (two 16-wide B tiles sharing each A
// fragment) and up to 16 tokens, whose rows are staged once in LDS (row stride
// padded by 16 bytes so that the 16 rows of a fragment read fall in distinct
// banks).  Each wavefront issues the weight loads of kBatch chunks at once.
template <bool BF16>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(6)))
w4a_kernel(const W4Args a) {   // 6 wavefronts per SIMD: 3 workgroups per CU, the 576 of the FLUX shape at once
  extern __shared__ __align__(16) unsigned char smem[];
  uint32_t* tab = reinterpret_cast<uint32_t*>(smem);
  float* red = reinterpret_cast<float*>(smem + kTabBytes);
  unsigned char* xs = smem + kTabBytes + kRedBytes;

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int lr = lane & 15, j = lane >> 4;
  const int n0 = blockIdx.x * kFeat;
  const int64_t t0 = (int64_t)blockIdx.y * a.tt;
  const int K = a.K, N = a.N;
  const int rows = a.T - t0 < a.tt ? (int)(a.T - t0) : a.tt;
  const int xstride = 2 * K + 16;

  // this wavefront's 128-wide chunks
  const int C = K / 128;
  const int c0 = (int)((int64_t)C * wave / kWaves), c1 = (int)((int64_t)C * (wave + 1) / kWaves);
  const int cpg = a.group / 128;   // chunks per group

  // weights of the first batch (HBM): issued first, the longest wait
  int nf[2];
  const uint8_t* qrow[2];
  const float* srow[2];
#pragma unroll
  for (int f = 0; f < 2; ++f) {
    const int nn = n0 + 16 * f + lr;
    nf[f] = nn < N ? nn : N - 1;
    qrow[f] = a.q + (size_t)nf[f] * (K / 2) + j * 16;
    srow[f] = a.scale + (size_t)nf[f] * (K / a.group);
  }
  u32x4 wq[kBatch][2];
  float scl[kBatch][2];   // scale of each chunk's group, loaded with its codes
  auto wload = [&](int cb) {
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const int c = cb + i < c1 ? cb + i : c1 - 1;
#pragma unroll
      for (int f = 0; f < 2; ++f) {
        wq[i][f] = *reinterpret_cast<const u32x4*>(qrow[f] + (size_t)c * 64);
        scl[i][f] = srow[f][c / cpg];
      }
    }
  };
  if (c0 < c1) wload(c0);

  // activation rows -> LDS (16-byte pieces), nibble-pair table
  {
    const uint16_t* xg = static_cast<const uint16_t*>(a.x) + (size_t)t0 * K;
    const int per_row = K / 8, np = rows * per_row;
    for (int p0 = 0; p0 < np; p0 += kThreads * 2) {
      u32x4 v[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int p = p0 + tid + u * kThreads;
        if (p < np) v[u] = *reinterpret_cast<const u32x4*>(xg + (size_t)p * 8);
      }
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int p = p0 + tid + u * kThreads;
        if (p < np) *reinterpret_cast<u32x4*>(xs + (p / per_row) * xstride + (p % per_row) * 16) = v[u];
      }
    }
  }
  if (tid < 256) {
    // byte e = (hi nibble, lo nibble) of two's-complement codes -> two exact 16-bit values
    const int lo = (tid & 15) - ((tid & 8) << 1), hi = (tid >> 4) - ((tid & 128) >> 3);
    uint32_t vlo, vhi;
    if (BF16) {
      vlo = __float_as_uint((float)lo) >> 16;   // small integers: the top 16 bits are exact
      vhi = __float_as_uint((float)hi) >> 16;
    } else {
      vlo = __builtin_bit_cast(uint16_t, (_Float16)lo);
      vhi = __builtin_bit_cast(uint16_t, (_Float16)hi);
    }
    tab[tid] = vlo | (vhi << 16);
  }
  __syncthreads();

  const bool trow = lr < rows;
  const unsigned char* xa = xs + lr * xstride + j * 64;
  f32x4 tot[2], acc[2];
#pragma unroll
  for (int f = 0; f < 2; ++f) tot[f] = acc[f] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int cb = c0; cb < c1; cb += kBatch) {
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const int c = cb + i;
      if (c < c1) {
#pragma unroll
        for (int st = 0; st < 4; ++st) {
          const u32x4 av = trow ? *reinterpret_cast<const u32x4*>(xa + c * 256 + st * 16) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
          for (int f = 0; f < 2; ++f) acc[f] = mfma<BF16>(av, decode8(tab, wq[i][f][st]), acc[f]);
        }
        // end of a group (or of this wavefront's range): scale it into the total
        if ((c + 1) % cpg == 0 || c + 1 == c1) {
#pragma unroll
          for (int f = 0; f < 2; ++f) {
#pragma unroll
            for (int r = 0; r < 4; ++r) tot[f][r] = fmaf(scl[i][f], acc[f][r], tot[f][r]);
            acc[f] = f32x4{0.f, 0.f, 0.f, 0.f};
          }
        }
      }
    }
    if (cb + kBatch < c1) wload(cb + kBatch);
  }

  // partial tiles -> LDS, then a fixed-order sum over the wavefronts
  float* rw = red + wave * 16 * kRedStride;
#pragma unroll
  for (int f = 0; f < 2; ++f)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = 4 * j + r;
      if (row < rows) rw[row * kRedStride + 16 * f + lr] = tot[f][r];
    }
  __syncthreads();
  for (int e = tid; e < rows * kFeat; e += kThreads) {
    const int row = e / kFeat, col = e % kFeat;
    if (n0 + col >= N) continue;
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) v += red[(w * 16 + row) * kRedStride + col];
    if (a.bias) v += a.bias[n0 + col];
    a.y[(size_t)(t0 + row) * N + n0 + col] = v;
  }
}

}  // namespace

hipError_t rtn_launch(const RtnArgs& a, bool bf16, hipStream_t st) {
  const int64_t waves = (int64_t)a.N * (a.K / a.group);
  if (waves == 0) return hipSuccess;
  const int64_t grid = (waves + 3) / 4;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
  if (bf16) hipLaunchKernelGGL(rtn_kernel<true>, dim3((unsigned)grid), dim3(256), 0, st, a);
  else hipLaunchKernelGGL(rtn_kernel<false>, dim3((unsigned)grid), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t w4a_launch(const W4Args& a_in, bool bf16, hipStream_t st) {
  if (a_in.T == 0 || a_in.N == 0) return hipSuccess;
  W4Args a = a_in;
  // tokens per workgroup: up to the 16 rows of the MFMA tile, as many as fit the LDS
  const int xstride = 2 * a.K + 16;
  const int64_t fit = kXLdsMax / xstride;
  if (fit < 1) return hipErrorInvalidValue;
  a.tt = (int)(fit < 16 ? fit : 16);
  const int64_t tt = a.tt < a.T ? a.tt : a.T;
  const int64_t gy = (a.T + a.tt - 1) / a.tt;   // token tiles
  if (gy > 65535) return hipErrorInvalidValue;
  const size_t lds = kTabBytes + kRedBytes + (size_t)tt * xstride;
  {
    // set on every launch (cheap; no host-side memo is kept)
    const void* fn = bf16 ? (const void*)w4a_kernel<true> : (const void*)w4a_kernel<false>;
    hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       kTabBytes + kRedBytes + kXLdsMax);
    if (e != hipSuccess) return e;
  }
  const dim3 grid((unsigned)((a.N + kFeat - 1) / kFeat), (unsigned)gy);
  if (bf16) hipLaunchKernelGGL(w4a_kernel<true>, grid, dim3(kThreads), lds, st, a);
  else hipLaunchKernelGGL(w4a_kernel<false>, grid, dim3(kThreads), lds, st, a);
  return hipGetLastError();
}

}  // namespace oq
