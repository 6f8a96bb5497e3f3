/*
 * oq.h -- C ABI of liboq, the OrbitQuant quantized linear layer on AMD
 * Instinct MI355X (gfx950).
 *
 * The method (pages: "OrbitQuant: data-agnostic quantization for image and
 * video", rcap.io summary of the paper -- mechanism paragraphs and the
 * offline / online pseudo-code; "OrbitQuant quantizes FLUX.1 and Wan 2.1
 * with no calibration data", aiweekly.co):
 *
 *   offline, once per input dimension d:
 *     rotation[d]    = RPBH(d): random permutation, random sign flips,
 *                      block-diagonal Walsh-Hadamard blocks of size h
 *     codebook[d, b] = Lloyd-Max quantizer with 2^b centroids for the fixed
 *                      marginal f_d of one coordinate of a rotated unit vector
 *   offline, per weight matrix W (d_out x d_in):
 *     W_rot = W R^T; n = row norms; w_idx = nearest centroid of W_rot / n
 *   online, per token x:
 *     x_rot = R x; s = ||x_rot||; x_idx = nearest centroid of x_rot / (s + eps)
 *   layer output (the rotation cancels: W R^T R x = W x):
 *     y[t][o] = s_t n_o sum_k c_a[x_idx[t][k]] c_w[w_idx[o][k]]
 *
 * Conventions for every call:
 *   - The caller owns every buffer; the library never allocates or frees.
 *     "dev" pointers are device memory on the current HIP device; "host"
 *     pointers are ordinary host memory read before the call returns.
 *   - Arguments are validated before anything is launched.  Invalid
 *     arguments return OQ_EINVAL and touch nothing; a shape or bit width with
 *     no kernel returns OQ_EUNSUPPORTED; a HIP launch / device error returns
 *     OQ_EDEVICE.  oq_last_error() gives a message for the calling thread.
 *   - Device calls are asynchronous and stream-ordered: OQ_OK means enqueued
 *     on `stream` (0 = the null stream).  T = 0 is a valid no-op.
 *   - Index order: index 0 is the most negative centroid.  Packed indices are
 *     row-major, contiguous along d_in; index k of a row occupies bits
 *     [k b, (k+1) b) of the row read as a little-endian bit stream.  For
 *     b = 2, 4, 8 that is least-significant bits first within each byte (4, 2,
 *     1 per byte); 3- and 6-bit indices straddle byte boundaries.
 *   - The only global state is the thread-local error message.
 */
#ifndef OQ_H_
#define OQ_H_

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t oq_status;
enum {
  OQ_OK = 0,
  OQ_EINVAL = -1,        /* invalid argument; nothing done */
  OQ_EUNSUPPORTED = -2,  /* valid, but no kernel for this shape / width */
  OQ_ENOCONV = -3,       /* Lloyd-Max solve did not reach its tolerance */
  OQ_EDEVICE = -4        /* HIP runtime or launch error */
};

typedef enum { OQ_F32 = 0, OQ_BF16 = 1, OQ_F16 = 2 } oq_dtype;
enum { OQ_EPI_NONE = 0, OQ_EPI_GELU_ERF = 1, OQ_EPI_OUT_BF16 = 0x100 };

/* eps added to the activation norm (and to weight row norms) before the
 * division; the pages use an eps without giving its value. */
#define OQ_EPS 1e-12

/* Message for the calling thread's last non-OK return ("" if none). */
const char* oq_last_error(void);

/* Library version string. */
const char* oq_version(void);

/*
 * oq_build_rpbh -- the seeded RPBH rotation of the offline pseudo-code
 * (rcap.io summary, "Randomized Permuted Block-Hadamard" paragraph).
 *
 * R = B D P: (P x)_i = x[perm[i]] (a gather over all d coordinates),
 * D = diag(sign), B = blockdiag(H_h / sqrt(h)) with the Sylvester matrix
 * H[i][j] = (-1)^popcount(i & j).  Randomness: splitmix64 seeded with `seed`;
 * Fisher-Yates for i = d-1 .. 1 with j = floor(next() * (i+1) / 2^64); then
 * sign[i] = -1 if the top bit of next() is set, else +1, for i = 0 .. d-1.
 * Deterministic in (d, h, seed).
 *
 * d      : dimension, >= 2.
 * h      : block size, a power of two, 2 <= h, h divides d.
 * perm   : host [d] int32, written.
 * sign   : host [d] int8 (+1 / -1), written.
 * Errors : OQ_EINVAL on a bad shape or NULL pointer.
 */
oq_status oq_build_rpbh(int32_t d, int32_t h, uint64_t seed, int32_t* perm, int8_t* sign);

/*
 * oq_build_block_rht -- the rotation-ablation variant of the same page
 * (rcap.io summary, ablation paragraph: RPBH without its leading uniform
 * permutation, "Block-RHT"): perm[i] = i, and sign[i] = -1 if the top bit of
 * the (i+1)-th output of splitmix64(seed) is set, else +1 (the sign draws of
 * oq_build_rpbh without the shuffle draws before them).  The tables feed the
 * same kernels as RPBH tables (oq_quantize_weights, oq_rotate_quantize_act).
 *
 * Arguments and errors as oq_build_rpbh.
 */
oq_status oq_build_block_rht(int32_t d, int32_t h, uint64_t seed, int32_t* perm, int8_t* sign);

/*
 * oq_lloyd_max -- codebook[d, b] of the offline pseudo-code: the Lloyd-Max
 * quantizer (rcap.io summary, "core trick" paragraph) with L = 2^bits levels
 * for the exact marginal f_d(t) = C_d (1 - t^2)^((d-3)/2) on [-1, 1] of one
 * coordinate of a uniformly rotated unit vector in R^d.  Centroids are the
 * conditional means of their cells and thresholds the midpoints of adjacent
 * centroids; solved in fp64 (Lloyd steps, then Newton on the tridiagonal
 * Jacobian), with the symmetry c_j = -c_{L-1-j} enforced.
 *
 * d          : >= 3.
 * bits       : 1 .. 8.
 * centroids  : host [L] double, ascending, written.
 * thresholds : host [L-1] double, thresholds[j] = (c[j] + c[j+1]) / 2, written.
 * mse        : host double or NULL: E[(t - Q(t))^2] under f_d.
 * Errors     : OQ_EINVAL (bad d / bits / NULL); OQ_ENOCONV if the relative
 *              fixed-point residual stays above 1e-10 (outputs still written).
 */
oq_status oq_lloyd_max(int32_t d, int32_t bits, double* centroids, double* thresholds, double* mse);

/*
 * oq_quantize_weights -- the offline weight step of the pseudo-code:
 * W_rot = W R^T, n_o = ||W_rot[o]||, w_idx[o] = nearest centroid of
 * W_rot[o] / (n_o + OQ_EPS), i.e. #{j : thresholds[j] < u}.  Computed in fp64
 * on the device (offline, not on the hot path).
 *
 * W          : dev [d_out][d_in], fp32 or bf16 (w_dtype), row-major.
 * d_out      : >= 0 rows.   d_in: dimension, h | d_in, d_in * bits_w % 8 == 0.
 * h          : RPBH block size (power of two, 2 .. 256).
 * perm, sign : dev [d_in] int32 / int8 from oq_build_rpbh(d_in, h, seed).
 * thresholds : host [2^bits_w - 1] double, strictly increasing.
 * bits_w     : 2, 3, 4, 6 or 8.
 * w_idx      : dev [d_out][d_in * bits_w / 8] bytes, written.
 * w_norm     : dev [d_out] float, written (n_o rounded to fp32).
 * Errors     : OQ_EINVAL, OQ_EUNSUPPORTED (h > 256), OQ_EDEVICE.
 */
oq_status oq_quantize_weights(const void* W, oq_dtype w_dtype, int32_t d_out, int32_t d_in, int32_t h,
                              const int32_t* perm, const int8_t* sign,
                              const double* thresholds, int32_t bits_w,
                              uint8_t* w_idx, float* w_norm, hipStream_t stream);

/*
 * oq_rotate_quantize_act -- the online activation step of the pseudo-code,
 * per token: x_rot = R x (fast block Hadamard, O(d log h)), s = ||x_rot||,
 * x_idx = #{j : thresholds[j] < x_rot / (s + OQ_EPS)}.  Hot path.
 *
 * The rotation runs in fp32.  A coordinate whose fp32 value lies within a
 * certified rounding bound of a decision threshold is recomputed in fp64 and
 * compared with the fp64 threshold before its index is chosen, so every index
 * is the one exact arithmetic gives, up to fp64 rounding (coordinates within
 * ~1e-12 relative of a threshold).
 *
 * x          : dev [T][d], fp32 or bf16 (x_dtype), row-major.
 * T          : tokens, >= 0 (int64).   d: h | d, and d/16 either a multiple of 64
 *              up to 768 (d = 1024 .. 12288) or a power of two below 64 (d <= 512).
 * h          : RPBH block size (power of two, 2 .. 256).
 * perm, sign : dev [d] int32 / int8 from oq_build_rpbh(d, h, seed).
 * thresholds : host [2^bits_a - 1] double, strictly increasing; used as fp32.
 * bits_a     : 2, 3, 4, 6 or 8.
 * x_idx      : dev [T][d * bits_a / 8] bytes, written.
 * s          : dev [T] float, written (the norm, without eps).
 * x_rot      : dev [T][d] float or NULL: the fp32 rotated rows (checking only).
 * x, x_idx and x_rot must be 16-byte aligned (OQ_EINVAL otherwise).
 * Errors     : OQ_EINVAL, OQ_EUNSUPPORTED, OQ_EDEVICE.
 */
oq_status oq_rotate_quantize_act(const void* x, oq_dtype x_dtype, int64_t T, int32_t d, int32_t h,
                                 const int32_t* perm, const int8_t* sign,
                                 const double* thresholds, int32_t bits_a,
                                 uint8_t* x_idx, float* s, float* x_rot, hipStream_t stream);

/*
 * oq_qlinear -- the layer product in the rotated basis (the rotation cancels,
 * rcap.io summary, "rotation cancels" paragraph), as the fused codebook GEMM
 * the same page names as future work (caveats paragraph):
 *
 *   y[t][o] = s[t] * w_norm[o] * sum_k c_a[x_idx[t][k]] * c_w[w_idx[o][k]]
 *             (+ bias[o]) (then GELU(y) = y Phi(y) if epilogue == OQ_EPI_GELU_ERF)
 *
 * Indices are decoded through LDS tables of fp16(sqrt(d_in) * c) into fp16
 * MFMA operands with fp32 accumulation; the epilogue scales by
 * s * w_norm / d_in.  Hot path.
 *
 * The last, partial round of 256 x 256 output tiles (all tiles, when there
 * are fewer than the device's CUs) is split by K (stream-K) when it holds at
 * least 8 tiles and would leave more than a fifth of the CUs idle: the
 * workgroups of each XCD exchange fp32 partial tiles through a workspace that
 * the library owns, one per (device, stream): cus * 256 KB plus cus flags,
 * allocated on the first such launch on that stream and kept until the
 * process ends (at most 16 streams per device; past that, while the stream is
 * being captured into a graph and has no workspace yet, or on a device whose
 * workgroups are not dealt round-robin over 8 XCDs, the launch runs whole
 * tiles).  The first such launch on a device also runs a small probe kernel
 * of the XCD dispatch and synchronises its stream once.  The partial tiles
 * are added in a fixed order, so results are deterministic; launches that
 * share a stream are ordered by it.  A graph captured on a stream that
 * already has a workspace records that workspace: replay it only ordered
 * with the other launches that use it (on the capture stream, or after them);
 * two split launches that overlap on one workspace race, and the tiles whose
 * exchange fails come out as NaN.
 *
 * x_idx       : dev [T][d_in * bits_a / 8], from oq_rotate_quantize_act.
 * s           : dev [T] float.
 * T           : tokens >= 0.   d_out >= 0.   d_in: multiple of 128 (bits_a = 3
 *               or 4) or of 64 (bits_a = 6 or 8).
 * w_idx       : dev [d_out][d_in * bits_w / 8], from oq_quantize_weights.
 * w_norm      : dev [d_out] float.
 * centroids_a : host [2^bits_a] double, ascending.
 * centroids_w : host [2^bits_w] double, ascending.
 *               (bits_w, bits_a) with a kernel: W4A4, W2A4, W4A8, W2A8 and the
 *               other widths the pages name, W3A4, W2A3, W6A6.  3- and 6-bit
 *               indices are widened to 4 and 8 bits as they are staged.
 * bias        : dev [d_out] float or NULL.
 * epilogue    : OQ_EPI_NONE or OQ_EPI_GELU_ERF, optionally | OQ_EPI_OUT_BF16.
 * y           : dev [T][d_out], written: float, or bf16 (the fp32 result
 *               rounded to nearest even) with OQ_EPI_OUT_BF16.
 * x_idx, w_idx, w_norm, bias and y must be 16-byte aligned (OQ_EINVAL otherwise).
 * Errors      : OQ_EINVAL, OQ_EUNSUPPORTED, OQ_EDEVICE.
 */
oq_status oq_qlinear(const uint8_t* x_idx, const float* s, int64_t T,
                     const uint8_t* w_idx, const float* w_norm, int32_t d_out, int32_t d_in,
                     const double* centroids_a, int32_t bits_a,
                     const double* centroids_w, int32_t bits_w,
                     const float* bias, int32_t epilogue, void* y, hipStream_t stream);

/*
 * oq_quantize_weights_int4 -- INT4 round-to-nearest, weight only, for the
 * AdaLN modulation projections, which the method keeps out of the codebooks:
 * their timestep-dependent scale and shift cannot absorb the rotation
 * (rcap.io summary: deployment paragraph and AdaLN caveat; FLUX.2 Klein
 * OrbitQuant W4A8 model card, Components table).  The pages name only "INT4
 * weight round-to-nearest"; the scheme here is symmetric:
 *
 *   s[o][g] = fp32(max_{k in g} |W[o][k]| / 7)      (fp64 division)
 *   q[o][k] = clamp(rint(W[o][k] / s[o][g]), -8, 7)  (fp64, half to even;
 *                                                     q = 0 where s = 0)
 *
 * Offline, not on the hot path.
 *
 * W       : dev [d_out][d_in], fp32 or bf16 (w_dtype), row-major.
 * d_out   : >= 0.   d_in: > 0.
 * group   : input columns per scale: a multiple of 128 dividing d_in (d_in =
 *           one scale per output row).
 * q       : dev [d_out][d_in / 2] bytes, written: two's-complement nibbles,
 *           code k in bits [4k, 4k + 4) of the row (low nibble first).
 * scale   : dev [d_out][d_in / group] float, written.
 * Errors  : OQ_EINVAL, OQ_EDEVICE.
 */
oq_status oq_quantize_weights_int4(const void* W, oq_dtype w_dtype, int32_t d_out, int32_t d_in, int32_t group,
                                   uint8_t* q, float* scale, hipStream_t stream);

/*
 * oq_linear_w4a16 -- the AdaLN modulation projection with INT4 RTN weights
 * and 16-bit activations (same passages as oq_quantize_weights_int4):
 *
 *   y[t][o] = sum_g s[o][g] sum_{k in g} q[o][k] x[t][k]   (+ bias[o])
 *
 * Codes are decoded through an LDS table into exact bf16 / fp16 MFMA
 * operands; fp32 accumulation; each group's sum is scaled into an fp32
 * total.  Built for the modulation shape (T = images in the batch, a few
 * rows): it streams the packed weights once and is bound by HBM bandwidth.
 *
 * x       : dev [T][d_in], bf16 or fp16 (x_dtype), row-major.
 * T       : >= 0 rows, at most 65535 * 16.
 * q, scale: from oq_quantize_weights_int4 with the same d_out, d_in, group.
 * d_in    : multiple of 128.   group: multiple of 128 dividing d_in.
 * bias    : dev [d_out] float or NULL.
 * y       : dev [T][d_out] float, written.
 * x, q, scale, bias and y must be 16-byte aligned (OQ_EINVAL otherwise).
 * Errors  : OQ_EINVAL, OQ_EUNSUPPORTED, OQ_EDEVICE.
 */
oq_status oq_linear_w4a16(const void* x, oq_dtype x_dtype, int64_t T, const uint8_t* q, const float* scale,
                          int32_t d_out, int32_t d_in, int32_t group, const float* bias, float* y,
                          hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* OQ_H_ */
