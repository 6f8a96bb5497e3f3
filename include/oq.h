/*
 * oq.h -- C ABI of liboq, the OrbitQuant quantized linear layer on AMD
 * Instinct MI355X (gfx950).
 *
 * What the layer computes (method: "OrbitQuant: data-agnostic quantization
 * for image and video", rcap.io summary of the paper -- the mechanism
 * paragraphs and the offline / online pseudo-code; "OrbitQuant quantizes
 * FLUX.1 and Wan 2.1 with no calibration data", aiweekly.co -- one codebook
 * per input dimension).  For input dimension d let R = B D P be an orthogonal
 * d x d matrix (P a seeded uniform permutation, D a seeded diagonal of +-1,
 * B block-diagonal with h x h Walsh-Hadamard blocks scaled by 1/sqrt(h)), and
 * let c_0 < ... < c_{L-1} be the L = 2^b levels of the Lloyd-Max quantizer of
 * one coordinate of a uniformly random unit vector in R^d, with midpoints
 * theta_j = (c_j + c_{j+1}) / 2.  Writing q(v)_k = #{j : theta_j < v_k} for
 * the index vector of v:
 *
 *   weights, once:   n_o = |R w_o|,   iw_o = q(R w_o / (n_o + eps))
 *   each token x_t:  s_t = |R x_t|,   ia_t = q(R x_t / (s_t + eps))
 *   output:          y[t][o] = s_t n_o sum_k c^a_{ia_t,k} c^w_{iw_o,k}
 *
 * Since R is orthogonal (R^T R = I), y approximates W x: the product runs in
 * the rotated basis and the rotation is never undone.
 *
 * Conventions for every call:
 *   - The caller owns every buffer, workspaces included; the library never
 *     allocates or frees (oq_qlinear_splitk_noalloc uses a static device
 *     array instead of a workspace).  "dev" pointers are device memory on the current
 *     HIP device; "host" pointers are ordinary host memory read before the
 *     call returns.
 *   - Arguments are validated before anything is launched.  Invalid
 *     arguments return OQ_EINVAL and touch nothing; a shape or bit width with
 *     no kernel returns OQ_EUNSUPPORTED; a HIP launch / device error returns
 *     OQ_EDEVICE.  oq_last_error() gives a message for the calling thread.
 *   - Device calls are asynchronous and stream-ordered: OQ_OK means enqueued
 *     on `stream` (0 = the null stream).  T = 0 is a valid no-op.  No call
 *     synchronises, allocates or issues a memset, so device calls can be
 *     captured into HIP graphs.
 *   - Index order: index 0 is the most negative centroid.  Packed indices are
 *     row-major, contiguous along d_in; index k of a row occupies bits
 *     [k b, (k+1) b) of the row read as a little-endian bit stream.  For
 *     b = 2, 4, 8 that is least-significant bits first within each byte (4, 2,
 *     1 per byte); 3- and 6-bit indices straddle byte boundaries.
 *   - The only global state is the thread-local error message, and the
 *     device scratch of oq_qlinear_splitk_noalloc with its address per device.
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
 * The solve takes at most 300 Newton steps; the environment variable
 * OQ_LLOYD_MAX_NEWTON_STEPS = n (0 <= n < 300) lowers that cap, which lets
 * the OQ_ENOCONV path be exercised.
 */
oq_status oq_lloyd_max(int32_t d, int32_t bits, double* centroids, double* thresholds, double* mse);

/*
 * oq_quantize_weights -- the offline weight step (rcap.io summary, offline
 * part of the pseudo-code): for each weight row w_o, n_o = |R w_o| and
 * w_idx[o] = q(R w_o / (n_o + OQ_EPS)), q(v)_k = #{j : thresholds[j] < v_k}
 * (the index of the nearest centroid).  Computed in fp64 on the device
 * (offline, not on the hot path).
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
 * oq_fold_permutation -- moves the next layer's input permutation into this
 * layer's output channels (offline).  The RPBH rotation of a layer's input
 * starts with a uniform random permutation (rcap.io summary, RPBH paragraph;
 * online pseudo-code).  When the next layer's input is an elementwise
 * function of this layer's output -- GELU of an MLP's up projection -- the
 * permutation commutes with that function: with the rows of this layer's
 * quantized weights, norms and bias reordered as
 *
 *   w_idx_out[i] = w_idx[perm_next[i]], w_norm_out[i] = w_norm[perm_next[i]],
 *   bias_out[i] = bias[perm_next[i]]   (i = 0 .. d_out - 1),
 *
 * the layer writes y'[t][i] = y[t][perm_next[i]] bit for bit, and the next
 * oq_rotate_quantize_act on GELU(y') with perm = identity (perm[i] = i) and
 * the next layer's own sign table gives the same rotation, indices and norm
 * as on GELU(y) with (perm_next, sign): its gather reads the staged row in
 * order.  Nothing is re-quantized.
 *
 * w_idx, w_norm : dev, this layer's oq_quantize_weights output ([d_out][d_in *
 *                 bits_w / 8] bytes, [d_out] float).
 * bias          : dev [d_out] float or NULL (then bias_out is not written).
 * d_out         : this layer's output width = the next layer's d_in.
 * d_in, bits_w  : this layer's; d_in * bits_w / 8 a multiple of 16.
 * perm_next     : dev [d_out] int32, the next layer's RPBH permutation (from
 *                 oq_build_rpbh(d_out, h, seed)); entries outside [0, d_out)
 *                 are clamped, so the copy stays in bounds.
 * w_idx_out, w_norm_out, bias_out : dev, same shapes, written; they must not
 *                 overlap the inputs; w_idx and w_idx_out 16-byte aligned.
 * Errors        : OQ_EINVAL, OQ_EDEVICE.
 */
oq_status oq_fold_permutation(const uint8_t* w_idx, const float* w_norm, const float* bias, int32_t d_out,
                              int32_t d_in, int32_t bits_w, const int32_t* perm_next, uint8_t* w_idx_out,
                              float* w_norm_out, float* bias_out, hipStream_t stream);

/*
 * oq_rotate_quantize_act -- the online activation step (rcap.io summary,
 * online part of the pseudo-code), per token x: v = R x (fast block Hadamard,
 * O(d log h)), s = |v|, x_idx = q(v / (s + OQ_EPS)).  Hot path.
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
 * s * w_norm / d_in.  Hot path.  Persistent workgroups (one per compute unit)
 * compute whole 256 x 256 output tiles; no workspace.
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
 * oq_qlinear_workspace_size -- bytes of workspace oq_qlinear_splitk needs for
 * this shape on the current device: 0 if the shape takes no split, else
 * 256 + 4 cus (rounded up to 256) + cus * 256 KB for a device with cus
 * compute units (64 MB + 1280 bytes on a 256-CU MI355X).  The same passages
 * as oq_qlinear.
 *
 * T, d_out, d_in, bits_a, bits_w : as for oq_qlinear.
 * bytes   : host size_t, written.
 * Errors  : OQ_EINVAL, OQ_EUNSUPPORTED, OQ_EDEVICE (no device to query).
 */
oq_status oq_qlinear_workspace_size(int64_t T, int32_t d_out, int32_t d_in, int32_t bits_a, int32_t bits_w,
                                    size_t* bytes);

/*
 * oq_qlinear_splitk -- oq_qlinear (same passages, same result up to fp32
 * summation order, deterministic) with the last, partial round of output
 * tiles split along K: when a launch has a partial last round (or fewer
 * tiles than compute units) and splitting it is expected to be faster, the
 * workgroups cut that round's K stages (of 128, or 64 for 6- and 8-bit
 * activations) into equal runs, and the workgroup that holds a tile's last
 * stage adds the fp32 partial tiles the others left in the workspace, in a
 * fixed order, before the epilogue (stream-K).  "Expected faster" is a cost
 * model fitted to measurements: with nst stages per tile, rem tiles in the
 * last round and cus compute units, split iff nst * w * (1 - rem / cus) > 15,
 * w = 1 for activations of at most 4 bits, 0.7 for 8-bit, 1.05 for 6-bit.
 * Other shapes run as oq_qlinear and ignore the workspace.
 *
 * workspace       : dev, 256-byte aligned, at least the bytes that
 *                   oq_qlinear_workspace_size gives for this shape (NULL / 0
 *                   is fine when it gives 0).  Caller-owned.  It must be
 *                   zero-filled once before its first use; every launch
 *                   leaves its control words ready for the next one (a launch
 *                   generation that each launch advances, and per-workgroup
 *                   flags tagged with it), so later launches need no clearing.
 *                   Launches that share a workspace must be ordered (one
 *                   stream, or events): two launches running at once on one
 *                   workspace race, and their tiles can come out wrong.  A
 *                   graph that captures a launch records the workspace.
 * workspace_bytes : its size.
 * Other arguments : as oq_qlinear.
 * A finishing workgroup waits for its contributors with a bounded spin;
 * contributors never wait and are dispatched before it, so the bound is
 * reached only if the device stops dispatching them (then that tile is
 * written as NaN; the status, returned at enqueue time, cannot show it).
 * Errors          : OQ_EINVAL (also: workspace missing, too small or
 *                   misaligned), OQ_EUNSUPPORTED, OQ_EDEVICE.
 */
oq_status oq_qlinear_splitk(const uint8_t* x_idx, const float* s, int64_t T,
                            const uint8_t* w_idx, const float* w_norm, int32_t d_out, int32_t d_in,
                            const double* centroids_a, int32_t bits_a,
                            const double* centroids_w, int32_t bits_w,
                            const float* bias, int32_t epilogue, void* y,
                            void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * oq_qlinear_splitk_noalloc -- oq_qlinear_splitk without a workspace
 * argument, for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc).  The
 * split's workspace is the library's own fixed device scratch: 64 MB + 1280
 * bytes (256 partial-tile slots), a static device array that every device
 * the library runs on holds from the moment the library's code is loaded
 * until the process ends; this call allocates nothing and calls no
 * allocating routine.  Results are bit-identical to oq_qlinear_splitk with a
 * workspace of its own.
 *
 * Every call on one device shares that device's scratch, which keeps the
 * last call's contents (its launch generation advances each call, so nothing
 * needs clearing): calls that can run at the same time on one device (other
 * streams, graphs) race, and their tiles can come out wrong; order them.
 * Arguments and result as oq_qlinear.
 * Errors : as oq_qlinear; OQ_EUNSUPPORTED if the split would need more than
 *          the scratch's 256 slots (a device with more than 256 compute units).
 */
oq_status oq_qlinear_splitk_noalloc(const uint8_t* x_idx, const float* s, int64_t T,
                                    const uint8_t* w_idx, const float* w_norm, int32_t d_out, int32_t d_in,
                                    const double* centroids_a, int32_t bits_a,
                                    const double* centroids_w, int32_t bits_w,
                                    const float* bias, int32_t epilogue, void* y, hipStream_t stream);

/*
 * oq_quantize_weights_int4 -- INT4 round-to-nearest, weight only, for the
 * AdaLN modulation projections, which the method keeps out of the codebooks:
 * their timestep-dependent scale and shift cannot absorb the rotation
 * (rcap.io summary: deployment paragraph and AdaLN caveat; "FLUX.3 Image
 * Klein OrbitQuant W4A8" model card, Components table).  The pages name only "INT4
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
