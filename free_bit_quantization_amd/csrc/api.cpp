// C ABI of liboq: argument validation, launch planning, error reporting.
// Every entry point validates all arguments before launching anything; an
// invalid argument returns OQ_EINVAL with no side effect.
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "oq_internal.h"

namespace {

thread_local char g_err[512] = "";

oq_status fail(oq_status code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

oq_status ok() {
  g_err[0] = 0;
  return OQ_OK;
}

oq_status device_error(hipError_t e, const char* what) {
  return fail(OQ_EDEVICE, "%s: %s", what, hipGetErrorString(e));
}

int log2_exact(int32_t h) {
  if (h < 2 || (h & (h - 1)) != 0) return -1;
  int m = 0;
  while ((1 << m) < h) ++m;
  return m;
}

bool bits_ok(int32_t b) { return b == 2 || b == 3 || b == 4 || b == 6 || b == 8; }

// Thresholds must be finite and strictly increasing, also after rounding to fp32.
oq_status check_thresholds(const double* th, int n, bool need_f32) {
  if (!th) return fail(OQ_EINVAL, "thresholds is NULL");
  for (int i = 0; i < n; ++i) {
    if (!std::isfinite(th[i])) return fail(OQ_EINVAL, "threshold %d is not finite", i);
    if (i > 0 && !(th[i] > th[i - 1])) return fail(OQ_EINVAL, "thresholds not strictly increasing at %d", i);
    if (need_f32 && i > 0 && !((float)th[i] > (float)th[i - 1]))
      return fail(OQ_EINVAL, "thresholds %d and %d coincide in fp32", i - 1, i);
  }
  return OQ_OK;
}

// (bits_w, bits_a) pairs with a GEMM kernel: W4A4, W2A4, W4A8, W2A8 and the
// other widths the pages name, W3A4, W2A3, W6A6
bool gemm_widths_ok(int bits_a, int bits_w) {
  return (bits_a == 4 && (bits_w == 2 || bits_w == 3 || bits_w == 4)) || (bits_a == 8 && (bits_w == 2 || bits_w == 4)) ||
         (bits_a == 3 && bits_w == 2) || (bits_a == 6 && bits_w == 6);
}

uint16_t to_f16_bits(double v) {
  const _Float16 h = (_Float16)v;
  uint16_t b;
  std::memcpy(&b, &h, 2);
  return b;
}

}  // namespace

extern "C" {

const char* oq_last_error(void) { return g_err; }

const char* oq_version(void) { return "liboq 0.1 (gfx950)"; }

oq_status oq_build_rpbh(int32_t d, int32_t h, uint64_t seed, int32_t* perm, int8_t* sign) {
  if (d < 2) return fail(OQ_EINVAL, "d must be >= 2 (got %d)", d);
  if (log2_exact(h) < 0) return fail(OQ_EINVAL, "h must be a power of two >= 2 (got %d)", h);
  if (d % h != 0) return fail(OQ_EINVAL, "h (%d) must divide d (%d)", h, d);
  if (!perm || !sign) return fail(OQ_EINVAL, "perm / sign is NULL");
  oq::build_rpbh_tables(d, seed, perm, sign);
  return ok();
}

oq_status oq_build_block_rht(int32_t d, int32_t h, uint64_t seed, int32_t* perm, int8_t* sign) {
  if (d < 2) return fail(OQ_EINVAL, "d must be >= 2 (got %d)", d);
  if (log2_exact(h) < 0) return fail(OQ_EINVAL, "h must be a power of two >= 2 (got %d)", h);
  if (d % h != 0) return fail(OQ_EINVAL, "h (%d) must divide d (%d)", h, d);
  if (!perm || !sign) return fail(OQ_EINVAL, "perm / sign is NULL");
  oq::build_block_rht_tables(d, seed, perm, sign);
  return ok();
}

oq_status oq_lloyd_max(int32_t d, int32_t bits, double* centroids, double* thresholds, double* mse) {
  if (d < 3) return fail(OQ_EINVAL, "d must be >= 3 (got %d)", d);
  if (bits < 1 || bits > 8) return fail(OQ_EINVAL, "bits must be in 1..8 (got %d)", bits);
  if (!centroids || !thresholds) return fail(OQ_EINVAL, "centroids / thresholds is NULL");
  // The Newton step cap can be lowered through the environment, so that the
  // non-convergence path can be exercised (OQ_LLOYD_MAX_NEWTON_STEPS = n >= 0).
  int max_newton = oq::kLloydMaxNewton;
  if (const char* env = std::getenv("OQ_LLOYD_MAX_NEWTON_STEPS")) {
    char* end = nullptr;
    const long v = std::strtol(env, &end, 10);
    if (end != env && *end == 0 && v >= 0 && v < max_newton) max_newton = (int)v;
  }
  double resid = 0.0;
  if (oq::lloyd_max_fd(d, bits, max_newton, centroids, thresholds, mse, &resid) != 0)
    return fail(OQ_ENOCONV, "Lloyd-Max residual %.3g above 1e-10 (d=%d, bits=%d)", resid, d, bits);
  return ok();
}

oq_status oq_quantize_weights(const void* W, oq_dtype w_dtype, int32_t d_out, int32_t d_in, int32_t h,
                              const int32_t* perm, const int8_t* sign, const double* thresholds, int32_t bits_w,
                              uint8_t* w_idx, float* w_norm, hipStream_t stream) {
  const int m = log2_exact(h);
  if (w_dtype != OQ_F32 && w_dtype != OQ_BF16) return fail(OQ_EINVAL, "w_dtype must be OQ_F32 or OQ_BF16");
  if (d_out < 0) return fail(OQ_EINVAL, "d_out must be >= 0");
  if (d_in < 2 || m < 0 || d_in % h != 0) return fail(OQ_EINVAL, "need h a power of two >= 2 dividing d_in");
  if (!bits_ok(bits_w)) return fail(OQ_EINVAL, "bits_w must be 2, 3, 4, 6 or 8 (got %d)", bits_w);
  if ((d_in * bits_w) % 8 != 0) return fail(OQ_EINVAL, "d_in * bits_w must fill whole bytes");
  const int nthr = (1 << bits_w) - 1;
  oq_status st = check_thresholds(thresholds, nthr, false);
  if (st != OQ_OK) return st;
  if (d_out > 0 && (!W || !perm || !sign || !w_idx || !w_norm)) return fail(OQ_EINVAL, "NULL device pointer");
  if (h > 256) return fail(OQ_EUNSUPPORTED, "h > 256 has no kernel");
  if ((size_t)d_in * 8 + 256 * 8 + 64 > 160 * 1024) return fail(OQ_EUNSUPPORTED, "d_in %d too large for the LDS row", d_in);
  if (d_out == 0) return ok();
  oq::WqArgs a{};
  a.W = W; a.d_out = d_out; a.d = d_in; a.h = h; a.perm = perm; a.sign = sign;
  a.w_idx = w_idx; a.w_norm = w_norm; a.nthr = nthr;
  for (int i = 0; i < nthr; ++i) a.thr[i] = thresholds[i];
  hipError_t e = oq::wq_launch(a, w_dtype == OQ_BF16, bits_w, stream);
  if (e != hipSuccess) return device_error(e, "oq_quantize_weights launch");
  return ok();
}

oq_status oq_rotate_quantize_act(const void* x, oq_dtype x_dtype, int64_t T, int32_t d, int32_t h,
                                 const int32_t* perm, const int8_t* sign, const double* thresholds, int32_t bits_a,
                                 uint8_t* x_idx, float* s, float* x_rot, hipStream_t stream) {
  const int m = log2_exact(h);
  if (x_dtype != OQ_F32 && x_dtype != OQ_BF16) return fail(OQ_EINVAL, "x_dtype must be OQ_F32 or OQ_BF16");
  if (T < 0) return fail(OQ_EINVAL, "T must be >= 0");
  if (d < 16 || d % 16 != 0) return fail(OQ_EINVAL, "d must be a positive multiple of 16 (got %d)", d);
  if (m < 0 || d % h != 0) return fail(OQ_EINVAL, "need h a power of two >= 2 dividing d");
  if (!bits_ok(bits_a)) return fail(OQ_EINVAL, "bits_a must be 2, 3, 4, 6 or 8 (got %d)", bits_a);
  const int nthr = (1 << bits_a) - 1;
  oq_status st = check_thresholds(thresholds, nthr, true);
  if (st != OQ_OK) return st;
  if (T > 0 && (!x || !perm || !sign || !x_idx || !s)) return fail(OQ_EINVAL, "NULL device pointer");
  if (((reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(x_idx) | reinterpret_cast<uintptr_t>(x_rot)) & 15) != 0)
    return fail(OQ_EINVAL, "x, x_idx and x_rot must be 16-byte aligned");
  if (m > 8) return fail(OQ_EUNSUPPORTED, "h > 256 has no kernel");

  // Threshold-search grid: cells of width w over [theta_0, theta_{L-2}], each
  // widened by 0.02 w (rounding of the cell index) and by the largest guard
  // radius, must hold at most one threshold.  The radius is at most
  // (m + 1) u L1 c + k u max|theta| with L1 c <= 1 (Cauchy-Schwarz over a
  // block), max|theta| < 1 and k = 6 (workgroup kernel) or 4 J + 5 <= 25
  // (wavefront kernel, m >= 6): below (2 m + 24) u, u = 2^-24.
  float th32[oq::kMaxThr];
  for (int i = 0; i < nthr; ++i) th32[i] = (float)thresholds[i];
  const double lo = th32[0], hi = th32[nthr - 1];
  double min_gap = INFINITY;
  for (int i = 1; i < nthr; ++i) min_gap = std::fmin(min_gap, (double)th32[i] - (double)th32[i - 1]);
  const double rmax = (2.0 * m + 24.0) * std::ldexp(1.0, -24);
  int G = 0;
  if (hi > lo) {
    const double wmax = (min_gap - 2.2 * rmax) / 1.1;
    if (wmax > 0) {
      const double need = (hi - lo) / wmax;
      int g = 1;
      while (g < need && g <= oq::kMaxGrid) g <<= 1;
      if (g <= oq::kMaxGrid) G = g;
    }
  }
  oq::RqPlan plan;
  if (!oq::rq_plan(d, m, x_dtype == OQ_BF16, bits_a, T, G, &plan))
    return fail(OQ_EUNSUPPORTED, "no rotate-quantize kernel for d=%d h=%d (d/16 must be a multiple of 64 up to 768, or a power of two below 64)", d, h);
  if (T == 0) return ok();

  oq::RqArgs a{};
  a.x = x; a.T = T; a.d = d; a.log2h = m; a.perm = perm; a.sign = sign;
  a.x_idx = x_idx; a.s = s; a.x_rot = x_rot; a.nthr = nthr; a.G = G;
  a.g_lo = lo;
  a.g_invw = G > 0 ? G / (hi - lo) : 0.0;
  a.g_rmax = rmax;
  a.thr_absmax = 0.f;
  for (int i = 0; i < nthr; ++i) {
    a.thr_absmax = std::fmax(a.thr_absmax, std::fabs(th32[i]));
    a.thr[i] = th32[i];
    a.thr_lo[i] = (float)(thresholds[i] - (double)th32[i]);   // the difference is exact in fp64
  }
  if (G > 0 && G <= oq::kHostGrid) {
    // cell c covers u in [lo + (c - 0.02) w - rmax, lo + (c + 1.02) w + rmax]: the
    // number of thresholds below it and the one threshold inside it (or +inf)
    const double w = 1.0 / a.g_invw;
    for (int c = 0; c < G; ++c) {
      const double ulo = c == 0 ? -INFINITY : lo + (c - 0.02) * w - rmax;
      const double uhi = c == G - 1 ? INFINITY : lo + (c + 1.02) * w + rmax;
      int base = 0;
      while (base < nthr && (double)th32[base] < ulo) ++base;
      const float th = (base < nthr && (double)th32[base] <= uhi) ? th32[base] : INFINITY;
      std::memcpy(&a.glut[c][0], &th, 4);
      a.glut[c][1] = base;
    }
  }
  hipError_t e = oq::rq_launch(a, x_dtype == OQ_BF16, bits_a, plan, stream);
  if (e != hipSuccess) return device_error(e, "oq_rotate_quantize_act launch");
  return ok();
}

}  // extern "C"

namespace {

// Validation shared by the GEMM entry points; fills everything of a but the
// work split.  Returns OQ_OK with *nothing = true for an empty product.
oq_status qlinear_args(const uint8_t* x_idx, const float* s, int64_t T, const uint8_t* w_idx, const float* w_norm,
                       int32_t d_out, int32_t d_in, const double* centroids_a, int32_t bits_a,
                       const double* centroids_w, int32_t bits_w, const float* bias, int32_t epilogue, void* y,
                       oq::QlArgs* a, bool* nothing) {
  if (T < 0 || d_out < 0) return fail(OQ_EINVAL, "T and d_out must be >= 0");
  if (d_in <= 0) return fail(OQ_EINVAL, "d_in must be > 0");
  if (!bits_ok(bits_a) || !bits_ok(bits_w)) return fail(OQ_EINVAL, "bits must be 2, 3, 4, 6 or 8");
  if ((epilogue & ~(0xFF | OQ_EPI_OUT_BF16)) != 0 ||
      ((epilogue & 0xFF) != OQ_EPI_NONE && (epilogue & 0xFF) != OQ_EPI_GELU_ERF))
    return fail(OQ_EINVAL, "unknown epilogue %d", epilogue);
  if (!centroids_a || !centroids_w) return fail(OQ_EINVAL, "centroids is NULL");
  const int La = 1 << bits_a, Lw = 1 << bits_w;
  for (int i = 0; i < La; ++i)
    if (!std::isfinite(centroids_a[i])) return fail(OQ_EINVAL, "centroids_a[%d] not finite", i);
  for (int i = 0; i < Lw; ++i)
    if (!std::isfinite(centroids_w[i])) return fail(OQ_EINVAL, "centroids_w[%d] not finite", i);
  if (T > 0 && d_out > 0 && (!x_idx || !s || !w_idx || !w_norm || !y)) return fail(OQ_EINVAL, "NULL device pointer");
  auto misaligned = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) != 0; };
  if (misaligned(x_idx) || misaligned(w_idx) || misaligned(w_norm) || misaligned(y) || misaligned(bias))
    return fail(OQ_EINVAL, "x_idx, w_idx, w_norm, bias and y must be 16-byte aligned");
  if (!gemm_widths_ok(bits_a, bits_w)) return fail(OQ_EUNSUPPORTED, "no GEMM kernel for W%dA%d", bits_w, bits_a);
  const int kstage = oq::ql_stage_k(bits_a);
  if (d_in % kstage != 0) return fail(OQ_EUNSUPPORTED, "d_in must be a multiple of %d for A%d (got %d)", kstage, bits_a, d_in);
  const double sk = std::sqrt((double)d_in);
  for (int i = 0; i < La; ++i)
    if (std::fabs(sk * centroids_a[i]) > 60000.0) return fail(OQ_EINVAL, "sqrt(d_in)*centroids_a exceeds fp16");
  for (int i = 0; i < Lw; ++i)
    if (std::fabs(sk * centroids_w[i]) > 60000.0) return fail(OQ_EINVAL, "sqrt(d_in)*centroids_w exceeds fp16");
  *nothing = T == 0 || d_out == 0;
  *a = oq::QlArgs{};
  a->x_idx = x_idx; a->s = s; a->T = T; a->w_idx = w_idx; a->w_norm = w_norm;
  a->N = d_out; a->K = d_in; a->bias = bias; a->y = y; a->epilogue = epilogue;
  a->scale = (float)(1.0 / d_in);
  for (int i = 0; i < 256; ++i) a->tab_a[i] = i < La ? to_f16_bits(sk * centroids_a[i]) : 0;
  for (int i = 0; i < 256; ++i) a->tab_w[i] = i < Lw ? to_f16_bits(sk * centroids_w[i]) : 0;
  return OQ_OK;
}

// Compute units of the current device.
oq_status device_cus(int* cus) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return device_error(e, "hipGetDevice");
  e = hipDeviceGetAttribute(cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return device_error(e, "hipDeviceGetAttribute");
  if (*cus <= 0) return fail(OQ_EDEVICE, "device reports %d compute units", *cus);
  return OQ_OK;
}

oq::QlSplit qlinear_plan(int64_t T, int32_t d_out, int32_t d_in, int32_t bits_a, int cus, int64_t slots) {
  const int64_t ntiles = ((T + 255) / 256) * (((int64_t)d_out + 255) / 256);
  return oq::ql_split_plan(ntiles, d_in / oq::ql_stage_k(bits_a), cus, slots, oq::ql_stage_weight(bits_a));
}

// Launch with a workspace of `slots` partial-tile slots laid out at ws (ws may
// be NULL with slots = 0: whole tiles only).
oq_status qlinear_launch(oq::QlArgs& a, int32_t bits_a, int32_t bits_w, int cus, unsigned char* ws, int64_t slots,
                         hipStream_t stream) {
  a.sp = qlinear_plan(a.T, a.N, a.K, bits_a, cus, slots);
  if (a.sp.sk_tiles > 0) {
    a.hdr = reinterpret_cast<uint64_t*>(ws);
    a.flags = reinterpret_cast<uint32_t*>(ws + oq::ql_ws_flags_offset());
    a.slots = reinterpret_cast<float*>(ws + oq::ql_ws_slots_offset(slots));
  }
  hipError_t e = oq::ql_launch(a, bits_a, bits_w, stream);
  if (e != hipSuccess) return device_error(e, "oq_qlinear launch");
  return ok();
}

}  // namespace

extern "C" {

oq_status oq_qlinear(const uint8_t* x_idx, const float* s, int64_t T, const uint8_t* w_idx, const float* w_norm,
                     int32_t d_out, int32_t d_in, const double* centroids_a, int32_t bits_a,
                     const double* centroids_w, int32_t bits_w, const float* bias, int32_t epilogue, void* y,
                     hipStream_t stream) {
  oq::QlArgs a;
  bool nothing = false;
  oq_status st = qlinear_args(x_idx, s, T, w_idx, w_norm, d_out, d_in, centroids_a, bits_a, centroids_w, bits_w,
                              bias, epilogue, y, &a, &nothing);
  if (st != OQ_OK) return st;
  if (nothing) return ok();
  int cus = 0;
  if ((st = device_cus(&cus)) != OQ_OK) return st;
  return qlinear_launch(a, bits_a, bits_w, cus, nullptr, 0, stream);
}

oq_status oq_qlinear_workspace_size(int64_t T, int32_t d_out, int32_t d_in, int32_t bits_a, int32_t bits_w,
                                    size_t* bytes) {
  if (!bytes) return fail(OQ_EINVAL, "bytes is NULL");
  if (T < 0 || d_out < 0 || d_in <= 0) return fail(OQ_EINVAL, "need T >= 0, d_out >= 0, d_in > 0");
  if (!bits_ok(bits_a) || !bits_ok(bits_w)) return fail(OQ_EINVAL, "bits must be 2, 3, 4, 6 or 8");
  if (!gemm_widths_ok(bits_a, bits_w)) return fail(OQ_EUNSUPPORTED, "no GEMM kernel for W%dA%d", bits_w, bits_a);
  if (d_in % oq::ql_stage_k(bits_a) != 0)
    return fail(OQ_EUNSUPPORTED, "d_in must be a multiple of %d for A%d", oq::ql_stage_k(bits_a), bits_a);
  *bytes = 0;
  if (T == 0 || d_out == 0) return ok();
  int cus = 0;
  oq_status st = device_cus(&cus);
  if (st != OQ_OK) return st;
  if (qlinear_plan(T, d_out, d_in, bits_a, cus, cus).sk_tiles > 0) *bytes = (size_t)oq::ql_ws_bytes(cus);
  return ok();
}

oq_status oq_qlinear_splitk(const uint8_t* x_idx, const float* s, int64_t T, const uint8_t* w_idx,
                            const float* w_norm, int32_t d_out, int32_t d_in, const double* centroids_a,
                            int32_t bits_a, const double* centroids_w, int32_t bits_w, const float* bias,
                            int32_t epilogue, void* y, void* workspace, size_t workspace_bytes,
                            hipStream_t stream) {
  oq::QlArgs a;
  bool nothing = false;
  oq_status st = qlinear_args(x_idx, s, T, w_idx, w_norm, d_out, d_in, centroids_a, bits_a, centroids_w, bits_w,
                              bias, epilogue, y, &a, &nothing);
  if (st != OQ_OK) return st;
  if ((reinterpret_cast<uintptr_t>(workspace) & 255) != 0) return fail(OQ_EINVAL, "workspace must be 256-byte aligned");
  if (nothing) return ok();
  int cus = 0;
  if ((st = device_cus(&cus)) != OQ_OK) return st;
  const bool split = qlinear_plan(T, d_out, d_in, bits_a, cus, cus).sk_tiles > 0;
  if (split) {
    const size_t need = (size_t)oq::ql_ws_bytes(cus);
    if (!workspace || workspace_bytes < need)
      return fail(OQ_EINVAL, "workspace of %zu bytes needed (got %zu)", need, workspace ? workspace_bytes : (size_t)0);
  }
  return qlinear_launch(a, bits_a, bits_w, cus, static_cast<unsigned char*>(workspace), split ? cus : 0, stream);
}

oq_status oq_qlinear_splitk_noalloc(const uint8_t* x_idx, const float* s, int64_t T, const uint8_t* w_idx,
                                    const float* w_norm, int32_t d_out, int32_t d_in, const double* centroids_a,
                                    int32_t bits_a, const double* centroids_w, int32_t bits_w, const float* bias,
                                    int32_t epilogue, void* y, hipStream_t stream) {
  static_assert(oq::kScratchBytes == oq::ql_ws_bytes(oq::kScratchSlots), "scratch layout");
  oq::QlArgs a;
  bool nothing = false;
  oq_status st = qlinear_args(x_idx, s, T, w_idx, w_norm, d_out, d_in, centroids_a, bits_a, centroids_w, bits_w,
                              bias, epilogue, y, &a, &nothing);
  if (st != OQ_OK) return st;
  if (nothing) return ok();
  int cus = 0;
  if ((st = device_cus(&cus)) != OQ_OK) return st;
  const bool split = qlinear_plan(T, d_out, d_in, bits_a, cus, cus).sk_tiles > 0;
  if (!split) return qlinear_launch(a, bits_a, bits_w, cus, nullptr, 0, stream);
  if (cus > oq::kScratchSlots)
    return fail(OQ_EUNSUPPORTED, "the split needs %d partial-tile slots; the library scratch holds %d", cus,
                oq::kScratchSlots);
  void* ws = nullptr;
  hipError_t e = oq::ql_scratch(&ws);
  if (e != hipSuccess) return device_error(e, "library scratch address");
  return qlinear_launch(a, bits_a, bits_w, cus, static_cast<unsigned char*>(ws), oq::kScratchSlots, stream);
}

oq_status oq_fold_permutation(const uint8_t* w_idx, const float* w_norm, const float* bias, int32_t d_out,
                              int32_t d_in, int32_t bits_w, const int32_t* perm_next, uint8_t* w_idx_out,
                              float* w_norm_out, float* bias_out, hipStream_t stream) {
  if (d_out < 0 || d_in <= 0) return fail(OQ_EINVAL, "need d_out >= 0 and d_in > 0");
  if (!bits_ok(bits_w)) return fail(OQ_EINVAL, "bits_w must be 2, 3, 4, 6 or 8 (got %d)", bits_w);
  const int64_t row_bytes = (int64_t)d_in * bits_w / 8;
  if (((int64_t)d_in * bits_w) % 128 != 0) return fail(OQ_EINVAL, "d_in * bits_w / 8 must be a multiple of 16");
  if (d_out == 0) return ok();
  if (!w_idx || !w_norm || !perm_next || !w_idx_out || !w_norm_out || (bias && !bias_out))
    return fail(OQ_EINVAL, "NULL device pointer");
  auto misaligned = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) != 0; };
  if (misaligned(w_idx) || misaligned(w_idx_out)) return fail(OQ_EINVAL, "w_idx and w_idx_out must be 16-byte aligned");
  auto overlap = [](const void* a, const void* b, int64_t n) {
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + (uintptr_t)n && y < x + (uintptr_t)n;
  };
  if (overlap(w_idx, w_idx_out, (int64_t)d_out * row_bytes) || overlap(w_norm, w_norm_out, 4 * (int64_t)d_out) ||
      (bias && overlap(bias, bias_out, 4 * (int64_t)d_out)))
    return fail(OQ_EINVAL, "outputs must not overlap the inputs");
  oq::FoldArgs a{w_idx, w_norm, bias, perm_next, d_out, row_bytes, w_idx_out, w_norm_out, bias_out};
  hipError_t e = oq::fold_launch(a, stream);
  if (e != hipSuccess) return device_error(e, "oq_fold_permutation launch");
  return ok();
}

oq_status oq_quantize_weights_int4(const void* W, oq_dtype w_dtype, int32_t d_out, int32_t d_in, int32_t group,
                                   uint8_t* q, float* scale, hipStream_t stream) {
  if (w_dtype != OQ_F32 && w_dtype != OQ_BF16) return fail(OQ_EINVAL, "w_dtype must be OQ_F32 or OQ_BF16");
  if (d_out < 0 || d_in <= 0) return fail(OQ_EINVAL, "need d_out >= 0 and d_in > 0");
  if (group <= 0 || group % 128 != 0 || d_in % group != 0)
    return fail(OQ_EINVAL, "group must be a positive multiple of 128 dividing d_in (got %d, d_in %d)", group, d_in);
  if (d_out > 0 && (!W || !q || !scale)) return fail(OQ_EINVAL, "NULL device pointer");
  if (d_out == 0) return ok();
  oq::RtnArgs a{W, d_out, d_in, group, q, scale};
  hipError_t e = oq::rtn_launch(a, w_dtype == OQ_BF16, stream);
  if (e != hipSuccess) return device_error(e, "oq_quantize_weights_int4 launch");
  return ok();
}

oq_status oq_linear_w4a16(const void* x, oq_dtype x_dtype, int64_t T, const uint8_t* q, const float* scale,
                          int32_t d_out, int32_t d_in, int32_t group, const float* bias, float* y,
                          hipStream_t stream) {
  if (x_dtype != OQ_BF16 && x_dtype != OQ_F16) return fail(OQ_EINVAL, "x_dtype must be OQ_BF16 or OQ_F16");
  if (T < 0 || d_out < 0 || d_in <= 0) return fail(OQ_EINVAL, "need T >= 0, d_out >= 0, d_in > 0");
  if (d_in % 128 != 0) return fail(OQ_EINVAL, "d_in must be a multiple of 128 (got %d)", d_in);
  if (group <= 0 || group % 128 != 0 || d_in % group != 0)
    return fail(OQ_EINVAL, "group must be a positive multiple of 128 dividing d_in (got %d, d_in %d)", group, d_in);
  if (T > 0 && d_out > 0 && (!x || !q || !scale || !y)) return fail(OQ_EINVAL, "NULL device pointer");
  auto misaligned = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) != 0; };
  if (misaligned(x) || misaligned(q)) return fail(OQ_EINVAL, "x and q must be 16-byte aligned");
  if (misaligned(scale) || misaligned(bias) || misaligned(y)) return fail(OQ_EINVAL, "scale, bias and y must be 16-byte aligned");
  if (2 * (int64_t)d_in + 16 > 96 * 1024) return fail(OQ_EUNSUPPORTED, "d_in %d too large for the LDS row", d_in);
  {
    const int64_t tt = std::min<int64_t>(16, (96 * 1024) / (2 * (int64_t)d_in + 16));
    if ((T + tt - 1) / tt > 65535) return fail(OQ_EUNSUPPORTED, "T %lld has no launch shape", (long long)T);
  }
  if (T == 0 || d_out == 0) return ok();
  oq::W4Args a{x, T, d_in, d_out, q, scale, group, bias, y, 0};
  hipError_t e = oq::w4a_launch(a, x_dtype == OQ_BF16, stream);
  if (e != hipSuccess) return device_error(e, "oq_linear_w4a16 launch");
  return ok();
}

}  // extern "C"
