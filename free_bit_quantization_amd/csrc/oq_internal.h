// Internal declarations shared by the C-ABI layer and the HIP kernels.
#ifndef OQ_INTERNAL_H_
#define OQ_INTERNAL_H_

#include <hip/hip_runtime.h>
#include <cstdint>

#include "oq.h"
#include "ql_split.h"

namespace oq {

// ---- host math --------------------------------------------------------------
void build_rpbh_tables(int32_t d, uint64_t seed, int32_t* perm, int8_t* sign);
void build_block_rht_tables(int32_t d, uint64_t seed, int32_t* perm, int8_t* sign);
// 0 on convergence (relative fixed-point residual <= 1e-10), -1 otherwise;
// at most max_newton Newton steps after the Lloyd steps.
constexpr int kLloydMaxNewton = 300;
int lloyd_max_fd(int d, int bits, int max_newton, double* centroids, double* thresholds, double* mse, double* resid);

// ---- rotate-quantize (activations, fp32 fast path + fp64 recheck) ------------
constexpr int kMaxThr = 255;     // 2^8 - 1 thresholds
constexpr int kMaxGrid = 4096;   // cells of the threshold-search grid
constexpr int kHostGrid = 64;    // grids up to this size are built on the host (RqArgs::glut)

struct RqArgs {
  const void* x;
  int64_t T;
  int32_t d;
  int32_t log2h;
  const int32_t* perm;
  const int8_t* sign;
  uint8_t* x_idx;
  float* s;
  float* x_rot;
  int32_t nthr;      // 2^bits - 1
  int32_t G;         // grid cells (power of two), 0 = binary search
  double g_lo;       // grid origin (u units)
  double g_invw;     // cells per unit u
  double g_rmax;     // widening of each cell for the recheck guard (u units)
  float thr_absmax;  // max |thr| (the slot-wide guard radius)
  float thr[kMaxThr];
  float thr_lo[kMaxThr];         // threshold - thr, rounded to fp32: thr + thr_lo is the fp64 threshold to 2^-48
  int32_t glut[kHostGrid][2];   // G <= kHostGrid: cell c -> {bits of its threshold (or +inf), thresholds below it}
};

// Plan of a launch, chosen on the host from (d, h, dtype, bits, T).
struct RqPlan {
  int ns;        // slots (16 coordinates each) per token
  int tpw;       // tokens per workgroup iteration
  int threads;   // workgroup size
  int grid;      // workgroups
  size_t lds;    // dynamic LDS bytes
  int wave_j;    // > 0: one wavefront per token, wave_j slots of 16 coordinates per lane
  int wpb;       // wavefronts per workgroup of that kernel
  int pad;       // workgroup kernel: staged rows padded (16 coordinates per 256)
};

// Returns false if (d, h) has no kernel.
bool rq_plan(int32_t d, int32_t log2h, bool bf16, int32_t bits, int64_t T, int G, RqPlan* plan);
hipError_t rq_launch(const RqArgs& a, bool bf16, int bits, const RqPlan& plan, hipStream_t stream);

// ---- weight quantization (offline, fp64) --------------------------------------
struct WqArgs {
  const void* W;
  int32_t d_out;
  int32_t d;
  int32_t h;
  const int32_t* perm;
  const int8_t* sign;
  uint8_t* w_idx;
  float* w_norm;
  int32_t nthr;
  double thr[kMaxThr];
};
hipError_t wq_launch(const WqArgs& a, bool bf16, int bits, hipStream_t stream);

// ---- codebook GEMM ------------------------------------------------------------
struct QlArgs {
  const uint8_t* x_idx;
  const float* s;
  int64_t T;
  const uint8_t* w_idx;
  const float* w_norm;
  int32_t N;
  int32_t K;
  const float* bias;
  void* y;               // float, or bf16 bits with OQ_EPI_OUT_BF16
  float scale;           // 1 / K (tables hold sqrt(K) * c)
  int32_t epilogue;      // OQ_EPI_NONE / OQ_EPI_GELU_ERF, | OQ_EPI_OUT_BF16
  uint16_t tab_a[256];   // fp16 bits of sqrt(K) * c_a
  uint16_t tab_w[256];   // fp16 bits of sqrt(K) * c_w
  // Work split over the persistent workgroups (ql_split.h).  With a split
  // tail the workgroups exchange fp32 partial tiles through a workspace: hdr
  // (launch generation and started-workgroup count in one word), one flag per
  // workgroup and one 256 x 256 slot per workgroup.
  QlSplit sp;
  uint64_t* hdr;
  uint32_t* flags;
  float* slots;
};
// K indices per pipeline stage of the GEMM (a tile's K is cut into K / stage stages)
inline int ql_stage_k(int bits_a) { return (bits_a == 8 || bits_a == 6) ? 64 : 128; }
hipError_t ql_launch(const QlArgs& a, int bits_a, int bits_w, hipStream_t stream);
// The library's fixed device scratch for the split GEMM (oq_qlinear_splitk_noalloc):
// a workspace laid out for kScratchSlots slots; *ptr = its address on the current device.
constexpr int kScratchSlots = 256;
constexpr int64_t kScratchBytes = 256 + ((kScratchSlots * 4 + 255) / 256) * 256 + (int64_t)kScratchSlots * 256 * 256 * 4;
hipError_t ql_scratch(void** ptr);

// ---- folding the next layer's permutation into the output channels -----------
struct FoldArgs {
  const uint8_t* w_idx;   // [rows][row_bytes]
  const float* w_norm;    // [rows]
  const float* bias;      // [rows] or null
  const int32_t* perm;    // [rows]
  int64_t rows;
  int64_t row_bytes;      // multiple of 16
  uint8_t* w_idx_out;
  float* w_norm_out;
  float* bias_out;
};
hipError_t fold_launch(const FoldArgs& a, hipStream_t stream);

// ---- INT4 round-to-nearest weight-only linear (AdaLN modulation) --------------
struct RtnArgs {
  const void* W;      // [N][K] fp32 or bf16
  int32_t N;
  int32_t K;
  int32_t group;      // input columns per scale, multiple of 128 dividing K
  uint8_t* q;         // [N][K / 2] two's-complement nibbles
  float* scale;       // [N][K / group]
};
hipError_t rtn_launch(const RtnArgs& a, bool bf16, hipStream_t stream);

struct W4Args {
  const void* x;      // [T][K] bf16 or fp16
  int64_t T;
  int32_t K;
  int32_t N;
  const uint8_t* q;
  const float* scale;
  int32_t group;
  const float* bias;  // [N] or null
  float* y;           // [T][N]
  int32_t tt;         // tokens per workgroup (set by w4a_launch)
};
hipError_t w4a_launch(const W4Args& a, bool bf16, hipStream_t stream);

}  // namespace oq

#endif  // OQ_INTERNAL_H_
