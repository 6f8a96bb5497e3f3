// Folding the next layer's input permutation into this layer's output
// channels (offline).
//
// Method: "OrbitQuant: data-agnostic quantization for image and video"
// (rcap.io summary): the RPBH rotation of a layer's input starts with a
// uniform random permutation (RPBH paragraph), applied to every token online
// (online pseudo-code).  When that input is an elementwise function of the
// previous quantized linear's output (the GELU of an MLP's up projection),
// the permutation can move into the previous layer: a layer whose output
// channels are reordered, o' = perm[o], produces the permuted vector, and the
// elementwise GELU keeps the order.  The next rotate-quantize then gathers
// with the identity: only the sign flips and the block Hadamard remain.
//
// A quantized layer's output channel o is row o of its packed weight
// indices, its row norm and its bias, so folding is a row permutation of
// those three arrays: out[i] = in[perm[i]].  Offline, not on the hot path.
#include "oq_internal.h"

namespace oq {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// One workgroup per output row: the row's packed indices in 16-byte pieces
// (a whole number of them: row_bytes % 16 == 0), its norm and its bias.
__global__ void __launch_bounds__(256) fold_rows_kernel(const FoldArgs a) {
  const int64_t i = blockIdx.x;
  const int32_t p = a.perm[i];
  const int64_t src = p < 0 ? 0 : (p >= a.rows ? a.rows - 1 : p);   // stays in bounds whatever perm holds
  const u32x4* s = reinterpret_cast<const u32x4*>(a.w_idx + src * a.row_bytes);
  u32x4* d = reinterpret_cast<u32x4*>(a.w_idx_out + i * a.row_bytes);
  for (int64_t k = threadIdx.x; k < a.row_bytes / 16; k += blockDim.x) d[k] = s[k];
  if (threadIdx.x == 0) {
    a.w_norm_out[i] = a.w_norm[src];
    if (a.bias) a.bias_out[i] = a.bias[src];
  }
}

}  // namespace

hipError_t fold_launch(const FoldArgs& a, hipStream_t st) {
  if (a.rows == 0) return hipSuccess;
  hipLaunchKernelGGL(fold_rows_kernel, dim3((unsigned)a.rows), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace oq
