// Greedy sampling after the LM head: the argmax of each sequence's logits row, on the
// device, so that only the token ids -- not the vocabulary-sized logits -- need to leave
// the GPU ("Kernels, Fusion & CUDA Graphs", Fix 1: the sampling kernel keeps the logits
// on chip; "The serving engine's kernel stack": a sampling kernel turns logits into
// token ids before the small copy back to the CPU).
//
// One work group of 1024 threads per row; every thread scans a strided share of the row
// keeping the first largest value, then the work group reduces (value, index) pairs,
// larger value first, lower index on ties.  NaN never wins; a row with no number
// larger than -inf returns the first -inf, a row of NaN returns 0.

#include "common.h"
#include "kernels.h"

namespace dec {

namespace {
constexpr int AT = 1024;  // threads per row

__device__ __forceinline__ bool better(float v, int i, float bv, int bi) {
  // bi < 0: nothing held yet (then any non-NaN value is taken)
  return v > bv || (v == bv && (bi < 0 || (i >= 0 && i < bi)));
}
}  // namespace

__global__ __launch_bounds__(AT) void k_argmax(const float* logits, int ldl, int V, int32_t* out) {
  __shared__ float sv[AT / WAVE];
  __shared__ int si[AT / WAVE];
  const int row = blockIdx.x, tid = threadIdx.x, lane = tid % WAVE, w = tid / WAVE;
  const float* z = logits + (int64_t)row * ldl;
  float bv = -INFINITY;
  int bi = -1;
  for (int i = tid; i < V; i += AT) {
    const float v = gld(z + i);
    if (better(v, i, bv, bi)) { bv = v; bi = i; }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const float ov = __shfl_xor(bv, off);
    const int oi = __shfl_xor(bi, off);
    if (oi >= 0 && better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
  }
  if (lane == 0) { sv[w] = bv; si[w] = bi; }
  __syncthreads();
  if (tid == 0) {
    for (int k = 1; k < AT / WAVE; ++k)
      if (si[k] >= 0 && better(sv[k], si[k], bv, bi)) { bv = sv[k]; bi = si[k]; }
    gst(out + row, bi < 0 ? 0 : bi);
  }
}

hipError_t launch_argmax(const float* logits, int ldl, int V, int n, int32_t* out, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_argmax, dim3(n), dim3(AT), 0, s, logits, ldl, V, out);
  return hipGetLastError();
}

}  // namespace dec
