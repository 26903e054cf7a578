// The unfused step (measurement only): the elementwise work of the step as kernels of
// their own, every intermediate through HBM, for the fused-versus-unfused comparison
// ("Kernels, Fusion & CUDA Graphs", Fix 1: what each fused kernel replaces; the
// kernel-fusion study, section 8: intermediates round-tripping through memory).  The
// matrix kernels then run with the plain fp32 epilogue and these kernels do the rest:
// RoPE + KV write, SiLU x mul, residual add.

#include "common.h"
#include "epilogue.h"
#include "kernels.h"

namespace dec {

// qkv [Bp][N] fp32 rows of the QKV product -> RoPE on q and k, q -> p.q, k / v -> cache
__global__ __launch_bounds__(256) void k_rope_kv(MatmulParams p, const float* qkv, bool kv_fp8) {
  const int pairs = p.N / 2;
  const int idx = blockIdx.x * 256 + threadIdx.x;
  if (idx >= p.Bp * pairs) return;
  const int b = idx / pairs, i = idx % pairs;
  const f32x2 v = gld(reinterpret_cast<const f32x2*>(qkv + (int64_t)b * p.N + 2 * i));
  qkv_pair_out(p, kv_fp8, b, 2 * i, v.x, v.y);
}

// a[b][i] = bf16(silu(gu[b][i]) * gu[b][d_ff + i])
__global__ __launch_bounds__(256) void k_silu_mul(const float* gu, int d_ff, int Bp, uint16_t* a, int lda) {
  const int idx = blockIdx.x * 256 + threadIdx.x;
  if (idx >= Bp * d_ff) return;
  const int b = idx / d_ff, i = idx % d_ff;
  const float* row = gu + (int64_t)b * 2 * d_ff;
  gst(a + (int64_t)b * lda + i, f32_to_bf16(silu_f(gld(row + i)) * gld(row + d_ff + i)));
}

// h += delta (n elements)
__global__ __launch_bounds__(256) void k_add(float* h, const float* delta, int n) {
  const int idx = blockIdx.x * 256 + threadIdx.x;
  if (idx >= n) return;
  gst(h + idx, gld(h + idx) + gld(delta + idx));
}

hipError_t launch_rope_kv(const MatmulParams& p, const float* qkv, bool kv_fp8, hipStream_t s) {
  const int n = p.Bp * (p.N / 2);
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_rope_kv, dim3((n + 255) / 256), dim3(256), 0, s, p, qkv, kv_fp8);
  return hipGetLastError();
}

hipError_t launch_silu_mul(const float* gu, int d_ff, int Bp, uint16_t* a, int lda, hipStream_t s) {
  const int n = Bp * d_ff;
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_silu_mul, dim3((n + 255) / 256), dim3(256), 0, s, gu, d_ff, Bp, a, lda);
  return hipGetLastError();
}

hipError_t launch_add(float* h, const float* delta, int n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_add, dim3((n + 255) / 256), dim3(256), 0, s, h, delta, n);
  return hipGetLastError();
}

}  // namespace dec
