// Embedding gather, RMSNorm, RoPE table and the HBM bandwidth probe.
//
// RMSNorm (Zhang & Sennrich, cited by the kernel-fusion architecture study):
// x_i = g_i h_i / sqrt(mean_j h_j^2 + eps), computed in fp32 from the fp32
// residual stream and stored as the bf16 operand of the next matrix kernel.

#include "common.h"
#include "kernels.h"

namespace dec {

// one work group of 256 threads per batch row
template <bool EMBED, bool FP8>
__global__ __launch_bounds__(256) void k_norm(NormParams p) {
  __shared__ float red[4];
  const int b = blockIdx.x;
  const int d = p.d;
  const float* hrow = p.h + (int64_t)b * d;
  float* hout = p.h_out ? p.h_out + (int64_t)b * d : nullptr;
  float ss = 0.f;
  float e_scale = 1.f;
  const int64_t id = EMBED ? (int64_t)p.ids[b] : 0;
  if (EMBED && FP8) e_scale = p.E_scale[id];
  // pass 1: (gather) and sum of squares; each thread covers elements tid, tid + 256, ...
  for (int i = threadIdx.x; i < d; i += 256) {
    float v;
    if (EMBED) {
      if (FP8) {
        const uint8_t c = static_cast<const uint8_t*>(p.E)[id * d + i];
        v = e4m3x2_to_f32x2<false>((uint32_t)c).x * e_scale;
      } else {
        v = bf16_to_f32(static_cast<const uint16_t*>(p.E)[id * d + i]);
      }
      hout[i] = v;
    } else {
      v = hrow[i];
    }
    ss += v * v;
  }
  ss = block256_sum(ss, red);
  const float r = 1.0f / sqrtf(ss / (float)d + p.eps);
  // pass 2: normalize (re-reading our own values)
  const float* src = EMBED ? hout : hrow;
  for (int i = threadIdx.x; i < d; i += 256) p.x[(int64_t)b * d + i] = f32_to_bf16(src[i] * r * p.gain[i]);
}

hipError_t launch_embed_norm(const NormParams& p, bool w_fp8, hipStream_t s) {
  if (w_fp8)
    hipLaunchKernelGGL((k_norm<true, true>), dim3(p.Bp), dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL((k_norm<true, false>), dim3(p.Bp), dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_rmsnorm(const NormParams& p, hipStream_t s) {
  hipLaunchKernelGGL((k_norm<false, false>), dim3(p.Bp), dim3(256), 0, s, p);
  return hipGetLastError();
}

// RoPE angles phi = p * theta^(-2i/dh) (RoFormer, adjacent pairs), in double precision
__global__ void k_rope_table(float2* rope, int max_seq, int half, double theta) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)max_seq * half) return;
  const int pos = (int)(idx / half), i = (int)(idx % half);
  const double inv = pow(theta, -2.0 * (double)i / (double)(2 * half));
  const double phi = (double)pos * inv;
  rope[idx] = make_float2((float)cos(phi), (float)sin(phi));
}

hipError_t launch_rope_table(float2* rope, int max_seq, int dh, double theta, hipStream_t s) {
  const int half = dh / 2;
  const int64_t n = (int64_t)max_seq * half;
  const int grid = (int)((n + 255) / 256);
  hipLaunchKernelGGL(k_rope_table, dim3(grid), dim3(256), 0, s, rope, max_seq, half, theta);
  return hipGetLastError();
}

// read-only streaming sum over the buffer; the sink write is never taken in practice
__global__ __launch_bounds__(256) void k_bw_probe(const u32x4* __restrict__ buf, size_t n16, float* sink) {
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  uint32_t acc = 0;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u32x4 a = ld_stream(buf + i), b = ld_stream(buf + i + stride);
    const u32x4 c = ld_stream(buf + i + 2 * stride), d = ld_stream(buf + i + 3 * stride);
    acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^ d.z ^ d.w;
  }
  for (; i < n16; i += stride) {
    const u32x4 a = ld_stream(buf + i);
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  if (acc == 0x9E3779B9u && sink) sink[0] = 1.0f;
}

hipError_t launch_bw_probe(const void* buf, size_t bytes, float* sink, hipStream_t s) {
  hipLaunchKernelGGL(k_bw_probe, dim3(512), dim3(256), 0, s, static_cast<const u32x4*>(buf), bytes / 16, sink);
  return hipGetLastError();
}

}  // namespace dec
