// Embedding gather, RMSNorm, RoPE table and the HBM bandwidth probe.
//
// RMSNorm (Zhang & Sennrich, cited by the kernel-fusion architecture study):
// x_i = g_i h_i / sqrt(mean_j h_j^2 + eps), computed in fp32 from the fp32
// residual stream and stored as the bf16 operand of the next matrix kernel.

#include "common.h"
#include "kernels.h"

namespace dec {

// One work group of 256 threads per batch row.  Each thread keeps its NV float4 of the
// row in registers, so the row is read once and the kernel costs one load round trip
// plus a block reduction (NV * 1024 >= d; NV = 0 selects a two-pass loop for wider rows).
template <bool EMBED, int WQ, int NV>
__global__ __launch_bounds__(256) void k_norm(NormParams p) {
  __shared__ float red[4];
  const int b = blockIdx.x, tid = threadIdx.x;
  if (EMBED && b == 0)
    for (int i = tid; i < p.n_pend; i += 256) cst(p.pend + i, ATTN_O_PENDING2);
  const int d = p.d;  // a multiple of 16
  const float* hrow = p.h + (int64_t)b * d;
  float* hout = p.h_out ? p.h_out + (int64_t)b * d : nullptr;
  uint16_t* xrow = p.x + (int64_t)b * d;
  const int64_t id = EMBED ? (int64_t)p.ids[b] : 0;
  const float e_scale = (EMBED && WQ != W_BF16) ? p.E_scale[id] : 1.f;
  // 4 consecutive elements of the row starting at i (embedding rows are dequantized)
  auto load4 = [&](int i) -> f32x4 {
    if (!EMBED) return *reinterpret_cast<const f32x4*>(hrow + i);
    f32x4 v;
    if constexpr (WQ != W_BF16) {
      const uint32_t c = *reinterpret_cast<const uint32_t*>(static_cast<const uint8_t*>(p.E) + id * d + i);
      const f32x2 lo = b8x2_to_f32x2<WQ, false>(c), hi = b8x2_to_f32x2<WQ, true>(c);
      v = f32x4{lo.x * e_scale, lo.y * e_scale, hi.x * e_scale, hi.y * e_scale};
    } else {
      const u32x2 w = *reinterpret_cast<const u32x2*>(static_cast<const uint16_t*>(p.E) + id * d + i);
      v = f32x4{bf16_lo(w.x), bf16_hi(w.x), bf16_lo(w.y), bf16_hi(w.y)};
    }
    *reinterpret_cast<f32x4*>(hout + i) = v;
    return v;
  };
  // x = bf16(y), y = h r g; with x_lo also the remainder bf16(y - x); fp16(y) if x_f16
  uint16_t* xlrow = p.x_lo ? p.x_lo + (int64_t)b * d : nullptr;
  auto store4 = [&](int i, f32x4 v, float r) {
    const f32x4 g = *reinterpret_cast<const f32x4*>(p.gain + i);
    const float y[4] = {v.x * r * g.x, v.y * r * g.y, v.z * r * g.z, v.w * r * g.w};
    uint16_t hb[4], lb[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      hb[j] = p.x_f16 ? f32_to_f16(y[j]) : f32_to_bf16(y[j]);
      lb[j] = f32_to_bf16(y[j] - bf16_to_f32(hb[j]));
    }
    *reinterpret_cast<u32x2*>(xrow + i) =
        u32x2{(uint32_t)hb[0] | ((uint32_t)hb[1] << 16), (uint32_t)hb[2] | ((uint32_t)hb[3] << 16)};
    if (xlrow)
      *reinterpret_cast<u32x2*>(xlrow + i) =
          u32x2{(uint32_t)lb[0] | ((uint32_t)lb[1] << 16), (uint32_t)lb[2] | ((uint32_t)lb[3] << 16)};
  };
  float ss = 0.f;
  if (NV > 0) {
    f32x4 v[NV > 0 ? NV : 1];
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int i = (j * 256 + tid) * 4;
      v[j] = i < d ? load4(i) : f32x4{0.f, 0.f, 0.f, 0.f};
      ss += v[j].x * v[j].x + v[j].y * v[j].y + v[j].z * v[j].z + v[j].w * v[j].w;
    }
    ss = block256_sum(ss, red);
    const float r = 1.0f / sqrtf(ss / (float)d + p.eps);
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int i = (j * 256 + tid) * 4;
      if (i < d) store4(i, v[j], r);
    }
  } else {
    for (int i = tid * 4; i < d; i += 1024) {
      const f32x4 v = load4(i);
      ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
    }
    ss = block256_sum(ss, red);
    const float r = 1.0f / sqrtf(ss / (float)d + p.eps);
    const float* src = EMBED ? hout : hrow;  // this thread's own values, re-read
    for (int i = tid * 4; i < d; i += 1024) store4(i, *reinterpret_cast<const f32x4*>(src + i), r);
  }
}

namespace {
template <bool EMBED, int WQ>
hipError_t norm_go(const NormParams& p, hipStream_t s) {
  if (p.x_f16 && p.x_lo) return hipErrorInvalidValue;  // fp16 x is one part
  const int nv = (p.d + 1023) / 1024;
  if (nv <= 1) hipLaunchKernelGGL((k_norm<EMBED, WQ, 1>), dim3(p.Bp), dim3(256), 0, s, p);
  else if (nv <= 2) hipLaunchKernelGGL((k_norm<EMBED, WQ, 2>), dim3(p.Bp), dim3(256), 0, s, p);
  else if (nv <= 4) hipLaunchKernelGGL((k_norm<EMBED, WQ, 4>), dim3(p.Bp), dim3(256), 0, s, p);
  else if (nv <= 8) hipLaunchKernelGGL((k_norm<EMBED, WQ, 8>), dim3(p.Bp), dim3(256), 0, s, p);
  else hipLaunchKernelGGL((k_norm<EMBED, WQ, 0>), dim3(p.Bp), dim3(256), 0, s, p);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_embed_norm(const NormParams& p, WFmt wq, hipStream_t s) {
  switch (wq) {
    case W_E4M3: return norm_go<true, W_E4M3>(p, s);
    case W_I8: return norm_go<true, W_I8>(p, s);
    default: return norm_go<true, W_BF16>(p, s);
  }
}

hipError_t launch_rmsnorm(const NormParams& p, hipStream_t s) { return norm_go<false, W_BF16>(p, s); }

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
