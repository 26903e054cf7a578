// The unfused step (measurement only): the elementwise work of the step as kernels of
// their own, every intermediate through HBM, for the fused-versus-unfused comparison
// ("Kernels, Fusion & CUDA Graphs", Fix 1: what each fused kernel replaces; the
// kernel-fusion study, section 8: intermediates round-tripping through memory).  The
// matrix kernels then run with the plain fp32 epilogue and these kernels do the rest:
// RoPE + KV write, SiLU x mul, residual add -- and attention as the textbook sequence of
// a score product, a softmax and a probability-weighted sum, with the scores written to
// HBM and read back ("GPU Inference Internals", Kernels: FlashAttention and the Memory
// Hierarchy: the naive form materializes the score matrix).

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

// ---------------------------------------------------------------- unfused attention

// scores[b][j][i] = q_j . K_c[i] / sqrt(dh) for positions i <= p_b (c = j / g); work group
// (head j, row b), a thread per position.
template <int DH, bool FP8>
__global__ __launch_bounds__(256) void k_attn_scores(AttnParams p, float* scores, int ld_s) {
  __shared__ float qs[DH];
  const int j = blockIdx.x, b = blockIdx.y, g = p.Hq / p.Hkv, c = j / g;
  const float* qg = p.q + ((int64_t)b * p.Hq + j) * DH;
  for (int e = threadIdx.x; e < DH; e += 256) qs[e] = gld(qg + e) / sqrtf((float)DH);
  __syncthreads();
  const int ntok = gld(p.seq_lens + b) + 1;
  float* srow = scores + ((int64_t)b * p.Hq + j) * ld_s;
  for (int i = threadIdx.x; i < ntok; i += 256) {
    const int blk = gld(p.bt + (int64_t)b * p.bps + i / KV_BLOCK);
    const int64_t off = kv_offset(p.layer, 0, blk, c, i % KV_BLOCK, 0, p.num_blocks, p.Hkv, DH);
    float acc = 0.f;
#pragma unroll 4
    for (int e = 0; e < DH; e += 8) {
      float kf[8];
      if (FP8) {
        const u32x2 w = gld(reinterpret_cast<const u32x2*>(static_cast<const uint8_t*>(p.pool) + off + e));
        const f32x2 a = e4m3x2_to_f32x2<false>(w.x), bb = e4m3x2_to_f32x2<true>(w.x);
        const f32x2 cc = e4m3x2_to_f32x2<false>(w.y), d = e4m3x2_to_f32x2<true>(w.y);
        kf[0] = a.x; kf[1] = a.y; kf[2] = bb.x; kf[3] = bb.y; kf[4] = cc.x; kf[5] = cc.y; kf[6] = d.x; kf[7] = d.y;
      } else {
        const u32x4 w = gld16(static_cast<const uint16_t*>(p.pool) + off + e);
        const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int t = 0; t < 4; ++t) { kf[2 * t] = bf16_lo(ww[t]); kf[2 * t + 1] = bf16_hi(ww[t]); }
      }
#pragma unroll
      for (int t = 0; t < 8; ++t) acc = fmaf(qs[e + t], kf[t], acc);
    }
    gst(srow + i, acc);
  }
}

// softmax in place over positions 0..p of each (row b, head j)
__global__ __launch_bounds__(256) void k_softmax_rows(AttnParams p, float* scores, int ld_s) {
  __shared__ float red[4];
  const int j = blockIdx.x, b = blockIdx.y;
  const int ntok = gld(p.seq_lens + b) + 1;
  float* srow = scores + ((int64_t)b * p.Hq + j) * ld_s;
  float mx = -INFINITY;
  for (int i = threadIdx.x; i < ntok; i += 256) mx = fmaxf(mx, gld(srow + i));
  mx = wave_max(mx);
  __syncthreads();
  if (threadIdx.x % WAVE == 0) red[threadIdx.x / WAVE] = mx;
  __syncthreads();
  mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  float sum = 0.f;
  for (int i = threadIdx.x; i < ntok; i += 256) sum += __expf(gld(srow + i) - mx);
  sum = block256_sum(sum, red);
  for (int i = threadIdx.x; i < ntok; i += 256) gst(srow + i, __expf(gld(srow + i) - mx) / sum);
}

// o[b][j][e] = sum_i P[b][j][i] V_c[i][e]; work group (head j, row b), a thread per element e
template <int DH, bool FP8>
__global__ __launch_bounds__(DH) void k_attn_pv(AttnParams p, const float* scores, int ld_s) {
  const int j = blockIdx.x, b = blockIdx.y, g = p.Hq / p.Hkv, c = j / g, e = threadIdx.x;
  const int ntok = gld(p.seq_lens + b) + 1;
  const float* srow = scores + ((int64_t)b * p.Hq + j) * ld_s;
  float acc = 0.f;
  for (int i = 0; i < ntok; ++i) {
    const int blk = gld(p.bt + (int64_t)b * p.bps + i / KV_BLOCK);
    const int64_t off = kv_offset(p.layer, 1, blk, c, i % KV_BLOCK, e, p.num_blocks, p.Hkv, DH);
    float v;
    if (FP8) {
      const uint32_t code = static_cast<const uint8_t*>(p.pool)[off];
      v = e4m3x2_to_f32x2<false>(code).x;
    } else {
      v = bf16_to_f32(static_cast<const uint16_t*>(p.pool)[off]);
    }
    acc = fmaf(gld(srow + i), v, acc);
  }
  gst(p.o + ((int64_t)b * p.Hq + j) * DH + e, f32_to_bf16(acc));
}

template <int DH, bool FP8>
hipError_t attn_unfused_go(const AttnParams& p, float* scores, int ld_s, hipStream_t s) {
  const dim3 grid(p.Hq, p.Bp);
  hipLaunchKernelGGL((k_attn_scores<DH, FP8>), grid, dim3(256), 0, s, p, scores, ld_s);
  hipLaunchKernelGGL(k_softmax_rows, grid, dim3(256), 0, s, p, scores, ld_s);
  hipLaunchKernelGGL((k_attn_pv<DH, FP8>), grid, dim3(DH), 0, s, p, scores, ld_s);
  return hipGetLastError();
}

hipError_t launch_attention_unfused(const AttnParams& p, float* scores, int ld_s, bool kv_fp8, hipStream_t s) {
  if (p.dh == 64) return kv_fp8 ? attn_unfused_go<64, true>(p, scores, ld_s, s) : attn_unfused_go<64, false>(p, scores, ld_s, s);
  if (p.dh == 128)
    return kv_fp8 ? attn_unfused_go<128, true>(p, scores, ld_s, s) : attn_unfused_go<128, false>(p, scores, ld_s, s);
  return hipErrorInvalidValue;
}

// ---------------------------------------------------------------- launchers

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
