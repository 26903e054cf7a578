// Epilogues of the weight-streaming matrix kernels: what each fused kernel does with its
// fp32 row sums ("Kernels, Fusion & CUDA Graphs", Fix 1 table of fused kernels).
#pragma once

#include "common.h"
#include "kernels.h"

namespace dec {

__device__ __forceinline__ float silu_f(float z) { return z / (1.0f + __expf(-z)); }

// Rows (r0, r0 + 1) of the fused QKV matrix for batch row b, values v0, v1 (scaled).
__device__ __forceinline__ void qkv_pair_out(const MatmulParams& p, bool kv_fp8, int b, int r0,
                                             float v0, float v1) {
  const int dh = p.dh;
  const int qrows = p.Hq * dh, krows = p.Hkv * dh;
  const int pos = gld(p.seq_lens + b);
  const int pr = pos < 0 ? 0 : pos;
  if (r0 < qrows + krows) {  // q or k: rotate the adjacent pair (r0 even)
    const int e = r0 % dh;
    const f32x2 cs = gld(reinterpret_cast<const f32x2*>(p.rope + (int64_t)pr * (dh / 2) + (e >> 1)));
    const float y0 = v0 * cs.x - v1 * cs.y;
    const float y1 = v0 * cs.y + v1 * cs.x;
    v0 = y0;
    v1 = y1;
  }
  if (r0 < qrows) {
    const int j = r0 / dh, e = r0 % dh;
    cst_f2(p.q + ((int64_t)b * p.Hq + j) * dh + e, v0, v1);
    return;
  }
  if (pos < 0) return;  // padded row: no cache write
  const int kv = r0 < qrows + krows ? 0 : 1;
  const int rr = r0 - qrows - kv * krows;
  const int c = rr / dh, e = rr % dh;
  const int blk = gld(p.bt + (int64_t)b * p.bps + pos / KV_BLOCK);
  const int64_t off = kv_offset(p.layer, kv, blk, c, pos % KV_BLOCK, e, p.num_blocks, p.Hkv, dh);
  if (kv_fp8) {
    const uint32_t c0 = f32_to_e4m3(v0), c1 = f32_to_e4m3(v1);
    cst(reinterpret_cast<uint16_t*>(static_cast<uint8_t*>(p.pool) + off), (uint16_t)(c0 | (c1 << 8)));
  } else {
    const uint32_t w = (uint32_t)f32_to_bf16(v0) | ((uint32_t)f32_to_bf16(v1) << 16);
    cst(reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(p.pool) + off), w);
  }
}

// Epilogue for one row pair (r0, r1) and batch row b; a0/a1 are unscaled sums.
template <int EPI>
__device__ __forceinline__ void pair_epilogue(const MatmulParams& p, bool kv_fp8, int b, int item, int r0,
                                              int r1, float a0, float a1) {
  const float s0 = p.scale ? gld(p.scale + r0) : 1.0f;
  const float s1 = p.scale ? gld(p.scale + r1) : 1.0f;
  const float y0 = a0 * s0, y1 = a1 * s1;
  if (EPI == EPI_LOGITS) {
    float* o = p.out + (int64_t)b * p.ldo;
    gst(o + r0, y0);
    gst(o + r1, y1);
  } else if (EPI == EPI_RESID) {
    float* o = p.out + (int64_t)b * p.ldo;
    cst(o + r0, cld(o + r0) + y0);
    cst(o + r1, cld(o + r1) + y1);
  } else if (EPI == EPI_SILU) {
    cst(p.act + (int64_t)b * p.ldact + item, f32_to_bf16(silu_f(y0) * y1));
  } else {
    qkv_pair_out(p, kv_fp8, b, r0, y0, y1);
  }
}

// The per-op kernels fetch what their epilogue reads (scales, the residual rows, the
// token's position, RoPE angles and cache block) when they start, so that these loads
// overlap the weight stream instead of following it.
template <int EPI, int BT>
struct EpiInputs {
  float s0, s1;
  float h0[EPI == EPI_RESID ? BT : 1], h1[EPI == EPI_RESID ? BT : 1];
  int pos[EPI == EPI_QKV ? BT : 1], blk[EPI == EPI_QKV ? BT : 1];
  f32x2 cs[EPI == EPI_QKV ? BT : 1];
};

template <int EPI, int BT>
__device__ __forceinline__ void epi_fetch(const MatmulParams& p, int r0, int r1, EpiInputs<EPI, BT>& in) {
  in.s0 = p.scale ? gld(p.scale + r0) : 1.0f;
  in.s1 = p.scale ? gld(p.scale + r1) : 1.0f;
  if (EPI == EPI_RESID) {
#pragma unroll
    for (int b = 0; b < BT; ++b) {
      const float* o = p.out + (int64_t)b * p.ldo;
      in.h0[b] = gld(o + r0);
      in.h1[b] = gld(o + r1);
    }
  }
  if (EPI == EPI_QKV) {
    const int qrows = p.Hq * p.dh, krows = p.Hkv * p.dh;
#pragma unroll
    for (int b = 0; b < BT; ++b) {
      in.pos[b] = gld(p.seq_lens + b);
      const int pr = in.pos[b] < 0 ? 0 : in.pos[b];
      in.cs[b] = r0 < qrows + krows
                     ? gld(reinterpret_cast<const f32x2*>(p.rope + (int64_t)pr * (p.dh / 2) + ((r0 % p.dh) >> 1)))
                     : f32x2{1.f, 0.f};
      in.blk[b] = r0 >= qrows && in.pos[b] >= 0 ? gld(p.bt + (int64_t)b * p.bps + in.pos[b] / KV_BLOCK) : 0;
    }
  }
}

// pair_epilogue with the inputs fetched by epi_fetch
template <int EPI, int BT>
__device__ __forceinline__ void pair_epilogue_pre(const MatmulParams& p, bool kv_fp8, const EpiInputs<EPI, BT>& in,
                                                  int b, int item, int r0, int r1, float a0, float a1) {
  float y0 = a0 * in.s0, y1 = a1 * in.s1;
  if (EPI == EPI_LOGITS) {
    float* o = p.out + (int64_t)b * p.ldo;
    gst(o + r0, y0);
    gst(o + r1, y1);
  } else if (EPI == EPI_RESID) {
    float* o = p.out + (int64_t)b * p.ldo;
    gst(o + r0, in.h0[b] + y0);
    gst(o + r1, in.h1[b] + y1);
  } else if (EPI == EPI_SILU) {
    gst(p.act + (int64_t)b * p.ldact + item, f32_to_bf16(silu_f(y0) * y1));
  } else {
    const int dh = p.dh, qrows = p.Hq * dh, krows = p.Hkv * dh;
    if (r0 < qrows + krows) {  // q or k: rotate the adjacent pair (r0 even)
      const f32x2 cs = in.cs[b];
      const float z0 = y0 * cs.x - y1 * cs.y;
      const float z1 = y0 * cs.y + y1 * cs.x;
      y0 = z0;
      y1 = z1;
    }
    if (r0 < qrows) {
      const int j = r0 / dh, e = r0 % dh;
      float* qp = p.q + ((int64_t)b * p.Hq + j) * dh + e;
      gst(reinterpret_cast<f32x2*>(qp), f32x2{y0, y1});
      return;
    }
    const int pos = in.pos[b];
    if (pos < 0) return;  // padded row: no cache write
    const int kv = r0 < qrows + krows ? 0 : 1;
    const int rr = r0 - qrows - kv * krows;
    const int c = rr / dh, e = rr % dh;
    const int64_t off = kv_offset(p.layer, kv, in.blk[b], c, pos % KV_BLOCK, e, p.num_blocks, p.Hkv, dh);
    if (kv_fp8) {
      const uint32_t c0 = f32_to_e4m3(y0), c1 = f32_to_e4m3(y1);
      uint16_t* kp = reinterpret_cast<uint16_t*>(static_cast<uint8_t*>(p.pool) + off);
      gst(kp, (uint16_t)(c0 | (c1 << 8)));
    } else {
      const uint32_t w = (uint32_t)f32_to_bf16(y0) | ((uint32_t)f32_to_bf16(y1) << 16);
      uint32_t* kp = reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(p.pool) + off);
      gst(kp, w);
    }
  }
}

template <int EPI>
__device__ __forceinline__ void item_rows(const MatmulParams& p, int item, int& r0, int& r1) {
  if (EPI == EPI_SILU) {
    r0 = item;
    r1 = item + p.d_ff;
  } else {
    r0 = 2 * item;
    r1 = 2 * item + 1;
  }
}

}  // namespace dec
