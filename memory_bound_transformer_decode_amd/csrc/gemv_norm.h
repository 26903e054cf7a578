// The norm-fused matrix-vector product of one work group.
#pragma once

#include "common.h"
#include "epilogue.h"
#include "kernels.h"

namespace dec {

// RMSNorm of the layer input costs no kernel of its own (h is a few KB per row and
// L2-resident; the kernel-fusion study's section 8 on intermediates round-tripping
// through HBM).  IPW waves per work group, one row pair per wave.  The first pass's
// weight loads are issued before the norm, so the norm runs under the weight stream.
//
// The work of work group `group`: ipw <= IPW_MAX waves, items group ipw .. group ipw +
// ipw - 1; xs is LDS of BT K bf16, twice that for QKV, whose input is kept as two bf16
// parts (x, then the remainder bf16(v - x) at xs + BT K: see MatmulParams::xl).
template <int BT, int WQ, int EPI, bool KVFP8, int U, int IPW_MAX>
__device__ __forceinline__ void gemv_norm_group(const MatmulParams& p, int n_items, int group, uint16_t* xs,
                                                int ipw) {
  constexpr bool XL = EPI == EPI_QKV;
  __shared__ float red[IPW_MAX][BT];
  constexpr int EPV = WQ != W_BF16 ? 16 : 8;
  const int NT = WAVE * ipw;
  const int tid = threadIdx.x, lane = tid % WAVE;
  const int w = __builtin_amdgcn_readfirstlane(tid / WAVE);
  const int K = p.K, KV = K / EPV;
  const int it = group * ipw + w;
  const bool have = it < n_items;
  int r0, r1;
  item_rows<EPI>(p, have ? it : n_items - 1, r0, r1);  // a wave without an item loads a valid row
  const u32x4* W = static_cast<const u32x4*>(p.W);
  const u32x4* w0p = W + (int64_t)r0 * KV;
  const u32x4* w1p = W + (int64_t)r1 * KV;

  // sum of squares of this thread's elements of each row (issued first: L2 hits that
  // complete ahead of the weight loads).  For small batches the thread keeps its h and
  // gain values in registers, so that x can be written without a second read, which
  // would queue behind the weight loads.
  constexpr int NHR = BT <= 2 ? 3 : 1;  // float4 of h per row held per thread (K <= 12 NT)
  const bool held = BT <= 2 && K <= NHR * NT * 4;
  f32x4 hv[BT][NHR], gv[NHR];
  float ss[BT];
#pragma unroll
  for (int b = 0; b < BT; ++b) ss[b] = 0.f;
  if (held) {
#pragma unroll
    for (int j = 0; j < NHR; ++j) {
      const int i = min((j * NT + tid) * 4, K - 4);  // past K: a re-read that is not counted
      const bool in = (j * NT + tid) * 4 < K;
      gv[j] = gld(reinterpret_cast<const f32x4*>(p.ng + i));
#pragma unroll
      for (int b = 0; b < BT; ++b) {
        hv[b][j] = gld(reinterpret_cast<const f32x4*>(p.nh + (int64_t)b * K + i));
        const f32x4 v = hv[b][j];
        ss[b] += in ? v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w : 0.f;
      }
    }
  } else {
    for (int i = tid * 4; i < K; i += NT * 4) {
#pragma unroll
      for (int b = 0; b < BT; ++b) {
        const f32x4 v = gld(reinterpret_cast<const f32x4*>(p.nh + (int64_t)b * K + i));
        ss[b] += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
      }
    }
  }
  EpiInputs<EPI, BT> ein;
  if (lane == 0) epi_fetch<EPI, BT>(p, r0, r1, ein);

  u32x4 w0[U], w1[U];
  auto load_pass = [&](int k0) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int kk = k0 + WAVE * u;
      if (kk < KV) {
        w0[u] = ld_stream(w0p + kk);
        w1[u] = ld_stream(w1p + kk);
      }
    }
  };
  float acc0[BT], acc1[BT];
#pragma unroll
  for (int b = 0; b < BT; ++b) acc0[b] = acc1[b] = 0.0f;
  auto compute_pass = [&](int k0) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int kk = k0 + WAVE * u;
      if (kk < KV) {
        // one-byte weights widened once to bf16 (elements 0..7, 8..15 of the vector)
        u32x4 v0a, v0b, v1a, v1b;
        if constexpr (WQ != W_BF16) {
          widen16_b8<WQ>(w0[u], v0a, v0b);
          widen16_b8<WQ>(w1[u], v1a, v1b);
        } else {
          v0a = w0[u];
          v1a = w1[u];
        }
#pragma unroll
        for (int part = 0; part < (XL ? 2 : 1); ++part) {
#pragma unroll
          for (int b = 0; b < BT; ++b) {
            const uint16_t* xb = xs + (part * BT + b) * K + kk * EPV;
            const u32x4 xa = *reinterpret_cast<const u32x4*>(xb);
            acc0[b] = dot8_bf16(v0a, xa, acc0[b]);
            acc1[b] = dot8_bf16(v1a, xa, acc1[b]);
            if constexpr (WQ != W_BF16) {
              const u32x4 xc = *reinterpret_cast<const u32x4*>(xb + 8);
              acc0[b] = dot8_bf16(v0b, xc, acc0[b]);
              acc1[b] = dot8_bf16(v1b, xc, acc1[b]);
            }
          }
        }
      }
    }
  };
  load_pass(lane);

  // the norm: reduce the sums over the work group, then write x into LDS
#pragma unroll
  for (int b = 0; b < BT; ++b) {
    const float t = wave_sum(ss[b]);
    if (lane == 0) red[w][b] = t;
  }
  __syncthreads();
  float r[BT];
#pragma unroll
  for (int b = 0; b < BT; ++b) {
    float t = 0.f;
#pragma unroll
    for (int ww = 0; ww < ipw; ++ww) t += red[ww][b];
    r[b] = 1.0f / sqrtf(t / (float)K + p.eps);
  }
  auto put_x = [&](int i, int b, const f32x4& v, const f32x4& g) {
    const float y[4] = {v.x * r[b] * g.x, v.y * r[b] * g.y, v.z * r[b] * g.z, v.w * r[b] * g.w};
    uint16_t hb[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) hb[j] = f32_to_bf16(y[j]);
    *reinterpret_cast<u32x2*>(xs + b * K + i) =
        u32x2{(uint32_t)hb[0] | ((uint32_t)hb[1] << 16), (uint32_t)hb[2] | ((uint32_t)hb[3] << 16)};
    if constexpr (XL) {
      uint16_t lb[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) lb[j] = f32_to_bf16(y[j] - bf16_to_f32(hb[j]));
      *reinterpret_cast<u32x2*>(xs + (BT + b) * K + i) =
          u32x2{(uint32_t)lb[0] | ((uint32_t)lb[1] << 16), (uint32_t)lb[2] | ((uint32_t)lb[3] << 16)};
    }
  };
  if (held) {
#pragma unroll
    for (int j = 0; j < NHR; ++j) {
      const int i = (j * NT + tid) * 4;
      if (i < K) {
#pragma unroll
        for (int b = 0; b < BT; ++b) put_x(i, b, hv[b][j], gv[j]);
      }
    }
  } else {
    for (int i = tid * 4; i < K; i += NT * 4) {
      const f32x4 g = gld(reinterpret_cast<const f32x4*>(p.ng + i));
#pragma unroll
      for (int b = 0; b < BT; ++b) put_x(i, b, gld(reinterpret_cast<const f32x4*>(p.nh + (int64_t)b * K + i)), g);
    }
  }
  __syncthreads();

  compute_pass(lane);
  for (int k0 = lane + WAVE * U; k0 < KV; k0 += WAVE * U) {
    load_pass(k0);
    compute_pass(k0);
  }
#pragma unroll
  for (int b = 0; b < BT; ++b) {
    acc0[b] = wave_sum(acc0[b]);
    acc1[b] = wave_sum(acc1[b]);
  }
  if (lane == 0 && have) {
#pragma unroll
    for (int b = 0; b < BT; ++b) pair_epilogue_pre<EPI, BT>(p, KVFP8, ein, b, it, r0, r1, acc0[b], acc1[b]);
  }
}

}  // namespace dec
