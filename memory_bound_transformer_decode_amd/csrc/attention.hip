// Split-K paged grouped-query decode attention.
//
// One query token per sequence attends to its cached positions 0..p (p = seq_len,
// the new token included).  The work is exact softmax attention computed
// tile-by-tile with a running max and sum, never materializing the score vector
// in HBM (FlashAttention, cited by "GPU Inference Internals", section Kernels:
// FlashAttention and the Memory Hierarchy), over a paged cache addressed through a
// per-sequence block table (PagedAttention).  The KV read of each new token is the
// term B S K of the step ledger that does not amortize over the batch ("GPU
// Inference Internals", Batching Economics), so every K/V tile is read once and
// shared by the g = Hq / Hkv query heads of its group.
//
// k_attn_split: work group (split j, kv head c, sequence b), 4 waves.  The blocks
// of positions 0..p are divided evenly between n_split work groups; each wave of a
// work group takes every 4th block.  A lane holds 16 bytes of one position's K and
// V row; scores are reduced over the lanes of a row, then the running max m, sum l
// and output o are updated (base-2 exponentials with log2(e) folded into q).  The
// waves merge in LDS and the work group writes (m, l, o) for each of its heads.
// The last work group of a (sequence, kv head) to finish -- counted by a
// self-resetting arrival counter -- combines the splits:
// o = sum_j 2^(m_j - M) o_j / sum_j 2^(m_j - M) l_j, M = max_j m_j, as bf16; a
// sequence with no positions (a padded row) gets o = 0.  Partials go through
// device-coherent stores and loads, since the work groups of one (sequence, kv
// head) run on different XCDs, whose L2 caches are not coherent with each other.

#include "common.h"
#include "kernels.h"

namespace dec {

constexpr int MAX_SPLIT = 64;  // splits per (sequence, kv head); the host keeps n_split within it

template <int DH, bool FP8, int G>
__global__ __launch_bounds__(256) void k_attn_split(AttnParams p) {
  constexpr int EPL = FP8 ? 16 : 8;  // cache elements per 16-byte load
  constexpr int LPP = DH / EPL;      // lanes per position row
  constexpr int PPP = WAVE / LPP;    // positions per pass
  constexpr int NPASS = KV_BLOCK / PPP;
  constexpr int NW = 4;
  const int split = blockIdx.x, c = blockIdx.y, b = blockIdx.z;
  const int wave = threadIdx.x / WAVE, lane = threadIdx.x % WAVE;
  const int prow = lane / LPP, eoff = (lane % LPP) * EPL;

  const int pos = p.seq_lens[b];
  const int ntok = pos + 1;  // 0 for a padded row
  const int nblk = pos >= 0 ? pos / KV_BLOCK + 1 : 0;
  const int per = (nblk + p.n_split - 1) / p.n_split;
  const int blk0 = split * per;
  const int blk1 = min(nblk, blk0 + per);

  const float qscale = 1.4426950408889634f / sqrtf((float)DH);  // log2(e) / sqrt(dh)
  float qv[G][EPL];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float* qh = p.q + ((int64_t)b * p.Hq + c * G + h) * DH + eoff;
#pragma unroll
    for (int e = 0; e < EPL; e += 4) {
      const float4 t = *reinterpret_cast<const float4*>(qh + e);
      qv[h][e] = t.x * qscale;
      qv[h][e + 1] = t.y * qscale;
      qv[h][e + 2] = t.z * qscale;
      qv[h][e + 3] = t.w * qscale;
    }
  }

  float m[G], l[G], o[G][EPL];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) o[h][e] = 0.f;
  }

  const uint8_t* pool = static_cast<const uint8_t*>(p.pool);
  constexpr int ESZ = FP8 ? 1 : 2;

  for (int blk = blk0 + wave; blk < blk1; blk += NW) {
    const int phys = p.bt[(int64_t)b * p.bps + blk];
    const int64_t kbase = kv_offset(p.layer, 0, phys, c, 0, 0, p.num_blocks, p.Hkv, DH);
    const int64_t vbase = kv_offset(p.layer, 1, phys, c, 0, 0, p.num_blocks, p.Hkv, DH);
    u32x4 kr[NPASS], vr[NPASS];
#pragma unroll
    for (int ps = 0; ps < NPASS; ++ps) {
      const int64_t off = (int64_t)(ps * PPP + prow) * DH + eoff;
      kr[ps] = ld16(pool + (kbase + off) * ESZ);
      vr[ps] = ld16(pool + (vbase + off) * ESZ);
    }
    float sc[NPASS][G];
    bool vld[NPASS];  // slots past the last position may hold anything (even NaN): mask them
#pragma unroll
    for (int ps = 0; ps < NPASS; ++ps) {
      float kf[EPL];
      if (FP8) {
        const uint32_t w[4] = {kr[ps].x, kr[ps].y, kr[ps].z, kr[ps].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const f32x2 lo = e4m3x2_to_f32x2<false>(w[i]), hi = e4m3x2_to_f32x2<true>(w[i]);
          kf[4 * i] = lo.x; kf[4 * i + 1] = lo.y; kf[4 * i + 2] = hi.x; kf[4 * i + 3] = hi.y;
        }
      } else {
        const uint32_t w[4] = {kr[ps].x, kr[ps].y, kr[ps].z, kr[ps].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) { kf[2 * i] = bf16_lo(w[i]); kf[2 * i + 1] = bf16_hi(w[i]); }
      }
      const bool valid = blk * KV_BLOCK + ps * PPP + prow < ntok;
      vld[ps] = valid;
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float s = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) s = fmaf(qv[h][e], kf[e], s);
#pragma unroll
        for (int off = 1; off < LPP; off <<= 1) s += __shfl_xor(s, off);
        sc[ps][h] = valid ? s : -INFINITY;
      }
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float bm = sc[0][h];
#pragma unroll
      for (int ps = 1; ps < NPASS; ++ps) bm = fmaxf(bm, sc[ps][h]);
#pragma unroll
      for (int off = LPP; off < WAVE; off <<= 1) bm = fmaxf(bm, __shfl_xor(bm, off));
      const float mn = fmaxf(m[h], bm);  // finite: the block's first position is valid
      const float alpha = exp2f(m[h] - mn);
      m[h] = mn;
      l[h] *= alpha;
#pragma unroll
      for (int e = 0; e < EPL; ++e) o[h][e] *= alpha;
#pragma unroll
      for (int ps = 0; ps < NPASS; ++ps) {
        const float pr = exp2f(sc[ps][h] - mn);
        l[h] += pr;
        float vf[EPL];
        const uint32_t w[4] = {vr[ps].x, vr[ps].y, vr[ps].z, vr[ps].w};
        if (FP8) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const f32x2 lo = e4m3x2_to_f32x2<false>(w[i]), hi = e4m3x2_to_f32x2<true>(w[i]);
            vf[4 * i] = lo.x; vf[4 * i + 1] = lo.y; vf[4 * i + 2] = hi.x; vf[4 * i + 3] = hi.y;
          }
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) { vf[2 * i] = bf16_lo(w[i]); vf[2 * i + 1] = bf16_hi(w[i]); }
        }
#pragma unroll
        for (int e = 0; e < EPL; ++e) o[h][e] = fmaf(pr, vld[ps] ? vf[e] : 0.f, o[h][e]);
      }
    }
  }

  // sum l and o over the position rows of the wave (lanes with the same eoff)
#pragma unroll
  for (int h = 0; h < G; ++h) {
#pragma unroll
    for (int off = LPP; off < WAVE; off <<= 1) {
      l[h] += __shfl_xor(l[h], off);
#pragma unroll
      for (int e = 0; e < EPL; ++e) o[h][e] += __shfl_xor(o[h][e], off);
    }
  }

  __shared__ float sm[NW][G], sl[NW][G];
  __shared__ float so[NW][G][DH];
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) { sm[wave][h] = m[h]; sl[wave][h] = l[h]; }
  }
  if (prow == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < EPL; ++e) so[wave][h][eoff + e] = o[h][e];
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < G * DH; idx += NW * WAVE) {
    const int h = idx / DH, e = idx % DH;
    float M = sm[0][h];
#pragma unroll
    for (int w = 1; w < NW; ++w) M = fmaxf(M, sm[w][h]);
    float O = 0.f, L = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const float f = exp2f(sm[w][h] - M);
        O = fmaf(f, so[w][h][e], O);
        L = fmaf(f, sl[w][h], L);
      }
    }
    const int64_t row = ((int64_t)b * p.Hq + c * G + h) * p.n_split + split;
    cst(p.part_o + row * DH + e, O);
    if (e == 0) cst_f2(p.part_ml + row * 2, M, L);
  }

  // arrival: the partial stores of every wave complete before this work group counts
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  __shared__ int last;
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned* cnt = p.cnt + (int64_t)b * p.Hkv + c;
    const unsigned prev = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    last = prev == (unsigned)p.n_split - 1;
    if (last) cst(cnt, 0u);  // ready for the next launch
  }
  __syncthreads();
  if (!last) return;

  // combine the n_split partials of the group's G heads
  __shared__ float cm[G][MAX_SPLIT], cl[G][MAX_SPLIT], cM[G];
  for (int idx = threadIdx.x; idx < G * p.n_split; idx += NW * WAVE) {
    const int h = idx / p.n_split, sp = idx % p.n_split;
    const int64_t row = ((int64_t)b * p.Hq + c * G + h) * p.n_split + sp;
    const uint64_t ml = cld(reinterpret_cast<const uint64_t*>(p.part_ml + row * 2));
    cm[h][sp] = __uint_as_float((uint32_t)ml);
    cl[h][sp] = __uint_as_float((uint32_t)(ml >> 32));
  }
  __syncthreads();
  if (threadIdx.x < G) {
    float M = -INFINITY;
    for (int sp = 0; sp < p.n_split; ++sp) M = fmaxf(M, cm[threadIdx.x][sp]);
    cM[threadIdx.x] = M;
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < G * DH; idx += NW * WAVE) {
    const int h = idx / DH, e = idx % DH;
    const float M = cM[h];
    const int64_t row0 = ((int64_t)b * p.Hq + c * G + h) * p.n_split;
    float out = 0.f;
    if (M != -INFINITY) {
      float O = 0.f, L = 0.f;
#pragma unroll 8
      for (int sp = 0; sp < p.n_split; ++sp) {
        const float f = exp2f(cm[h][sp] - M);
        O = fmaf(f, cld(p.part_o + (row0 + sp) * DH + e), O);
        L = fmaf(f, cl[h][sp], L);
      }
      out = O / L;
    }
    p.o[((int64_t)b * p.Hq + c * G + h) * DH + e] = f32_to_bf16(out);
  }
}

namespace {
template <int DH, bool FP8>
hipError_t attn_go(const AttnParams& p, hipStream_t s) {
  const int g = p.Hq / p.Hkv;
  const dim3 grid(p.n_split, p.Hkv, p.Bp);
  switch (g) {
    case 1: hipLaunchKernelGGL((k_attn_split<DH, FP8, 1>), grid, dim3(256), 0, s, p); break;
    case 2: hipLaunchKernelGGL((k_attn_split<DH, FP8, 2>), grid, dim3(256), 0, s, p); break;
    case 3: hipLaunchKernelGGL((k_attn_split<DH, FP8, 3>), grid, dim3(256), 0, s, p); break;
    case 4: hipLaunchKernelGGL((k_attn_split<DH, FP8, 4>), grid, dim3(256), 0, s, p); break;
    case 5: hipLaunchKernelGGL((k_attn_split<DH, FP8, 5>), grid, dim3(256), 0, s, p); break;
    case 6: hipLaunchKernelGGL((k_attn_split<DH, FP8, 6>), grid, dim3(256), 0, s, p); break;
    case 7: hipLaunchKernelGGL((k_attn_split<DH, FP8, 7>), grid, dim3(256), 0, s, p); break;
    case 8: hipLaunchKernelGGL((k_attn_split<DH, FP8, 8>), grid, dim3(256), 0, s, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}
}  // namespace

hipError_t launch_attention(const AttnParams& p, bool kv_fp8, hipStream_t s) {
  if (p.dh == 64) return kv_fp8 ? attn_go<64, true>(p, s) : attn_go<64, false>(p, s);
  if (p.dh == 128) return kv_fp8 ? attn_go<128, true>(p, s) : attn_go<128, false>(p, s);
  return hipErrorInvalidValue;
}

}  // namespace dec
