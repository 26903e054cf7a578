// Split-K paged GQA decode attention: the work of one work group (shared by the
// attention kernel and the fused attention + O-projection kernel).
#pragma once

#include "common.h"
#include "kernels.h"

namespace dec {


constexpr int MAX_SPLIT = 64;  // splits per (sequence, kv head); the host keeps n_split within it
#ifndef DEC_ATTN_WAVES
#define DEC_ATTN_WAVES 8
#endif
constexpr int ATTN_WAVES = DEC_ATTN_WAVES;  // waves per work group

// K and V of one block of one kv head for this lane: NPASS 16-byte loads each
// (a lane holds 8 cache elements of a row: 16 bytes of bf16 or 8 bytes of E4M3, in .x .y)
template <int DH, bool FP8, int NPASS, int PPP>
__device__ __forceinline__ void attn_load(const uint8_t* pool, int64_t kbase, int64_t vbase, int prow, int eoff,
                                          u32x4 (&kr)[NPASS], u32x4 (&vr)[NPASS]) {
  constexpr int ESZ = FP8 ? 1 : 2;
#pragma unroll
  for (int ps = 0; ps < NPASS; ++ps) {
    const int64_t off = (int64_t)(ps * PPP + prow) * DH + eoff;
    if (FP8) {
      const u32x2 k2 = gld(reinterpret_cast<const u32x2*>(pool + (kbase + off)));
      const u32x2 v2 = gld(reinterpret_cast<const u32x2*>(pool + (vbase + off)));
      kr[ps] = u32x4{k2.x, k2.y, 0u, 0u};
      vr[ps] = u32x4{v2.x, v2.y, 0u, 0u};
    } else {
      kr[ps] = gld16(pool + (kbase + off) * ESZ);
      vr[ps] = gld16(pool + (vbase + off) * ESZ);
    }
  }
}

// the 8 cache elements a lane holds, as fp32
template <bool FP8>
__device__ __forceinline__ void attn_widen(const u32x4& r, float (&f)[8]) {
  if (FP8) {
    const f32x2 a = e4m3x2_to_f32x2<false>(r.x), b = e4m3x2_to_f32x2<true>(r.x);
    const f32x2 c = e4m3x2_to_f32x2<false>(r.y), d = e4m3x2_to_f32x2<true>(r.y);
    f[0] = a.x; f[1] = a.y; f[2] = b.x; f[3] = b.y; f[4] = c.x; f[5] = c.y; f[6] = d.x; f[7] = d.y;
  } else {
    const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) { f[2 * i] = bf16_lo(w[i]); f[2 * i + 1] = bf16_hi(w[i]); }
  }
}

// online-softmax update of the G heads' (m, l, o) with one block (positions blk*16 ..)
template <int DH, bool FP8, int G, int NPASS, int PPP, int LPP, int EPL>
__device__ __forceinline__ void attn_update(int blk, int ntok, int prow, const float (&qv)[G][EPL],
                                            const u32x4 (&kr)[NPASS], const u32x4 (&vr)[NPASS], float (&m)[G],
                                            float (&l)[G], float (&o)[G][EPL]) {
  float sc[NPASS][G];
  bool vld[NPASS];  // slots past the last position may hold anything (even NaN): mask them
#pragma unroll
  for (int ps = 0; ps < NPASS; ++ps) {
    float kf[EPL];
    attn_widen<FP8>(kr[ps], kf);
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
      attn_widen<FP8>(vr[ps], vf);
#pragma unroll
      for (int e = 0; e < EPL; ++e) o[h][e] = fmaf(pr, vld[ps] ? vf[e] : 0.f, o[h][e]);
    }
  }
}

// One work group computes one (split, kv head c, sequence b) unit of attention.  With
// one split it writes o; otherwise it writes its partial, and the last split of the
// group to arrive combines.  o is written device-coherently.
template <int DH, bool FP8, int G, int NW>
__device__ __forceinline__ void attn_unit(const AttnParams& p, int split, int c, int b) {
  constexpr int EPL = 8;             // cache elements per lane per row
  constexpr int LPP = DH / EPL;      // lanes per position row
  constexpr int PPP = WAVE / LPP;    // positions per pass
  constexpr int NPASS = KV_BLOCK / PPP;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / WAVE), lane = threadIdx.x % WAVE;
  const int prow = lane / LPP, eoff = (lane % LPP) * EPL;

  const int pos = gld(p.seq_lens + b);
  const int ntok = pos + 1;  // 0 for a padded row
  const int nblk = pos >= 0 ? pos / KV_BLOCK + 1 : 0;
  const int per = (nblk + p.n_split - 1) / p.n_split;
  const int blk0 = split * per;
  const int blk1 = min(nblk, blk0 + per);
  // this wave's blocks: blk0 + wave + i NW, i < nb; lane i holds the physical id of the i-th
  const int nb = blk0 + wave < blk1 ? (blk1 - blk0 - wave + NW - 1) / NW : 0;
  const int my_blk = blk0 + wave + lane * NW;
  const int my_phys = lane < nb ? gld(p.bt + (int64_t)b * p.bps + my_blk) : 0;

  const float qscale = 1.4426950408889634f / sqrtf((float)DH);  // log2(e) / sqrt(dh)
  float qv[G][EPL];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float* qh = p.q + ((int64_t)b * p.Hq + c * G + h) * DH + eoff;
#pragma unroll
    for (int e = 0; e < EPL; e += 4) {
      const f32x4 t = gld(reinterpret_cast<const f32x4*>(qh + e));
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
  auto bases = [&](int i, int64_t& kb, int64_t& vb) {
    const int phys = __shfl(my_phys, i);
    kb = kv_offset(p.layer, 0, phys, c, 0, 0, p.num_blocks, p.Hkv, DH);
    vb = kv_offset(p.layer, 1, phys, c, 0, 0, p.num_blocks, p.Hkv, DH);
  };
  if (nb > 0 && G > 6) {
    // wide groups: the per-head state leaves no room for a second block in registers
    u32x4 ka[NPASS], va[NPASS];
    int64_t kbase, vbase;
    for (int i = 0; i < nb; ++i) {
      bases(i, kbase, vbase);
      attn_load<DH, FP8, NPASS, PPP>(pool, kbase, vbase, prow, eoff, ka, va);
      attn_update<DH, FP8, G, NPASS, PPP, LPP, EPL>(blk0 + wave + i * NW, ntok, prow, qv, ka, va, m, l, o);
    }
  } else if (nb > 0) {
    // two blocks in flight: the next block's loads are issued before this one's math
    u32x4 ka[NPASS], va[NPASS], kb2[NPASS], vb2[NPASS];
    int64_t kbase, vbase;
    bases(0, kbase, vbase);
    attn_load<DH, FP8, NPASS, PPP>(pool, kbase, vbase, prow, eoff, ka, va);
    for (int i = 0; i < nb; i += 2) {
      bases(min(i + 1, nb - 1), kbase, vbase);
      attn_load<DH, FP8, NPASS, PPP>(pool, kbase, vbase, prow, eoff, kb2, vb2);
      attn_update<DH, FP8, G, NPASS, PPP, LPP, EPL>(blk0 + wave + i * NW, ntok, prow, qv, ka, va, m, l, o);
      if (i + 1 >= nb) break;
      bases(min(i + 2, nb - 1), kbase, vbase);
      attn_load<DH, FP8, NPASS, PPP>(pool, kbase, vbase, prow, eoff, ka, va);
      attn_update<DH, FP8, G, NPASS, PPP, LPP, EPL>(blk0 + wave + (i + 1) * NW, ntok, prow, qv, kb2, vb2, m, l, o);
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
  const bool single = p.n_split == 1;
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
    if (single) {
      // the whole context in this work group: o directly
      cst(p.o + ((int64_t)b * p.Hq + c * G + h) * DH + e, f32_to_bf16(M != -INFINITY ? O / L : 0.f));
      continue;
    }
    const int64_t row = ((int64_t)b * p.Hq + c * G + h) * p.n_split + split;
    cst(p.part_o + row * DH + e, O);
    if (e == 0) cst_f2(p.part_ml + row * 2, M, L);
  }
  if (single) return;

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
    cst(p.o + ((int64_t)b * p.Hq + c * G + h) * DH + e, f32_to_bf16(out));
  }
}

}  // namespace dec
