// Split-K paged GQA decode attention: the work of one work group.
#pragma once

#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace dec {


// splits whose partial outputs the combine loads together with every split's max and
// sum (one round trip for up to this many splits)
constexpr int ATTN_COMBINE_PRE = 16;

// LDS of one attention work group
template <int DH, int G, int NW>
struct AttnSmem {
  float sm[NW][G], sl[NW][G];  // per-wave running max and sum
  float so[NW][G][DH];         // per-wave output
  float cm[G][ATTN_MAX_SPLIT], cl[G][ATTN_MAX_SPLIT], cM[G];  // the combine's partial max and sum
  int last;
};

// K and V of one block of one kv head for this lane: NPASS 16-byte loads each
// (a lane holds 8 cache elements of a row: 16 bytes of bf16 or 8 bytes of E4M3, in .x .y).
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

// online-softmax update of the G heads' (m, l, o) with one block (positions blk*16 ..);
// qf(h, e): element e of the lane's 8 scaled query elements of head h
template <int DH, bool FP8, int G, int NPASS, int PPP, int LPP, int EPL, typename QF>
__device__ __forceinline__ void attn_update(int blk, int ntok, int prow, const QF& qf,
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
      for (int e = 0; e < EPL; ++e) s = fmaf(qf(h, e), kf[e], s);
      s = group_sum<LPP>(s);  // over the LPP lanes of the position row
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
    const float alpha = exp2_hw(m[h] - mn);
    m[h] = mn;
    l[h] *= alpha;
#pragma unroll
    for (int e = 0; e < EPL; ++e) o[h][e] *= alpha;
#pragma unroll
    for (int ps = 0; ps < NPASS; ++ps) {
      sc[ps][h] = exp2_hw(sc[ps][h] - mn);  // the probability, in place of the score
      l[h] += sc[ps][h];
    }
  }
  // each V row is widened once and serves every head (one row's elements live at a time)
#pragma unroll
  for (int ps = 0; ps < NPASS; ++ps) {
    float vf[EPL];
    attn_widen<FP8>(vr[ps], vf);
#pragma unroll
    for (int e = 0; e < EPL; ++e) vf[e] = vld[ps] ? vf[e] : 0.f;
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < EPL; ++e) o[h][e] = fmaf(sc[ps][h], vf[e], o[h][e]);
  }
}

// KV blocks in flight per wave in the MFMA form (three or four measured slower at batch
// 32 and 64: the registers they take)
constexpr int ATTN_MFMA_DEPTH = 2;

// Tiles of one wave for the MFMA form: K then V, 16 position rows of DH bf16 each, a row
// padded by 16 bytes
template <int DH>
constexpr int attn_vt_row() { return DH * 2 + 16; }
template <int DH>
constexpr int attn_wave_lds() { return 2 * 16 * attn_vt_row<DH>(); }

// The MFMA form of one wave's blocks (batches where attention's arithmetic, not its
// memory latency, sets the pace: the scores and the P V products on the matrix cores).
// Per block of 16 positions:
//   S^T = K q^T     v_mfma_f32_16x16x32_bf16, A = K rows (the 16 positions, from the
//                   wave's K tile), B = the group's queries as 16 columns (heads >= G
//                   are zero); lane l ends with
//                   S[position 4 (l / 16) + j][head l % 16], j < 4;
//   online softmax per head (column): the block's max over the lane's 4 positions and the
//                   four lane groups; running max, this lane's share of the sum, and the
//                   output rescaled in the lane's registers;
//   O^T += V^T P^T  v_mfma_f32_16x16x16_bf16, A = V^T (16 dims x 16 positions, from the
//                   wave's LDS tile), B = the probabilities exactly as the lane holds them.
// q and P enter as bf16 high and low parts (two products each), so the scores and the
// weighted sum keep about 16 bits of their fp32 operands.  Writes the wave's running max,
// sum and output of each head h < G to sm, sl and so.
template <int DH, bool FP8, int G, int NW>
__device__ __forceinline__ void attn_wave_mfma(const AttnParams& p, int b, int c, int lane, int nb, int bfirst,
                                               int ntok, int my_phys, uint8_t* vt, float* sm, float* sl,
                                               float (*so)[DH]) {
  constexpr int NS = DH / 32;   // score k-steps
  constexpr int NC = DH / 16;   // output dim chunks
  constexpr int TR = attn_vt_row<DH>();
  typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
  const int m = lane % 16, g = lane / 16;
  const bool hv = m < G;
  const uint8_t* pool = static_cast<const uint8_t*>(p.pool);

  // q^T operands of head m: elements s 32 + 8 g + [0, 8), scaled, as bf16 high + low
  const float qscale = 1.4426950408889634f / sqrtf((float)DH);  // log2(e) / sqrt(dh)
  bf16x8 qh[NS], ql[NS];
  {
    const float* qp = p.q + ((int64_t)b * p.Hq + c * G + (hv ? m : 0)) * DH;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const f32x4 a0 = gld(reinterpret_cast<const f32x4*>(qp + s * 32 + g * 8));
      const f32x4 a1 = gld(reinterpret_cast<const f32x4*>(qp + s * 32 + g * 8 + 4));
      const float x[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float v = hv ? x[e] * qscale : 0.f;
        qh[s][e] = (__bf16)v;  // v_cvt_pk_bf16_f32: round to nearest even
        ql[s][e] = (__bf16)(v - (float)qh[s][e]);
      }
    }
  }

  // K and V of a block are read row-contiguously: load instruction s covers rows RPI s ..
  // RPI s + RPI - 1 whole (512 elements, lane l the 8 at element 8 l), which the memory
  // system serves in full lines; the tiles in LDS then give each lane its MFMA operands.
  // A lane holds 8 elements per instruction: bf16 (16 bytes) or E4M3 (8 bytes).
  constexpr int RPI = 512 / DH;  // rows per load instruction
  const int lrow = lane / (DH / 8), lcol = (lane % (DH / 8)) * 8;
  typedef u32x4 KVReg[2][NS];
  auto load = [&](int i, KVReg& r) {
    const int phys = __shfl(my_phys, i);
    const int64_t kb = kv_offset(p.layer, 0, phys, c, 0, 0, p.num_blocks, p.Hkv, DH);
    const int64_t vb = kv_offset(p.layer, 1, phys, c, 0, 0, p.num_blocks, p.Hkv, DH);
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int e = (s * RPI + lrow) * DH + lcol;
      if (FP8) {
        const u32x2 k2 = gld(reinterpret_cast<const u32x2*>(pool + kb + e));
        const u32x2 v2 = gld(reinterpret_cast<const u32x2*>(pool + vb + e));
        r[0][s] = u32x4{k2.x, k2.y, 0u, 0u};
        r[1][s] = u32x4{v2.x, v2.y, 0u, 0u};
      } else {
        r[0][s] = gld16(pool + (kb + e) * 2);
        r[1][s] = gld16(pool + (vb + e) * 2);
      }
    }
  };
  auto as_bf16x8 = [&](const u32x4& w) -> bf16x8 {
    if (FP8) {
      const bf16x2 a = e4m3x2_to_bf16x2<false>(w.x), bb = e4m3x2_to_bf16x2<true>(w.x);
      const bf16x2 cc = e4m3x2_to_bf16x2<false>(w.y), d = e4m3x2_to_bf16x2<true>(w.y);
      return bf16x8{a.x, a.y, bb.x, bb.y, cc.x, cc.y, d.x, d.y};
    }
    return __builtin_bit_cast(bf16x8, w);
  };

  float mrun = -INFINITY, lrun = 0.f;  // head m; lrun: this lane's positions only
  f32x4 o[NC];
#pragma unroll
  for (int t = 0; t < NC; ++t) o[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  uint8_t* kt = vt + 16 * TR;  // the wave's K tile
  auto block = [&](int i, const KVReg& r) {
    const int pos0 = (bfirst + i * NW) * KV_BLOCK;
    // the previous block's reads of the tiles come before these writes (LDS serves one
    // wave's accesses in order; the wave barrier keeps the compiler from reordering them)
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int row = s * RPI + lrow;
      // K rows past the last position only feed scores that are masked below; V rows
      // there are zeroed (those slots may hold anything, even NaN, which a zero
      // probability would not cancel in the product)
      *reinterpret_cast<u32x4*>(kt + row * TR + lcol * 2) = __builtin_bit_cast(u32x4, as_bf16x8(r[0][s]));
      *reinterpret_cast<u32x4*>(vt + row * TR + lcol * 2) =
          pos0 + row < ntok ? __builtin_bit_cast(u32x4, as_bf16x8(r[1][s])) : u32x4{0u, 0u, 0u, 0u};
    }
    // ... and these writes before this block's transposed reads below
    __builtin_amdgcn_wave_barrier();
    f32x4 sa = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      // A operand: K row m, elements 32 s + 8 g .. + 7
      const bf16x8 kv = *reinterpret_cast<const bf16x8*>(kt + m * TR + (s * 32 + g * 8) * 2);
      sa = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kv, qh[s], sa, 0, 0, 0);
      sa = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kv, ql[s], sa, 0, 0, 0);
    }
    float sc[4], bm = -INFINITY;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      sc[j] = pos0 + 4 * g + j < ntok ? sa[j] : -INFINITY;
      bm = fmaxf(bm, sc[j]);
    }
    bm = fmaxf(bm, __shfl_xor(bm, 16));
    bm = fmaxf(bm, __shfl_xor(bm, 32));
    const float mn = fmaxf(mrun, bm);  // finite: the block's first position is valid
    const float alpha = exp2_hw(mrun - mn);
    mrun = mn;
    bf16x4 ph, pl;
    float ps = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float pj = exp2_hw(sc[j] - mn);
      ps += pj;
      ph[j] = (__bf16)pj;  // the hardware conversion (round to nearest even), two per instruction
      pl[j] = (__bf16)(pj - (float)ph[j]);
    }
    lrun = lrun * alpha + ps;
    // the output is rescaled only when some head's running max rose in this block (once
    // the context's largest scores have been seen it rarely does): multiplying by exactly
    // 1 would change no bit, and the wave-uniform branch skips NC x 4 products
    if (__ballot(alpha != 1.f) != 0) {
#pragma unroll
      for (int t = 0; t < NC; ++t) o[t] *= alpha;
    }
#pragma unroll
    for (int t = 0; t < NC; ++t) {
      // V^T[dim 16 t + m][positions 4 g .. 4 g + 3] from the tile by one transposing LDS
      // read (ds_read_b64_tr_b16: in each 16-lane group, lane i receives element i % 4
      // of the 4 elements that lane 4 j + i / 4 points at, j = 0..3): lane 16 g + i
      // points at position row 4 g + i / 4, dims 16 t + 4 (i % 4) .. + 3
      const uint8_t* src = vt + (4 * g + m / 4) * TR + (16 * t + 4 * (m % 4)) * 2;
      const bf16x4 va = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((__attribute__((address_space(3))) bf16x4*)src);
      o[t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, ph, o[t], 0, 0, 0);
      o[t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, pl, o[t], 0, 0, 0);
    }
  };

  // MFA_DEPTH blocks in flight: block i + D is loaded into the registers block i leaves
  constexpr int D = ATTN_MFMA_DEPTH;
  if (nb > 0) {
    KVReg r[D];
#pragma unroll
    for (int j = 0; j < D; ++j)
      if (j < nb) load(j, r[j]);
    for (int i = 0; i < nb; i += D) {
#pragma unroll
      for (int j = 0; j < D; ++j) {
        if (i + j < nb) {
          block(i + j, r[j]);
          if (i + j + D < nb) load(i + j + D, r[j]);
        }
      }
    }
  }
  // the sum over the four lane groups' positions
  lrun += __shfl_xor(lrun, 16);
  lrun += __shfl_xor(lrun, 32);
  if (hv) {
    // o[t][j] = O[head m][dim 16 t + 4 g + j]
#pragma unroll
    for (int t = 0; t < NC; ++t)
#pragma unroll
      for (int j = 0; j < 4; ++j) so[m][16 * t + 4 * g + j] = o[t][j];
    if (g == 0) {
      sm[m] = mrun;
      sl[m] = lrun;
    }
  }
}

// One work group computes one (split, kv head c, sequence b) unit of attention.  With
// one split it writes o; otherwise it writes its partial, and the last split of the
// group to arrive combines.  o is written device-coherently.  Returns, in every thread,
// whether this work group wrote the group's o.
// MF: the wave's blocks in the MFMA form (attn_wave_mfma), with the wave's V and K tiles
// at vtile + wave attn_wave_lds<DH>() bytes of LDS.
// An attention output element as stored: bf16, with the NaN pattern that marks an
// unwritten element in the fused attention + O launch replaced by another NaN
__device__ __forceinline__ uint16_t o_bits(float v) {
  const uint16_t h = f32_to_bf16(v);
  return h == ATTN_O_PENDING ? (uint16_t)0xFFBFu : h;
}

template <int DH, bool FP8, int G, int NW, bool MF = false>
__device__ __forceinline__ bool attn_unit(const AttnParams& p, int split, int c, int b, AttnSmem<DH, G, NW>& S,
                                          uint8_t* vtile = nullptr) {
  constexpr int EPL = 8;             // cache elements per lane per row
  constexpr int LPP = DH / EPL;      // lanes per position row
  constexpr int PPP = WAVE / LPP;    // positions per pass
  constexpr int NPASS = KV_BLOCK / PPP;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / WAVE), lane = threadIdx.x % WAVE;
  const int prow = lane / LPP, eoff = (lane % LPP) * EPL;

  // The splits divide the longest context the block table holds (bps blocks), so that a
  // wave's block ids are fetched together with the sequence length rather than after it.
  const int per = (p.bps + p.n_split - 1) / p.n_split;
  const int blk0 = split * per;
  // lane i holds the physical id of the wave's i-th block, blk0 + wave + i NW (read for
  // every block the table holds; used for the i < nb that the context reaches)
  const int my_blk = blk0 + wave + lane * NW;
  // positions and block ids are clamped into the table and the pool, so that no
  // metadata, whatever its source, makes a read leave them
  const int pos = min(gld(p.seq_lens + b), p.bps * KV_BLOCK - 1);
  const int my_phys = my_blk < p.bps ? min(max(gld(p.bt + (int64_t)b * p.bps + my_blk), 0), p.num_blocks - 1) : 0;
  const int ntok = pos + 1;  // 0 for a padded row
  const int nblk = pos >= 0 ? pos / KV_BLOCK + 1 : 0;
  const int blk1 = min(nblk, blk0 + per);
  const int nb = blk0 + wave < blk1 ? (blk1 - blk0 - wave + NW - 1) / NW : 0;

  const uint8_t* pool = static_cast<const uint8_t*>(p.pool);
  // loads of the wave's i-th block
  auto load_blk = [&](int i, u32x4 (&kr)[NPASS], u32x4 (&vr)[NPASS]) {
    const int phys = __shfl(my_phys, i);
    const int64_t kb = kv_offset(p.layer, 0, phys, c, 0, 0, p.num_blocks, p.Hkv, DH);
    const int64_t vb = kv_offset(p.layer, 1, phys, c, 0, 0, p.num_blocks, p.Hkv, DH);
    attn_load<DH, FP8, NPASS, PPP>(pool, kb, vb, prow, eoff, kr, vr);
  };
  if constexpr (MF) {
    attn_wave_mfma<DH, FP8, G, NW>(p, b, c, lane, nb, blk0 + wave, ntok, my_phys,
                                   vtile + wave * attn_wave_lds<DH>(), S.sm[wave], S.sl[wave], S.so[wave]);
  } else {
    const float qscale = 1.4426950408889634f / sqrtf((float)DH);  // log2(e) / sqrt(dh)
    float qv[G][EPL];  // the lane's 8 elements of each head's query, scaled
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
    auto qf = [&](int h, int e) -> float { return qv[h][e]; };

    float m[G], l[G], o[G][EPL];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      m[h] = -INFINITY;
      l[h] = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) o[h][e] = 0.f;
    }
    u32x4 ka[NPASS], va[NPASS];
    if (nb > 0 && G > 6) {
      // wide groups: no room for a second block in registers
      for (int i = 0; i < nb; ++i) {
        load_blk(i, ka, va);
        attn_update<DH, FP8, G, NPASS, PPP, LPP, EPL>(blk0 + wave + i * NW, ntok, prow, qf, ka, va, m, l, o);
      }
    } else if (nb > 0) {
      // two blocks in flight: the next block's loads are issued before this one's math
      // (four in flight measured slower: the registers they take)
      u32x4 kb2[NPASS], vb2[NPASS];
      load_blk(0, ka, va);
      for (int i = 0; i < nb; i += 2) {
        load_blk(min(i + 1, nb - 1), kb2, vb2);
        attn_update<DH, FP8, G, NPASS, PPP, LPP, EPL>(blk0 + wave + i * NW, ntok, prow, qf, ka, va, m, l, o);
        if (i + 1 >= nb) break;
        load_blk(min(i + 2, nb - 1), ka, va);
        attn_update<DH, FP8, G, NPASS, PPP, LPP, EPL>(blk0 + wave + (i + 1) * NW, ntok, prow, qf, kb2, vb2, m, l,
                                                      o);
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
    if (lane == 0) {
#pragma unroll
      for (int h = 0; h < G; ++h) { S.sm[wave][h] = m[h]; S.sl[wave][h] = l[h]; }
    }
    if (prow == 0) {
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < EPL; ++e) S.so[wave][h][eoff + e] = o[h][e];
    }
  }
  __syncthreads();
  auto& sm = S.sm;
  auto& sl = S.sl;
  auto& so = S.so;
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
        const float f = exp2_hw(sm[w][h] - M);
        O = fmaf(f, so[w][h][e], O);
        L = fmaf(f, sl[w][h], L);
      }
    }
    if (single) {
      // the whole context in this work group: o directly
      cst(p.o + ((int64_t)b * p.Hq + c * G + h) * DH + e, o_bits(M != -INFINITY ? O / L : 0.f));
      continue;
    }
    const int64_t row = ((int64_t)b * p.Hq + c * G + h) * p.n_split + split;
    cst(p.part_o + row * DH + e, O);
    if (e == 0) cst_f2(p.part_ml + row * 2, M, L);
  }
  if (single) return true;

  // arrival: the partial stores of every wave complete before this work group counts
  if (!arrive_after_stores(p.cnt + (int64_t)b * p.Hkv + c, (unsigned)p.n_split, &S.last)) return false;

  // combine the n_split partials of the group's G heads: thread -> (head h, element e).
  // One round trip brings the max and sum of every (head, split) pair (into LDS) together
  // with each thread's partial outputs of the first ATTN_COMBINE_PRE splits (registers);
  // the partial outputs of further splits follow once the maximum is known.
  constexpr int PRE = ATTN_COMBINE_PRE;
  constexpr int NI = (G * DH + NW * WAVE - 1) / (NW * WAVE);  // outputs per thread
  auto& cm = S.cm;
  auto& cl = S.cl;
  auto& cM = S.cM;
  const int ns = p.n_split;
  const int64_t row_g = ((int64_t)b * p.Hq + c * G) * ns;  // (head c G, split 0)
  float po[NI][PRE];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int idx = min((int)threadIdx.x + i * NW * WAVE, G * DH - 1);  // past the end: a re-read
    const int64_t row0 = row_g + (int64_t)(idx / DH) * ns;
#pragma unroll
    for (int sp = 0; sp < PRE; ++sp) po[i][sp] = cld(p.part_o + (row0 + min(sp, ns - 1)) * DH + idx % DH);
  }
  for (int t = threadIdx.x; t < G * ns; t += NW * WAVE) {
    const uint64_t ml = cld(reinterpret_cast<const uint64_t*>(p.part_ml + (row_g + t) * 2));
    cm[t / ns][t % ns] = __uint_as_float((uint32_t)ml);
    cl[t / ns][t % ns] = __uint_as_float((uint32_t)(ml >> 32));
  }
  __syncthreads();
  if (threadIdx.x < G) {
    float M = -INFINITY;
    for (int sp = 0; sp < ns; ++sp) M = fmaxf(M, cm[threadIdx.x][sp]);
    cM[threadIdx.x] = M;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int idx = threadIdx.x + i * NW * WAVE;
    if (idx >= G * DH) break;
    const int h = idx / DH, e = idx % DH;
    const float M = cM[h];
    const int64_t row0 = row_g + (int64_t)h * ns;
    float out = 0.f;
    if (M != -INFINITY) {
      float O = 0.f, L = 0.f;
#pragma unroll
      for (int sp = 0; sp < PRE; ++sp) {
        if (sp < ns) {
          const float f = exp2_hw(cm[h][sp] - M);
          O = fmaf(f, po[i][sp], O);
          L = fmaf(f, cl[h][sp], L);
        }
      }
      for (int sp = PRE; sp < ns; ++sp) {
        const float f = exp2_hw(cm[h][sp] - M);
        O = fmaf(f, cld(p.part_o + (row0 + sp) * DH + e), O);
        L = fmaf(f, cl[h][sp], L);
      }
      out = O / L;
    }
    cst(p.o + ((int64_t)b * p.Hq + c * G + h) * DH + e, o_bits(out));
  }
  return true;
}

}  // namespace dec
