// Persistent decode step for small batches (padded batch <= 8).
//
// At batch 1..8 a decode step is a chain of short weight-streaming products
// separated by tiny elementwise and attention work; per-kernel launch overhead and
// the ramp-up / drain of every short kernel then cost as much as the bytes ("A
// decode step is hundreds of tiny GPU programs ..." -- "Kernels, Fusion & CUDA
// Graphs", opening section; the launch tax N tau of "CUDA graphs & kernel fusion",
// Direct answer).  This kernel runs the whole step -- embedding, every layer, the
// LM head -- as one launch: one work group of 8 waves per CU, all resident, with
// grid-wide barriers between the phases that depend on each other:
//
//   embed | per layer: [RMSNorm -> LDS, QKV + RoPE + KV write] | [attention, last
//   split of each head combines] | [O + residual] | [RMSNorm -> LDS, gate+up +
//   SiLU x mul] | [down + residual] | [RMSNorm -> LDS, LM head]
//
// Weight streaming never waits on a barrier: every wave keeps two chunks of its
// weight rows in flight (double-buffered registers), and when its share of a phase
// runs out the chunks it loads are the first two of its share of the *next*
// matrix, which does not depend on the barrier.  HBM stays busy while the grid
// synchronises, normalises and attends.  The norm is recomputed by every work
// group straight into LDS (the fp32 residual stream is L2-resident), so the
// normalised activations never go through HBM (kernel-fusion architecture study,
// section 8: intermediates round-tripping through HBM).
//
// Barrier waits are bounded by a timer: a wait that exceeds the limit sets an
// error word (read by the host at the next call) and lets the kernel finish.

#include "common.h"
#include "epilogue.h"
#include "kernels.h"

namespace dec {

constexpr int PW = 8;           // waves per work group
constexpr int PT = PW * WAVE;   // threads per work group
#ifndef DEC_PU
#define DEC_PU 8
#endif
constexpr int PU = DEC_PU;      // 16-byte vectors per row per lane per chunk
constexpr int MAX_ROUNDS = 8;   // items per wave when a phase splits K over waves

// the wave's index in its work group, as a wave-uniform (scalar) value
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x / WAVE); }

__device__ __forceinline__ DevMat load_mat(const DevMat* m) {
  DevMat r;
  r.w = gld(&m->w);
  r.scale = gld(&m->scale);
  return r;
}

// ---------------------------------------------------------------- grid barrier

__device__ __forceinline__ bool step_failed(const StepParams& p) {
  return __hip_atomic_load(p.err_dev, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u;
}

// Grid-wide barrier.  Every wave must have waited for its own device-coherent stores
// before calling (wait_stores); data is exchanged only through such stores and loads,
// so the barrier itself needs no cache maintenance: it orders, it does not flush.
__device__ void grid_sync(const StepParams& p) {
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned* count = p.bar;
    unsigned* gen = p.bar + 1;
    const unsigned g0 = __hip_atomic_load(gen, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    const unsigned arrived = __hip_atomic_fetch_add(count, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (arrived == gridDim.x - 1) {
      __hip_atomic_store(count, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __builtin_amdgcn_s_waitcnt(0);  // the reset lands before the release of the waiters
      __hip_atomic_fetch_add(gen, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else {
      const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
      while (__hip_atomic_load(gen, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == g0) {
        __builtin_amdgcn_s_sleep(1);
        if (__builtin_amdgcn_s_memrealtime() - t0 > p.timeout_ticks || step_failed(p)) {
          __hip_atomic_store(p.err_dev, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          __hip_atomic_store(p.err_host, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
          break;
        }
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
  }
  __syncthreads();
}

// Wait until this wave's stores have completed while its last `n_loads` loads (the next
// phase's prefetched weights, issued after the stores) stay in flight.  Vector memory
// operations retire in issue order on this architecture, so a count of outstanding
// operations <= n_loads means everything issued before those loads is done.
__device__ __forceinline__ void wait_stores(int n_loads) {
  // s_waitcnt immediates: vmcnt = n (bits 3:0 and 15:14), expcnt and lgkmcnt left open
  if (n_loads >= 32) __builtin_amdgcn_s_waitcnt(0x8F70);        // vmcnt(32)
  else if (n_loads >= 16) __builtin_amdgcn_s_waitcnt(0x4F70);   // vmcnt(16)
  else if (n_loads >= 8) __builtin_amdgcn_s_waitcnt(0x0F78);    // vmcnt(8)
  else __builtin_amdgcn_s_waitcnt(0x0F70);                      // vmcnt(0)
}

// ---------------------------------------------------------------- activations into LDS

// xs[b][i] = bf16(h[b][i] * g[i] / sqrt(mean_j h[b][j]^2 + eps)) for b < BT
template <int BT>
__device__ void norm_to_lds(const float* h, const float* gain, int d, float eps, uint16_t* xs, float* red) {
  const int tid = threadIdx.x, lane = tid % WAVE, w = tid / WAVE;
  float ss[BT];
#pragma unroll
  for (int b = 0; b < BT; ++b) ss[b] = 0.f;
  for (int i = tid * 4; i < d; i += PT * 4) {
#pragma unroll
    for (int b = 0; b < BT; ++b) {
      const f32x4 v = cld_f4(h + (int64_t)b * d + i);
      ss[b] += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
    }
  }
#pragma unroll
  for (int b = 0; b < BT; ++b) {
    const float s = wave_sum(ss[b]);
    if (lane == 0) red[w * BT + b] = s;
  }
  __syncthreads();
  float r[BT];
#pragma unroll
  for (int b = 0; b < BT; ++b) {
    float s = 0.f;
#pragma unroll
    for (int ww = 0; ww < PW; ++ww) s += red[ww * BT + b];
    r[b] = 1.0f / sqrtf(s / (float)d + eps);
  }
  for (int i = tid * 4; i < d; i += PT * 4) {
    const f32x4 g = gld(reinterpret_cast<const f32x4*>(gain + i));
#pragma unroll
    for (int b = 0; b < BT; ++b) {
      const f32x4 v = cld_f4(h + (int64_t)b * d + i);
      const uint32_t lo = (uint32_t)f32_to_bf16(v.x * r[b] * g.x) | ((uint32_t)f32_to_bf16(v.y * r[b] * g.y) << 16);
      const uint32_t hi = (uint32_t)f32_to_bf16(v.z * r[b] * g.z) | ((uint32_t)f32_to_bf16(v.w * r[b] * g.w) << 16);
      *reinterpret_cast<u32x2*>(xs + b * d + i) = u32x2{lo, hi};
    }
  }
  __syncthreads();
}

// xs[b][0..K) = x[b][0..K) (bf16 copy into LDS)
template <int BT>
__device__ void copy_to_lds(const uint16_t* x, int ldx, int K, uint16_t* xs) {
  for (int i = threadIdx.x * 8; i < K; i += PT * 8) {
#pragma unroll
    for (int b = 0; b < BT; ++b)
      *reinterpret_cast<u32x4*>(xs + b * K + i) = cld16(x + (int64_t)b * ldx + i);
  }
  __syncthreads();
}

// ---------------------------------------------------------------- one wave's share of a product

struct PWork {
  const u32x4* W;   // weight rows, KV 16-byte vectors each
  int KV;
  int rowmul;       // first row of item i: i * rowmul
  int rowoff;       // second row: first + rowoff
  int i0, i1, istep;  // items of this wave: i0, i0 + istep, ... < i1
  int kb, ke;         // this wave's vector range of each row
  int nch;            // chunks per item
  int n;              // units (item, chunk) of this wave
  int part, S;
};

__device__ __forceinline__ PWork make_work(const void* W, int K, bool fp8, int items, int rowmul, int rowoff, int S) {
  PWork k;
  const int epv = fp8 ? 16 : 8;
  k.W = static_cast<const u32x4*>(W);
  k.KV = K / epv;
  k.rowmul = rowmul;
  k.rowoff = rowoff;
  const int G = gridDim.x, g = blockIdx.x, w = wave_id();
  const int gi0 = (int)((int64_t)items * g / G), gi1 = (int)((int64_t)items * (g + 1) / G);
  const int slots = PW / S;
  k.S = S;
  k.part = w % S;
  k.i0 = gi0 + w / S;
  k.istep = slots;
  k.i1 = gi1;
  k.kb = (int)((int64_t)k.KV * k.part / S);
  k.ke = (int)((int64_t)k.KV * (k.part + 1) / S);
  k.nch = (k.ke - k.kb + WAVE * PU - 1) / (WAVE * PU);
  const int nit = k.i0 < k.i1 ? (k.i1 - k.i0 + k.istep - 1) / k.istep : 0;
  k.n = nit * k.nch;
  return k;
}

struct Chunk {
  u32x4 w0[PU], w1[PU];
};

// loads issued by unit_load(k, 0) and unit_load(k, 1)
static_assert(PU == 8 || PU == 4, "wait_stores encodes counts of 8, 16 and 32 prefetch loads");
__device__ __forceinline__ int prefetch_loads(const PWork& k) {
  return (k.n > 0 ? 2 * PU : 0) + (k.n > 1 ? 2 * PU : 0);
}

// issue the loads of unit u of work k (no-op outside [0, n))
__device__ __forceinline__ void unit_load(const PWork& k, int u, Chunk& c) {
  if (u < 0 || u >= k.n) return;
  const int lane = threadIdx.x % WAVE;
  const int it = k.i0 + (u / k.nch) * k.istep, j = u % k.nch;
  const int64_t r0 = (int64_t)it * k.rowmul;
  const u32x4* p0 = k.W + r0 * k.KV;
  const u32x4* p1 = k.W + (r0 + k.rowoff) * k.KV;
  const int base = k.kb + j * WAVE * PU + lane;
  // Every lane loads every slot: past the end of the range it re-reads the range's last
  // vector (a cache hit), which unit_compute then ignores.  Predicating the loads off
  // instead would make the compiler keep a second copy of both chunk buffers.
#pragma unroll
  for (int v = 0; v < PU; ++v) {
    const int kk = min(base + WAVE * v, k.ke - 1);
    c.w0[v] = ld_stream(p0 + kk);
    c.w1[v] = ld_stream(p1 + kk);
  }
}

template <int BT, bool FP8>
__device__ __forceinline__ void unit_compute(const PWork& k, int u, const Chunk& c, const uint16_t* x, int ldx,
                                             float (&a0)[BT], float (&a1)[BT]) {
  constexpr int EPV = FP8 ? 16 : 8;
  const int lane = threadIdx.x % WAVE;
  const int j = u % k.nch;
  const int base = k.kb + j * WAVE * PU + lane;
#pragma unroll
  for (int v = 0; v < PU; ++v) {
    const int kk = base + WAVE * v;
    if (kk < k.ke) {
#pragma unroll
      for (int b = 0; b < BT; ++b) {
        const uint16_t* xb = x + b * ldx + kk * EPV;
        if (FP8) {
          const u32x4 xa = ld16(xb), xc = ld16(xb + 8);
          a0[b] = dot16_e4m3(c.w0[v], xa, xc, a0[b]);
          a1[b] = dot16_e4m3(c.w1[v], xa, xc, a1[b]);
        } else {
          const u32x4 xa = ld16(xb);
          a0[b] = dot8_bf16(c.w0[v], xa, a0[b]);
          a1[b] = dot8_bf16(c.w1[v], xa, a1[b]);
        }
      }
    }
  }
}

__device__ __forceinline__ void run_epilogue(const MatmulParams& mp, int epi, bool kv_fp8, int b, int item, int r0,
                                             int r1, float a0, float a1) {
  switch (epi) {
    case EPI_LOGITS: pair_epilogue<EPI_LOGITS>(mp, kv_fp8, b, item, r0, r1, a0, a1); break;
    case EPI_RESID: pair_epilogue<EPI_RESID>(mp, kv_fp8, b, item, r0, r1, a0, a1); break;
    case EPI_SILU: pair_epilogue<EPI_SILU>(mp, kv_fp8, b, item, r0, r1, a0, a1); break;
    default: pair_epilogue<EPI_QKV>(mp, kv_fp8, b, item, r0, r1, a0, a1); break;
  }
}

// One product phase.  On entry A and B hold units 0 and 1 of k (loaded before the
// barrier that precedes the phase); on exit they hold units 0 and 1 of `next`, still
// in flight, and every store of the phase has completed.
// x: the phase's activations [BT][ldx] in LDS.
template <int BT, bool FP8, bool KVFP8>
__device__ __forceinline__ void gemv_phase(const MatmulParams& mp, int epi, const PWork& k, const PWork& next, const uint16_t* x,
                           int ldx, Chunk& A, Chunk& B, float* part_lds) {
  const int lane = threadIdx.x % WAVE, w = wave_id();
  const int n2 = (k.n + 1) & ~1;  // an even count keeps `next` landing in (A, B)
  float a0[BT], a1[BT];
#pragma unroll
  for (int b = 0; b < BT; ++b) a0[b] = a1[b] = 0.f;
  int round = 0;
  auto finish = [&](int u) {
    const int it = k.i0 + (u / k.nch) * k.istep;
    const int r0 = it * k.rowmul, r1 = r0 + k.rowoff;
#pragma unroll
    for (int b = 0; b < BT; ++b) {
      a0[b] = wave_sum(a0[b]);
      a1[b] = wave_sum(a1[b]);
    }
    if (k.S == 1) {
      if (lane == 0) {
#pragma unroll
        for (int b = 0; b < BT; ++b) run_epilogue(mp, epi, KVFP8, b, it, r0, r1, a0[b], a1[b]);
      }
    } else if (lane == 0) {
      float* dst = part_lds + ((w * MAX_ROUNDS + round) * 2) * BT;
#pragma unroll
      for (int b = 0; b < BT; ++b) {
        dst[b] = a0[b];
        dst[BT + b] = a1[b];
      }
    }
    ++round;
#pragma unroll
    for (int b = 0; b < BT; ++b) a0[b] = a1[b] = 0.f;
  };
  for (int u = 0; u < n2; u += 2) {
    if (u < k.n) {
      unit_compute<BT, FP8>(k, u, A, x, ldx, a0, a1);
      if (u % k.nch == k.nch - 1) finish(u);
    }
    unit_load(k, u + 2, A);
    if (u + 1 < k.n) {
      unit_compute<BT, FP8>(k, u + 1, B, x, ldx, a0, a1);
      if ((u + 1) % k.nch == k.nch - 1) finish(u + 1);
    }
    unit_load(k, u + 3, B);
  }
  if (k.S > 1) {
    // the waves of a slot each summed one K slice of the same items: add the slices in
    // a fixed order and run the epilogue once per item
    __syncthreads();
    if (k.part == 0 && lane == 0) {
      for (int rr = 0; rr < round; ++rr) {
        const int it = k.i0 + rr * k.istep;
        const int r0 = it * k.rowmul, r1 = r0 + k.rowoff;
#pragma unroll
        for (int b = 0; b < BT; ++b) {
          float s0 = 0.f, s1 = 0.f;
          for (int pp = 0; pp < k.S; ++pp) {
            const float* src = part_lds + (((w + pp) * MAX_ROUNDS + rr) * 2) * BT;
            s0 += src[b];
            s1 += src[BT + b];
          }
          run_epilogue(mp, epi, KVFP8, b, it, r0, r1, s0, s1);
        }
      }
    }
    __syncthreads();
  }
  // every store of this phase is issued: start streaming the next product's weights,
  // then let the stores retire under those loads before the barrier
  unit_load(next, 0, A);
  unit_load(next, 1, B);
  wait_stores(prefetch_loads(next));
}

// ---------------------------------------------------------------- attention, one work group per (sequence, head)
//
// The work group's 8 waves take every 8th KV block of the head's context, each keeping
// the next block's loads in flight while it works on the current one, and merge their
// (m, l, o) in LDS: no partial results leave the CU.  The g query heads of one KV head
// go to work groups of the same XCD (work groups are dealt round-robin over the 8 XCDs),
// so the K/V tiles they share are read from HBM once and hit that XCD's L2 after.

template <int DH, bool FP8>
__device__ __forceinline__ void attn_block_load(const uint8_t* pool, int64_t kb, int64_t vb, int prow, int eoff,
                                                bool coherent, u32x4 (&kr)[KV_BLOCK / (WAVE / (DH / (FP8 ? 16 : 8)))],
                                                u32x4 (&vr)[KV_BLOCK / (WAVE / (DH / (FP8 ? 16 : 8)))]) {
  constexpr int EPL = FP8 ? 16 : 8;
  constexpr int LPP = DH / EPL;
  constexpr int PPP = WAVE / LPP;
  constexpr int NPASS = KV_BLOCK / PPP;
  constexpr int ESZ = FP8 ? 1 : 2;
#pragma unroll
  for (int ps = 0; ps < NPASS; ++ps) {
    const int64_t off = (int64_t)(ps * PPP + prow) * DH + eoff;
    // the block holding this step's token was written by another work group: read it
    // device-coherently; older blocks never change within a step
    kr[ps] = coherent ? cld16(pool + (kb + off) * ESZ) : gld16(pool + (kb + off) * ESZ);
    vr[ps] = coherent ? cld16(pool + (vb + off) * ESZ) : gld16(pool + (vb + off) * ESZ);
  }
}

template <int DH, bool FP8>
__device__ __forceinline__ void attn_block_math(int blk, int ntok, int prow, const float (&qv)[FP8 ? 16 : 8],
                                                const u32x4 (&kr)[KV_BLOCK / (WAVE / (DH / (FP8 ? 16 : 8)))],
                                                const u32x4 (&vr)[KV_BLOCK / (WAVE / (DH / (FP8 ? 16 : 8)))],
                                                float& m, float& l, float (&o)[FP8 ? 16 : 8]) {
  constexpr int EPL = FP8 ? 16 : 8;
  constexpr int LPP = DH / EPL;
  constexpr int PPP = WAVE / LPP;
  constexpr int NPASS = KV_BLOCK / PPP;
  float sc[NPASS];
  bool vld[NPASS];
#pragma unroll
  for (int ps = 0; ps < NPASS; ++ps) {
    const uint32_t wv[4] = {kr[ps].x, kr[ps].y, kr[ps].z, kr[ps].w};
    float s = 0.f;
    if (FP8) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const f32x2 lo = e4m3x2_to_f32x2<false>(wv[i]), hi = e4m3x2_to_f32x2<true>(wv[i]);
        s = fmaf(qv[4 * i], lo.x, s);
        s = fmaf(qv[4 * i + 1], lo.y, s);
        s = fmaf(qv[4 * i + 2], hi.x, s);
        s = fmaf(qv[4 * i + 3], hi.y, s);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        s = fmaf(qv[2 * i], bf16_lo(wv[i]), s);
        s = fmaf(qv[2 * i + 1], bf16_hi(wv[i]), s);
      }
    }
#pragma unroll
    for (int off = 1; off < LPP; off <<= 1) s += __shfl_xor(s, off);
    vld[ps] = blk * KV_BLOCK + ps * PPP + prow < ntok;
    sc[ps] = vld[ps] ? s : -INFINITY;
  }
  float bm = sc[0];
#pragma unroll
  for (int ps = 1; ps < NPASS; ++ps) bm = fmaxf(bm, sc[ps]);
#pragma unroll
  for (int off = LPP; off < WAVE; off <<= 1) bm = fmaxf(bm, __shfl_xor(bm, off));
  const float mn = fmaxf(m, bm);  // finite: the block's first position is valid
  const float alpha = exp2f(m - mn);
  m = mn;
  l *= alpha;
#pragma unroll
  for (int e = 0; e < EPL; ++e) o[e] *= alpha;
#pragma unroll
  for (int ps = 0; ps < NPASS; ++ps) {
    const float pr = exp2f(sc[ps] - mn);
    l += pr;
    const uint32_t wv[4] = {vr[ps].x, vr[ps].y, vr[ps].z, vr[ps].w};
    float vf[EPL];
    if (FP8) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const f32x2 lo = e4m3x2_to_f32x2<false>(wv[i]), hi = e4m3x2_to_f32x2<true>(wv[i]);
        vf[4 * i] = lo.x; vf[4 * i + 1] = lo.y; vf[4 * i + 2] = hi.x; vf[4 * i + 3] = hi.y;
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) { vf[2 * i] = bf16_lo(wv[i]); vf[2 * i + 1] = bf16_hi(wv[i]); }
    }
#pragma unroll
    for (int e = 0; e < EPL; ++e) o[e] = fmaf(pr, vld[ps] ? vf[e] : 0.f, o[e]);
  }
}

template <int DH, bool FP8>
__device__ void attention_phase(const StepParams& p, int layer, float* lds) {
  constexpr int EPL = FP8 ? 16 : 8;
  constexpr int LPP = DH / EPL;
  constexpr int PPP = WAVE / LPP;
  constexpr int NPASS = KV_BLOCK / PPP;
  const int lane = threadIdx.x % WAVE, w = wave_id();
  const int prow = lane / LPP, eoff = (lane % LPP) * EPL;
  const int g = p.Hq / p.Hkv;
  const int G = gridDim.x;
  const float qscale = 1.4426950408889634f / sqrtf((float)DH);
  const uint8_t* pool = static_cast<const uint8_t*>(p.pool);
  float* sm = lds;           // [PW]
  float* sl = lds + PW;      // [PW]
  float* so = lds + 2 * PW;  // [PW][DH]
  // Unit (group grp = (sequence b, kv head c), head h of the group).  Group grp goes to
  // "XCD" grp % 8, i.e. to the work groups whose id is grp % 8 mod 8; within it the
  // group's g heads take consecutive slots.  (Any assignment is correct; this one lets
  // the heads of a group share one L2.)
  const int nx = min(G, 8);  // classes; a grid smaller than 8 still covers every group
  const int xcd = blockIdx.x % nx, per_xcd = (G + nx - 1 - xcd) / nx, idx = blockIdx.x / nx;
  const int groups = p.Bp * p.Hkv;
  const int groups_here = (groups + nx - 1 - xcd) / nx;
  for (int slot = idx; slot < groups_here * g; slot += per_xcd) {
    const int h = slot % g, grp = (slot / g) * nx + xcd;
    const int b = grp / p.Hkv, c = grp % p.Hkv, j = c * g + h;
    const int pos = gld(p.lens + b);
    const int ntok = pos + 1;
    const int nblk = pos >= 0 ? pos / KV_BLOCK + 1 : 0;
    float m = -INFINITY, l = 0.f, o[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) o[e] = 0.f;
    if (w < nblk) {
      float qv[EPL];
      const float* qh = p.q + ((int64_t)b * p.Hq + j) * DH + eoff;
#pragma unroll
      for (int e = 0; e < EPL; e += 4) {
        const f32x4 t = cld_f4(qh + e);
        qv[e] = t.x * qscale;
        qv[e + 1] = t.y * qscale;
        qv[e + 2] = t.z * qscale;
        qv[e + 3] = t.w * qscale;
      }
      u32x4 ka[NPASS], va[NPASS], kb2[NPASS], vb2[NPASS];
      auto block_base = [&](int blk, int64_t& kb, int64_t& vb) {
        const int phys = gld(p.bt + (int64_t)b * p.bps + blk);
        kb = kv_offset(layer, 0, phys, c, 0, 0, p.num_blocks, p.Hkv, DH);
        vb = kv_offset(layer, 1, phys, c, 0, 0, p.num_blocks, p.Hkv, DH);
      };
      // every load targets a valid block (clamped past the end) and the math is skipped
      // for blocks outside this wave's share
      int64_t kb, vb;
      block_base(w, kb, vb);
      attn_block_load<DH, FP8>(pool, kb, vb, prow, eoff, w == nblk - 1, ka, va);
      for (int blk = w; blk < nblk; blk += 2 * PW) {
        const int b1 = min(blk + PW, nblk - 1);
        block_base(b1, kb, vb);
        attn_block_load<DH, FP8>(pool, kb, vb, prow, eoff, b1 == nblk - 1, kb2, vb2);
        attn_block_math<DH, FP8>(blk, ntok, prow, qv, ka, va, m, l, o);
        if (blk + PW >= nblk) break;
        const int b2 = min(blk + 2 * PW, nblk - 1);
        block_base(b2, kb, vb);
        attn_block_load<DH, FP8>(pool, kb, vb, prow, eoff, b2 == nblk - 1, ka, va);
        attn_block_math<DH, FP8>(blk + PW, ntok, prow, qv, kb2, vb2, m, l, o);
      }
#pragma unroll
      for (int off = LPP; off < WAVE; off <<= 1) {
        l += __shfl_xor(l, off);
#pragma unroll
        for (int e = 0; e < EPL; ++e) o[e] += __shfl_xor(o[e], off);
      }
    }
    if (lane == 0) {
      sm[w] = m;
      sl[w] = l;
    }
    if (prow == 0) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) so[w * DH + eoff + e] = o[e];
    }
    __syncthreads();
    for (int e = threadIdx.x; e < DH; e += PT) {
      float M = sm[0];
#pragma unroll
      for (int ww = 1; ww < PW; ++ww) M = fmaxf(M, sm[ww]);
      float O = 0.f, Lsum = 0.f;
      if (M != -INFINITY) {
#pragma unroll
        for (int ww = 0; ww < PW; ++ww) {
          const float f = exp2f(sm[ww] - M);
          O = fmaf(f, so[ww * DH + e], O);
          Lsum = fmaf(f, sl[ww], Lsum);
        }
      }
      cst(p.o + ((int64_t)b * p.Hq + j) * DH + e, f32_to_bf16(M != -INFINITY ? O / Lsum : 0.f));
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------- the step

template <int BT, bool WFP8, bool KVFP8, int DH>
__global__ __launch_bounds__(PT, 1) void k_step(StepParams p) {
  extern __shared__ __align__(16) uint8_t smem[];
  uint16_t* xs = reinterpret_cast<uint16_t*>(smem);
  float* part_lds = reinterpret_cast<float*>(smem + p.xs_bytes);
  float* red = part_lds + PW * MAX_ROUNDS * 2 * BT;
  const int d = p.d, dh = p.dh, Hq = p.Hq, Hkv = p.Hkv;

  // embedding rows -> residual stream
  {
    const int total = BT * d;
    for (int e = blockIdx.x * PT + threadIdx.x; e < total; e += gridDim.x * PT) {
      const int b = e / d, i = e % d;
      const int64_t id = gld(p.ids + b);
      float v;
      if (WFP8)
        v = e4m3x2_to_f32x2<false>((uint32_t)gld(static_cast<const uint8_t*>(p.embed.w) + id * d + i)).x *
            gld(p.embed.scale + id);
      else
        v = bf16_to_f32(gld(static_cast<const uint16_t*>(p.embed.w) + id * d + i));
      cst(p.h + e, v);
    }
  }

  MatmulParams mp{};
  mp.Bp = BT;
  mp.seq_lens = p.lens;
  mp.bt = p.bt;
  mp.rope = p.rope;
  mp.pool = p.pool;
  mp.q = p.q;
  mp.Hq = Hq;
  mp.Hkv = Hkv;
  mp.dh = dh;
  mp.num_blocks = p.num_blocks;
  mp.bps = p.bps;
  mp.d_ff = p.dff;

  const int qkv_items = (Hq + 2 * Hkv) * dh / 2;
  // product phases in order: per layer QKV, O, gate+up, down (attention sits between QKV
  // and O), then the LM head; `g` counts product phases: layer g / 4, kind g % 4
  const int n_prod = 4 * p.L + 1;
  auto work_of = [&](int g) -> PWork {
    if (g >= n_prod) {
      PWork none = make_work(p.lm.w, d, WFP8, p.V / 2, 2, 1, 1);
      none.n = 0;
      return none;
    }
    if (g == n_prod - 1) return make_work(p.lm.w, d, WFP8, p.V / 2, 2, 1, p.split[4]);
    const int l = g / 4;
    switch (g % 4) {
      case 0: return make_work(load_mat(p.w_qkv + l).w, d, WFP8, qkv_items, 2, 1, p.split[0]);
      case 1: return make_work(load_mat(p.w_o + l).w, Hq * dh, WFP8, d / 2, 2, 1, p.split[1]);
      case 2: return make_work(load_mat(p.w_gu + l).w, d, WFP8, p.dff, 1, p.dff, p.split[2]);
      default: return make_work(load_mat(p.w_down + l).w, p.dff, WFP8, d / 2, 2, 1, p.split[3]);
    }
  };

  Chunk A, B;
  PWork cur = work_of(0);
  unit_load(cur, 0, A);
  unit_load(cur, 1, B);
  wait_stores(prefetch_loads(cur));
  grid_sync(p);

  for (int g = 0; g < n_prod; ++g) {
    const int l = g / 4;
    const int kind = g == n_prod - 1 ? 4 : g % 4;
    int epi, K;
    const uint16_t* x = xs;
    // stage this product's activations in LDS and set its epilogue
    if (kind == 0) {  // x = RMSNorm(h) g_attn; [q; k; v] = W_qkv x, RoPE, K/V -> cache
      norm_to_lds<BT>(p.h, p.attn_norm + (int64_t)l * d, d, p.eps, xs, red);
      const DevMat m = load_mat(p.w_qkv + l);
      mp.W = m.w;
      mp.scale = m.scale;
      mp.N = 2 * qkv_items;
      K = d;
      epi = EPI_QKV;
    } else if (kind == 1) {  // h += W_o o
      copy_to_lds<BT>(p.o, Hq * dh, Hq * dh, xs);
      const DevMat m = load_mat(p.w_o + l);
      mp.W = m.w;
      mp.scale = m.scale;
      mp.N = d;
      K = Hq * dh;
      mp.out = p.h;
      mp.ldo = d;
      epi = EPI_RESID;
    } else if (kind == 2) {  // a = silu(W_gate x) * (W_up x), x = RMSNorm(h) g_mlp
      norm_to_lds<BT>(p.h, p.mlp_norm + (int64_t)l * d, d, p.eps, xs, red);
      const DevMat m = load_mat(p.w_gu + l);
      mp.W = m.w;
      mp.scale = m.scale;
      mp.N = 2 * p.dff;
      K = d;
      mp.act = p.a;
      mp.ldact = p.dff;
      epi = EPI_SILU;
    } else if (kind == 3) {  // h += W_down a
      copy_to_lds<BT>(p.a, p.dff, p.dff, xs);
      const DevMat m = load_mat(p.w_down + l);
      mp.W = m.w;
      mp.scale = m.scale;
      mp.N = d;
      K = p.dff;
      mp.out = p.h;
      mp.ldo = d;
      epi = EPI_RESID;
    } else {  // logits = W_lm RMSNorm(h) g_final
      norm_to_lds<BT>(p.h, p.final_norm, d, p.eps, xs, red);
      mp.W = p.lm.w;
      mp.scale = p.lm.scale;
      mp.N = p.V;
      K = d;
      mp.out = p.logits;
      mp.ldo = p.V;
      epi = EPI_LOGITS;
    }
    mp.K = K;
    mp.layer = l;
    // the attention phase after QKV needs its registers: the O projection's first
    // chunks are loaded when attention is done, just before the barrier
    const PWork nxt = work_of(kind == 0 ? n_prod : g + 1);
    gemv_phase<BT, WFP8, KVFP8>(mp, epi, cur, nxt, x, K, A, B, part_lds);
    if (g == n_prod - 1) break;
    grid_sync(p);
    if (kind == 0) {
      // attention over positions 0..p, one work group per (sequence, head); the chunk
      // registers hold nothing useful here (QKV prefetched nothing): say so, so that
      // the compiler does not keep them alive through the attention code
      A = Chunk{};
      B = Chunk{};
      attention_phase<DH, KVFP8>(p, l, reinterpret_cast<float*>(smem));
      cur = work_of(g + 1);
      unit_load(cur, 0, A);
      unit_load(cur, 1, B);
      wait_stores(prefetch_loads(cur));
      grid_sync(p);
    } else {
      cur = nxt;
    }
  }
}

// ---------------------------------------------------------------- launch

namespace {
template <int BT, bool WFP8, bool KVFP8, int DH>
hipError_t step_go(const StepParams& p, size_t lds, int grid, hipStream_t s) {
  auto kern = k_step<BT, WFP8, KVFP8, DH>;
  static size_t attr_lds = 0;  // per instance: the dynamic LDS size allowed so far
  if (lds > attr_lds) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)lds);
    if (e != hipSuccess) return e;
    attr_lds = lds;
  }
  hipLaunchKernelGGL(kern, dim3(grid), dim3(PT), lds, s, p);
  return hipGetLastError();
}

template <bool WFP8, bool KVFP8, int DH>
hipError_t step_bt(const StepParams& p, size_t lds, int grid, hipStream_t s) {
  switch (p.Bp) {
    case 1: return step_go<1, WFP8, KVFP8, DH>(p, lds, grid, s);
    case 2: return step_go<2, WFP8, KVFP8, DH>(p, lds, grid, s);
    case 4: return step_go<4, WFP8, KVFP8, DH>(p, lds, grid, s);
    case 8: return step_go<8, WFP8, KVFP8, DH>(p, lds, grid, s);
    default: return hipErrorInvalidValue;
  }
}
}  // namespace

// At least 84 KB, so that a CU never holds two of these work groups: the grid is one
// work group per CU.
size_t step_lds_bytes(const StepParams& p) {
  const size_t need = (size_t)p.xs_bytes + PW * MAX_ROUNDS * 2 * 8 * 4 + PW * 8 * 4;
  return need > 84 * 1024 ? need : 84 * 1024;
}

int step_max_rounds() { return MAX_ROUNDS; }
int step_waves_per_group() { return PW; }

hipError_t launch_step(const StepParams& p, bool w_fp8, bool kv_fp8, int grid, hipStream_t s) {
  const size_t lds = step_lds_bytes(p);
  if (p.dh == 128) {
    if (w_fp8) return kv_fp8 ? step_bt<true, true, 128>(p, lds, grid, s) : step_bt<true, false, 128>(p, lds, grid, s);
    return kv_fp8 ? step_bt<false, true, 128>(p, lds, grid, s) : step_bt<false, false, 128>(p, lds, grid, s);
  }
  if (p.dh == 64) {
    if (w_fp8) return kv_fp8 ? step_bt<true, true, 64>(p, lds, grid, s) : step_bt<true, false, 64>(p, lds, grid, s);
    return kv_fp8 ? step_bt<false, true, 64>(p, lds, grid, s) : step_bt<false, false, 64>(p, lds, grid, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace dec
