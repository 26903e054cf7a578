// Attention and the O projection of one layer as one launch, for a single sequence on the
// matrix-vector path.
//
// At batch 1 both ops are short and latency-bound: attention is a chain of dependent
// memory round trips (block ids, K/V, partials, the combine) during which HBM is almost
// idle, and the O product is a few microseconds of weight streaming that a separate
// launch only starts once attention has drained.  Fusing across that boundary removes
// the intermediate launch ("Kernels, Fusion & CUDA Graphs", Fix 1, the fused-kernel
// table; the kernel-fusion architecture study on launch overhead).  Here:
//
//  * work groups 0 .. n_attn - 1 run the attention units exactly as k_attn_mfma does
//    (attn_unit, MFMA form); a unit that writes its (sequence, kv head) group's output
//    counts it on `done` once its stores are acknowledged;
//  * every later work group takes R <= 6 rows of W_o per wave, loads them whole into
//    registers (the weights depend on nothing), then waits until all groups are done,
//    stages the attention output in LDS and finishes h += s (W_o o) for its rows.  The
//    O weights thus stream while attention runs.
//
// The attention output is read with ordinary (L2-cached) loads, so that each XCD's L2
// fetches it once for all its work groups: no XCD holds a line of it from before this
// launch (caches are invalidated between launches, as for every buffer one launch writes
// and the next reads), and within the launch it is read only after the wait, by which
// time its writers' stores have reached memory; each (sequence, kv head) group's output
// is G d_head bf16 = a whole number of 128-byte lines, so no line mixes two writers.
//
// Forward progress: the attention work groups come first in block order and the
// dispatcher hands out each XCD's work groups in block order, so every attention work
// group is placed before an O work group can take its place.  The O work groups' wait
// is bounded all the same: after `spin` polls it sets *abort and goes on, so the launch
// always ends (with wrong values, which the host reports through the flag).

#include "attn_unit.h"

namespace dec {

namespace {

// Count the group's output on `done` once every thread's stores are acknowledged (the
// ordering argument of arrive_after_stores: vmcnt(0) also counts stores here, the
// barrier orders every thread's wait before thread 0's update, and the update is one
// agent-scope atomic).
__device__ __forceinline__ void attn_o_signal(unsigned* done) {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0), expcnt and lgkmcnt not waited on
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __syncthreads();
  if (threadIdx.x == 0) __hip_atomic_fetch_add(done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Wave 0 polls `done` until it reaches `need` (or gives up after `spin` polls, or once
// another wait has given up), then the work group goes on.  Loads issued after the
// barrier see what the counted work groups stored: their stores had reached memory before
// they counted (the compiler-only fences keep the loads below the wait).
__device__ __forceinline__ void attn_o_wait(const unsigned* done, unsigned need, int* abort, int spin) {
  if (threadIdx.x < WAVE) {
    for (int it = 0;; ++it) {
      if (it >= spin) {  // spin 0: give up at once (the failure path's own test)
        if (threadIdx.x == 0) cst(abort, 1);
        break;
      }
      if (cld(done) >= need) break;
      if ((it & 15) == 15 && cld(abort) != 0) break;
      __builtin_amdgcn_s_sleep(2);
    }
  }
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __syncthreads();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// h[r] += s_r sum_k W_o[r][k] o[k] for the rows of O work group `grp`: wave w takes rows
// (grp NW + w) R .. + R - 1 (R <= RM); lane l holds 16-byte vectors l, l + 64, ..., of
// each row (V = K / (64 EPV) of them), so that a row is reduced once over the wave.
template <int WQ, int NW, int RM>
__device__ __forceinline__ void attn_o_rows(const AttnOParams& P, int grp, uint16_t* xs) {
  constexpr int EPV = WQ != W_BF16 ? 16 : 8;  // weight elements per 16-byte vector
  constexpr int VM = ATTN_O_VMAX;
  static_assert(RM * VM <= ATTN_O_WREGS, "weights held per lane");
  const MatmulParams& p = P.m;
  const int lane = threadIdx.x % WAVE;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / WAVE);
  const int KV = p.K / EPV, V = KV / WAVE, R = P.rows;
  const int row0 = (grp * NW + w) * R;
  const u32x4* W = static_cast<const u32x4*>(p.W);

  u32x4 wr[RM][VM];
#pragma unroll
  for (int r = 0; r < RM; ++r) {
    const u32x4* wp = W + (int64_t)min(row0 + r, p.N - 1) * KV + lane;  // past N: a valid row
#pragma unroll
    for (int v = 0; v < VM; ++v)
      if (r < R && v < V) wr[r][v] = ld_stream(wp + v * WAVE);
  }
  // the epilogue's inputs: lane r < R holds row row0 + r's residual and scale
  const int my_row = min(row0 + min(lane, R - 1), p.N - 1);
  const float h_old = gld(p.out + my_row);
  const float sc = p.scale ? gld(p.scale + my_row) : 1.f;

  attn_o_wait(P.done, P.need, P.abort, P.spin);

  // o [K] bf16 into LDS, 16 bytes per thread per pass
  for (int i = threadIdx.x; i < p.K / 8; i += NW * WAVE)
    *reinterpret_cast<u32x4*>(xs + i * 8) = gld16(p.x + (int64_t)i * 8);
  __syncthreads();
  // vector by vector: the lane's o elements of vector v serve every row
  float acc[RM];
#pragma unroll
  for (int r = 0; r < RM; ++r) acc[r] = 0.f;
#pragma unroll
  for (int v = 0; v < VM; ++v) {
    if (v < V) {
      const uint16_t* xp = xs + (lane + v * WAVE) * EPV;
      const u32x4 xa = *reinterpret_cast<const u32x4*>(xp);  // bf16; xb: the second 8 of 16
      const u32x4 xb = WQ != W_BF16 ? *reinterpret_cast<const u32x4*>(xp + 8) : xa;
#pragma unroll
      for (int r = 0; r < RM; ++r) {
        if (r < R) {
          if constexpr (WQ != W_BF16)
            acc[r] = dot16_b8<WQ>(wr[r][v], xa, xb, acc[r]);
          else
            acc[r] = dot8_bf16(wr[r][v], xa, acc[r]);
        }
      }
    }
  }
  float mine = 0.f;  // lane r: the sum of row row0 + r
#pragma unroll
  for (int r = 0; r < RM; ++r) {
    if (r < R) {
      const float t = wave_sum_rows(acc[r]);
      mine = lane == r ? t : mine;
    }
  }
  if (lane < R && row0 + lane < p.N) gst(p.out + row0 + lane, h_old + mine * sc);
}

template <int DH, bool FP8, int G, int WQ, int RM>
__global__ __launch_bounds__(WAVE * ATTN_WAVES) void k_attn_o(AttnOParams P) {
  __shared__ AttnSmem<DH, G, ATTN_WAVES> S;
  __shared__ __align__(16) uint8_t vt[ATTN_WAVES * attn_wave_lds<DH>()];
  const int bid = blockIdx.x;
  if (bid < P.n_attn) {
    const int ns = P.a.n_split;
    const int split = bid % ns, c = (bid / ns) % P.a.Hkv, b = bid / (ns * P.a.Hkv);
    if (attn_unit<DH, FP8, G, ATTN_WAVES, true>(P.a, split, c, b, S, vt)) attn_o_signal(P.done);
    return;
  }
  static_assert(sizeof(vt) >= ATTN_O_VMAX * WAVE * 16 * 2, "o staging must fit the V tiles' LDS");
  attn_o_rows<WQ, ATTN_WAVES, RM>(P, bid - P.n_attn, reinterpret_cast<uint16_t*>(vt));
}

template <int DH, bool FP8, int G, int RM>
hipError_t attn_o_rm(const AttnOParams& P, WFmt wq, int grid, hipStream_t s) {
  const dim3 blk(WAVE * ATTN_WAVES);
  switch (wq) {
    case W_E4M3: hipLaunchKernelGGL((k_attn_o<DH, FP8, G, W_E4M3, RM>), dim3(grid), blk, 0, s, P); break;
    case W_I8: hipLaunchKernelGGL((k_attn_o<DH, FP8, G, W_I8, RM>), dim3(grid), blk, 0, s, P); break;
    default: hipLaunchKernelGGL((k_attn_o<DH, FP8, G, W_BF16, RM>), dim3(grid), blk, 0, s, P); break;
  }
  return hipGetLastError();
}

// up to 3 rows per wave, or up to ATTN_O_RMAX (the larger register set only when needed)
template <int DH, bool FP8, int G>
hipError_t attn_o_wq(const AttnOParams& P, WFmt wq, int grid, hipStream_t s) {
  return P.rows <= 3 ? attn_o_rm<DH, FP8, G, 3>(P, wq, grid, s) : attn_o_rm<DH, FP8, G, ATTN_O_RMAX>(P, wq, grid, s);
}

template <int DH, bool FP8>
hipError_t attn_o_g(const AttnOParams& P, WFmt wq, int grid, hipStream_t s) {
  switch (P.a.Hq / P.a.Hkv) {
    case 4: return attn_o_wq<DH, FP8, 4>(P, wq, grid, s);
    case 5: return attn_o_wq<DH, FP8, 5>(P, wq, grid, s);
    case 8: return attn_o_wq<DH, FP8, 8>(P, wq, grid, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

AttnOPlan attn_o_plan(const AttnShape& sh, int Bp, int N, WFmt wq, int n_cu) {
  const int epv = wq != W_BF16 ? 16 : 8;
  const int K = sh.Hq * sh.dh;
  if (Bp != 1 || !attn_o_supported(sh.Hq, sh.Hkv, sh.dh) || K % (epv * WAVE) != 0 ||
      K / (epv * WAVE) > ATTN_O_VMAX || N <= 0)
    return AttnOPlan{0, 0};
  const int V = K / (epv * WAVE);
  const int min_ns = (sh.bps + WAVE * ATTN_WAVES - 1) / (WAVE * ATTN_WAVES);
  // the most splits (from the standalone launch's count down) whose work groups leave room
  for (int ns = attn_splits(sh, Bp); ns >= min_ns && ns >= 1; --ns) {
    const int free_wg = n_cu - ns * sh.Hkv * Bp;  // one work group per CU (attention's registers)
    if (free_wg <= 0) continue;
    const int R = (N + free_wg * ATTN_WAVES - 1) / (free_wg * ATTN_WAVES);
    if (R <= ATTN_O_RMAX && R * V <= ATTN_O_WREGS) return AttnOPlan{R, ns};
  }
  return AttnOPlan{0, 0};
}

bool attn_o_supported(int Hq, int Hkv, int dh) {
  if (Hkv <= 0 || Hq % Hkv) return false;
  const int g = Hq / Hkv;
  return (dh == 64 || dh == 128) && (g == 4 || g == 5 || g == 8);
}

hipError_t launch_attn_o(const AttnOParams& P, WFmt wq, bool kv_fp8, hipStream_t s) {
  const AttnParams& a = P.a;
  const MatmulParams& m = P.m;
  if (!attn_o_supported(a.Hq, a.Hkv, a.dh) || a.Bp != 1 || !a.mfma || m.Bp != 1 || !P.done || !P.abort ||
      P.rows < 1 || P.rows > ATTN_O_RMAX || P.n_attn != a.n_split * a.Hkv * a.Bp || P.need != (unsigned)(a.Hkv * a.Bp))
    return hipErrorInvalidValue;
  const int epv = wq != W_BF16 ? 16 : 8;
  if (m.K != a.Hq * a.dh || m.K % (epv * WAVE) || m.K / (epv * WAVE) > ATTN_O_VMAX || m.N <= 0 || !m.x || !m.out)
    return hipErrorInvalidValue;
  if (a.n_split < 1 || a.n_split > ATTN_MAX_SPLIT || a.bps > a.n_split * WAVE * ATTN_WAVES) return hipErrorInvalidValue;
  const int rows_per_wg = P.rows * ATTN_WAVES;
  const int grid = P.n_attn + (m.N + rows_per_wg - 1) / rows_per_wg;
  if (a.dh == 64) return kv_fp8 ? attn_o_g<64, true>(P, wq, grid, s) : attn_o_g<64, false>(P, wq, grid, s);
  return kv_fp8 ? attn_o_g<128, true>(P, wq, grid, s) : attn_o_g<128, false>(P, wq, grid, s);
}

}  // namespace dec
