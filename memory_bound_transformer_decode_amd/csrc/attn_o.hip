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
//    (attn_unit, MFMA form), writing o;
//  * every later work group takes R <= 6 rows of W_o per wave, loads them whole into
//    registers (the weights depend on nothing), then polls o until every element is
//    written, and finishes h += s (W_o o) for its rows.  The O weights thus stream while
//    attention runs.
//
// o is its own completion flag: it holds ATTN_O_PENDING in every element when the launch
// starts (stored by an earlier launch: the step's embedding kernel for the first layer,
// the previous layer's launch otherwise; two buffers alternate by layer), each element is
// written once, by one two-byte device-coherent store of its final value, which is never
// that pattern, and the O work groups read o with device-coherent loads, so a 16-byte
// slice without the pattern holds final values.  Against a counter that the writers
// would raise after their stores are acknowledged, this saves the acknowledgement, the
// counter's round trip and the separate read of o.
//
// Forward progress: the attention work groups come first in block order and the
// dispatcher hands out each XCD's work groups in block order, so every attention work
// group is placed before an O work group can take its place.  The O work groups' wait
// is bounded all the same: after `spin` polls it sets *abort and goes on, so the launch
// always ends (with wrong values, which the host reports through the flag).

#include "attn_unit.h"

namespace dec {

namespace {

// Whether any of the 8 bf16 of v is ATTN_O_PENDING
__device__ __forceinline__ bool o_pending(const u32x4& v) {
  bool any = false;
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) any |= (w[j] & 0xFFFFu) == ATTN_O_PENDING || (w[j] >> 16) == ATTN_O_PENDING;
  return any;
}

// Copy o [K] bf16 into LDS (xs) once every element is written: each thread polls its
// 16-byte slices with device-coherent loads, keeps the complete ones and polls the rest
// again, until no thread of the work group has a slice pending (or `spin` polls have
// passed, or another work group has given up).  SPT: slices per thread, K <= SPT 8 NT.
template <int NT, int SPT>
__device__ __forceinline__ void attn_o_stage(const uint16_t* o, int K, uint16_t* xs, int* abort, int spin) {
  const int tid = threadIdx.x;
  unsigned pending = 0;
#pragma unroll
  for (int j = 0; j < SPT; ++j)
    if ((tid + j * NT) * 8 < K) pending |= 1u << j;
  for (int it = 0;; ++it) {
    if (it >= spin) {  // spin 0: give up at once (the failure path's own test)
      if (tid == 0) cst(abort, 1);
      break;
    }
    u32x4 v[SPT];
#pragma unroll
    for (int j = 0; j < SPT; ++j)
      if (pending >> j & 1u) v[j] = cld16(o + (tid + j * NT) * 8);
#pragma unroll
    for (int j = 0; j < SPT; ++j) {
      if ((pending >> j & 1u) && !o_pending(v[j])) {
        *reinterpret_cast<u32x4*>(xs + (tid + j * NT) * 8) = v[j];
        pending &= ~(1u << j);
      }
    }
    if (!__syncthreads_or(pending != 0)) break;
    if ((it & 15) == 15 && __syncthreads_or(tid == 0 && cld(abort) != 0)) break;
    __builtin_amdgcn_s_sleep(1);
  }
  __syncthreads();
}

// Mark the next layer's o as not yet written: the O work groups share its 16-byte slices.
__device__ __forceinline__ void attn_o_mark_next(uint16_t* next, int K, int grp, int n_grp, int NT) {
  for (int i = grp * NT + (int)threadIdx.x; i < K / 8; i += n_grp * NT) {
    uint64_t* q = reinterpret_cast<uint64_t*>(next + (int64_t)i * 8);
    cst(q, (uint64_t)ATTN_O_PENDING2 << 32 | ATTN_O_PENDING2);
    cst(q + 1, (uint64_t)ATTN_O_PENDING2 << 32 | ATTN_O_PENDING2);
  }
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

  attn_o_mark_next(P.next, p.K, grp, (int)gridDim.x - P.n_attn, NW * WAVE);
  attn_o_stage<NW * WAVE, (ATTN_O_VMAX * WAVE * 16 + NW * WAVE * 8 - 1) / (NW * WAVE * 8)>(p.x, p.K, xs, P.abort,
                                                                                       P.spin);

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
    attn_unit<DH, FP8, G, ATTN_WAVES, true>(P.a, split, c, b, S, vt);
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
  if (!attn_o_supported(a.Hq, a.Hkv, a.dh) || a.Bp != 1 || !a.mfma || m.Bp != 1 || !P.abort || !P.next ||
      P.next == a.o || m.x != a.o || P.rows < 1 || P.rows > ATTN_O_RMAX || P.n_attn != a.n_split * a.Hkv * a.Bp)
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
