// Weight-streaming matrix kernels of the decode step: y = s (.) (W x) for a skinny
// activation block x [Bp][K], with the step's fused epilogues.
//
// Decode reads every weight once per step to produce one column of activations per
// sequence, so these kernels are HBM-bound (intensity 2B/b_w FLOP/byte; "GPU
// Inference Internals", Roofline: Why Decode Is Memory-Bound).  Two shapes:
//
//  * k_gemv (Bp <= 8): one wave per work group; a wave owns a contiguous range of
//    row pairs and streams both rows with 16-byte non-temporal loads, U loads per
//    row in flight; activations come from L2 (they are tiny and shared by every
//    wave); bf16 products use v_dot2_f32_bf16, one-byte weights (E4M3 or int8 codes)
//    are widened to bf16 in registers (exact) and the per-row scale is applied once in
//    the epilogue, so that dequantization costs no pass of its own over the weights
//    (kernel-fusion architecture study, section 11).
//  * Bp >= 16: the batch is wide enough to make this a dense contraction, so MFMA
//    tiles do the products (gemm_mfma.hip).
//
// Fused epilogues (fused-kernel table of "Kernels, Fusion & CUDA Graphs", Fix 1):
// QKV + RoPE + paged KV-cache write, gate+up + SiLU x mul, residual add (O, down),
// and plain fp32 logits (LM head).

#include "common.h"
#include "epilogue.h"
#include "gemv_norm.h"
#include "kernels.h"

namespace dec {

// ---------------------------------------------------------------- gemv (Bp <= 8)

// Work group = one row pair (item blockIdx.x), S waves; wave w takes the contiguous
// slice [KV w / S, KV (w + 1) / S) of the 16-byte vectors of both rows, with U loads
// per row per lane in flight; the slices' sums are added in LDS in wave order.
// XL: the input is x + p.xl (two bf16 parts, see MatmulParams::xl).
template <int BT, int WQ, int EPI, bool KVFP8, int U, int S, bool XL>
__global__ __launch_bounds__(WAVE * S) void k_gemv(MatmulParams p) {
  constexpr int EPV = WQ != W_BF16 ? 16 : 8;  // weight elements per 16-byte vector
  const int lane = threadIdx.x % WAVE;
  const int w = S == 1 ? 0 : __builtin_amdgcn_readfirstlane(threadIdx.x / WAVE);
  const int it = blockIdx.x;
  const int KV = p.K / EPV;  // 16-byte vectors per weight row (K % EPV == 0)
  const int kb = (int)((int64_t)KV * w / S), ke = (int)((int64_t)KV * (w + 1) / S);
  const u32x4* W = static_cast<const u32x4*>(p.W);
  int r0, r1;
  item_rows<EPI>(p, it, r0, r1);
  const u32x4* w0p = W + (int64_t)r0 * KV;
  const u32x4* w1p = W + (int64_t)r1 * KV;
  EpiInputs<EPI, BT> ein;
  if (threadIdx.x == 0) epi_fetch<EPI, BT>(p, r0, r1, ein);
  float acc0[BT], acc1[BT];
#pragma unroll
  for (int b = 0; b < BT; ++b) acc0[b] = acc1[b] = 0.0f;

  for (int k0 = kb + lane; k0 < ke; k0 += WAVE * U) {
    u32x4 w0[U], w1[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int kk = k0 + WAVE * u;
      if (kk < ke) {
        w0[u] = ld_stream(w0p + kk);
        w1[u] = ld_stream(w1p + kk);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int kk = k0 + WAVE * u;
      if (kk < ke) {
        u32x4 v0a, v0b, v1a, v1b;  // the weights as bf16 (one-byte codes widened once)
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
            const uint16_t* xb = (part ? p.xl : p.x) + (int64_t)b * p.ldx + (int64_t)kk * EPV;
            const u32x4 xa = gld16(xb);
            acc0[b] = dot8_bf16(v0a, xa, acc0[b]);
            acc1[b] = dot8_bf16(v1a, xa, acc1[b]);
            if constexpr (WQ != W_BF16) {
              const u32x4 xc = gld16(xb + 8);
              acc0[b] = dot8_bf16(v0b, xc, acc0[b]);
              acc1[b] = dot8_bf16(v1b, xc, acc1[b]);
            }
          }
        }
      }
    }
  }
#pragma unroll
  for (int b = 0; b < BT; ++b) {
    acc0[b] = wave_sum(acc0[b]);
    acc1[b] = wave_sum(acc1[b]);
  }
  if (S == 1) {
    if (lane == 0) {
#pragma unroll
      for (int b = 0; b < BT; ++b) pair_epilogue_pre<EPI, BT>(p, KVFP8, ein, b, it, r0, r1, acc0[b], acc1[b]);
    }
  } else {
    __shared__ float red[S][2][BT];
    if (lane == 0) {
#pragma unroll
      for (int b = 0; b < BT; ++b) {
        red[w][0][b] = acc0[b];
        red[w][1][b] = acc1[b];
      }
    }
    __syncthreads();
    if (threadIdx.x == 0) {
#pragma unroll
      for (int b = 0; b < BT; ++b) {
        float s0 = 0.f, s1 = 0.f;
#pragma unroll
        for (int ww = 0; ww < S; ++ww) {
          s0 += red[ww][0][b];
          s1 += red[ww][1][b];
        }
        pair_epilogue_pre<EPI, BT>(p, KVFP8, ein, b, it, r0, r1, s0, s1);
      }
    }
  }
}

// The same products with the activations x = bf16(h g / sqrt(mean(h^2) + eps)) computed
// by the work group itself from the fp32 residual stream h into LDS, so that the
// RMSNorm fused into the matrix-vector product (the work of a group: gemv_norm.h), ipw
// <= NORM_IPW_MAX waves per work group.
constexpr int NORM_IPW_MAX = 10;

template <int BT, int WQ, int EPI, bool KVFP8, int U>
__global__ __launch_bounds__(WAVE * NORM_IPW_MAX) void k_gemv_norm(MatmulParams p, int n_items, int ipw) {
  extern __shared__ __align__(16) uint8_t gemv_smem[];
  gemv_norm_group<BT, WQ, EPI, KVFP8, U, NORM_IPW_MAX>(p, n_items, blockIdx.x,
                                                               reinterpret_cast<uint16_t*>(gemv_smem), ipw);
}

// ---------------------------------------------------------------- dispatch

namespace {

// One row pair per work group: more work groups than the CUs hold at once, so the
// hardware dispatcher hands out the rest as work groups retire and no CU is left with
// a long static share at the end.  Rows longer than one pass of a wave (64 U vectors)
// are split over S <= 8 waves of the work group (a wave takes more than one pass only
// beyond 8 passes' worth).
template <int BT, int WQ, int EPI, bool KVFP8, int U, bool XL>
hipError_t gemv_sx(const MatmulParams& p, int n_items, int kv, hipStream_t s) {
  const int need = (kv + WAVE * U - 1) / (WAVE * U);
  const dim3 grid(n_items);
  if (need <= 1)
    hipLaunchKernelGGL((k_gemv<BT, WQ, EPI, KVFP8, U, 1, XL>), grid, dim3(WAVE), 0, s, p);
  else if (need <= 2)
    hipLaunchKernelGGL((k_gemv<BT, WQ, EPI, KVFP8, U, 2, XL>), grid, dim3(2 * WAVE), 0, s, p);
  else if (need <= 4)
    hipLaunchKernelGGL((k_gemv<BT, WQ, EPI, KVFP8, U, 4, XL>), grid, dim3(4 * WAVE), 0, s, p);
  else
    hipLaunchKernelGGL((k_gemv<BT, WQ, EPI, KVFP8, U, 8, XL>), grid, dim3(8 * WAVE), 0, s, p);
  return hipGetLastError();
}

// QKV always takes its input in two parts; a plain product (the unfused step's QKV)
// does when given p.xl; the others never do
template <int BT, int WQ, int EPI, bool KVFP8, int U>
hipError_t gemv_s(const MatmulParams& p, int n_items, int kv, hipStream_t s) {
  if constexpr (EPI == EPI_QKV) {
    return gemv_sx<BT, WQ, EPI, KVFP8, U, true>(p, n_items, kv, s);
  } else if constexpr (EPI == EPI_LOGITS) {
    return p.xl ? gemv_sx<BT, WQ, EPI, KVFP8, U, true>(p, n_items, kv, s)
                : gemv_sx<BT, WQ, EPI, KVFP8, U, false>(p, n_items, kv, s);
  } else {
    return gemv_sx<BT, WQ, EPI, KVFP8, U, false>(p, n_items, kv, s);
  }
}

// Waves (row pairs) per work group of the norm-fused kernel.  Where every work group
// fits on the chip at once (two per CU), the waves per group are chosen so that the
// groups split evenly over the CUs: 384 groups of 8 would leave half of the 256 CUs with
// twice the rows of the other half, and the kernel ends with the slowest CU.  Otherwise
// 8, so that one normalization serves 8 row pairs (smaller work groups measured slower
// there: the normalization's L2 reads grow with the number of work groups), and the
// hardware dispatcher balances the rounds.
constexpr int NORM_IPW = 8;

int norm_ipw(const void* kern, int n_items, size_t lds) {
  static int n_cu = 0;
  if (n_cu == 0) {
    int dev = 0, v = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      v = 256;
    n_cu = v > 0 ? v : 256;
  }
  const int ipw = (n_items + 2 * n_cu - 1) / (2 * n_cu);
  if (ipw > NORM_IPW_MAX) return NORM_IPW;
  const int w = ipw < 1 ? 1 : ipw;
  int occ = 0;  // two groups per CU must be resident together
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kern, WAVE * w, lds) != hipSuccess || occ < 2)
    return w <= NORM_IPW ? w : NORM_IPW;
  return w;
}

template <int BT, int WQ, int EPI, bool KVFP8, int U>
hipError_t gemv_norm_go(const MatmulParams& p, int n_items, hipStream_t s) {
  auto kern = k_gemv_norm<BT, WQ, EPI, KVFP8, U>;
  const size_t lds = (size_t)BT * p.K * 2 * (EPI == EPI_QKV ? 2 : 1);  // QKV: two bf16 parts
  static size_t allowed = 64 * 1024;  // per instance: the dynamic LDS size enabled so far
  if (lds > allowed) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    allowed = lds;
  }
  // one choice per (instance, rows, LDS): launches are captured into graphs once per shape
  struct Pick { int n; size_t lds; int ipw; };
  static Pick cache[8];
  static int n_cache = 0;
  int ipw = 0;
  for (int i = 0; i < n_cache; ++i)
    if (cache[i].n == n_items && cache[i].lds == lds) ipw = cache[i].ipw;
  if (ipw == 0) {
    ipw = norm_ipw(reinterpret_cast<const void*>(kern), n_items, lds);
    if (n_cache < 8) cache[n_cache++] = Pick{n_items, lds, ipw};
  }
  const int grid = (n_items + ipw - 1) / ipw;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(WAVE * ipw), lds, s, p, n_items, ipw);
  return hipGetLastError();
}

template <int BT, int WQ, int EPI, bool KVFP8>
hipError_t gemv_go(const MatmulParams& p, hipStream_t s) {
  const int n_items = EPI == EPI_SILU ? p.d_ff : p.N / 2;
  if (n_items <= 0) return hipSuccess;
  const int kv = p.K / (WQ != W_BF16 ? 16 : 8);
  // one wave per row pair, 4 loads per row per lane in flight and as many passes as the
  // row needs (measured faster than one deeper pass, or than splitting the row over
  // waves, which multiplies the normalizations per row pair)
  if (p.nh) return gemv_norm_go<BT, WQ, EPI, KVFP8, 4>(p, n_items, s);
  // shallow per-wave load depth and many waves measured best (more waves resident per
  // CU): U = 4 for rows up to 1024 vectors (two waves per row pair at K = 4096 bf16),
  // U = 2 beyond (eight waves, two passes each, for the d_ff-long rows)
  if (kv <= 1024) return gemv_s<BT, WQ, EPI, KVFP8, 4>(p, n_items, kv, s);
  return gemv_s<BT, WQ, EPI, KVFP8, 2>(p, n_items, kv, s);
}

template <int WQ, int EPI, bool KVFP8>
hipError_t dispatch_bt(const MatmulParams& p, bool mfma, hipStream_t s) {
  if (!mfma) {
    if (p.Bp <= 1) return gemv_go<1, WQ, EPI, KVFP8>(p, s);
    if (p.Bp <= 2) return gemv_go<2, WQ, EPI, KVFP8>(p, s);
    if (p.Bp <= 4) return gemv_go<4, WQ, EPI, KVFP8>(p, s);
    if (p.Bp <= 8) return gemv_go<8, WQ, EPI, KVFP8>(p, s);
    // no-MFMA mode above 8 rows: run the 8-row gemv on slices of the batch
    for (int b0 = 0; b0 < p.Bp; b0 += 8) {
      MatmulParams q = p;
      q.x = p.x + (int64_t)b0 * p.ldx;
      q.xl = p.xl ? p.xl + (int64_t)b0 * p.ldx : nullptr;
      q.nh = p.nh ? p.nh + (int64_t)b0 * p.K : nullptr;
      q.Bp = p.Bp - b0 < 8 ? p.Bp - b0 : 8;
      q.out = p.out ? p.out + (int64_t)b0 * p.ldo : nullptr;
      q.act = p.act ? p.act + (int64_t)b0 * p.ldact : nullptr;
      q.q = p.q ? p.q + (int64_t)b0 * p.Hq * p.dh : nullptr;
      q.seq_lens = p.seq_lens ? p.seq_lens + b0 : nullptr;
      q.bt = p.bt ? p.bt + (int64_t)b0 * p.bps : nullptr;
      hipError_t e;
      if (q.Bp <= 1) e = gemv_go<1, WQ, EPI, KVFP8>(q, s);
      else if (q.Bp <= 2) e = gemv_go<2, WQ, EPI, KVFP8>(q, s);
      else if (q.Bp <= 4) e = gemv_go<4, WQ, EPI, KVFP8>(q, s);
      else e = gemv_go<8, WQ, EPI, KVFP8>(q, s);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
  return launch_gemm_mfma(p, EPI, (WFmt)WQ, KVFP8, s);
}

template <int WQ, bool KVFP8>
hipError_t dispatch_epi(const MatmulParams& p, int epi, bool mfma, hipStream_t s) {
  switch (epi) {
    case EPI_LOGITS: return dispatch_bt<WQ, EPI_LOGITS, KVFP8>(p, mfma, s);
    case EPI_RESID: return dispatch_bt<WQ, EPI_RESID, KVFP8>(p, mfma, s);
    case EPI_SILU: return dispatch_bt<WQ, EPI_SILU, KVFP8>(p, mfma, s);
    default: return dispatch_bt<WQ, EPI_QKV, KVFP8>(p, mfma, s);
  }
}

template <int WQ>
hipError_t dispatch_kv(const MatmulParams& p, int epi, bool kv_fp8, bool mfma, hipStream_t s) {
  return kv_fp8 ? dispatch_epi<WQ, true>(p, epi, mfma, s) : dispatch_epi<WQ, false>(p, epi, mfma, s);
}

}  // namespace

hipError_t launch_matmul(const MatmulParams& p, int epi, WFmt wq, bool kv_fp8, bool mfma, hipStream_t s) {
  // fp16 activations are read by the matrix cores only; the QKV input is fp16 there, and
  // two bf16 parts on the matrix-vector kernels (given, or formed by the norm-fused kernel)
  if (p.x_f16 && (!mfma || p.xl)) return hipErrorInvalidValue;
  if (epi == EPI_QKV && (mfma ? !p.x_f16 : !(p.xl || p.nh))) return hipErrorInvalidValue;
  // the cache dtype only matters for the QKV epilogue; keep one instance otherwise
  if (epi != EPI_QKV) kv_fp8 = false;
  switch (wq) {
    case W_E4M3: return dispatch_kv<W_E4M3>(p, epi, kv_fp8, mfma, s);
    case W_I8: return dispatch_kv<W_I8>(p, epi, kv_fp8, mfma, s);
    default: return dispatch_kv<W_BF16>(p, epi, kv_fp8, mfma, s);
  }
}

}  // namespace dec
