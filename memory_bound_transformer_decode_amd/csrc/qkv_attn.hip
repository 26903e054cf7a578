// QKV projection and decode attention in one kernel (batches of <= 8 rows).
//
// A layer's attention needs, for kv head c, only the q rows of c's g query heads and
// c's k and v rows of the QKV product.  As two kernels, attention starts only after the
// last QKV work group has drained, and then pays its own chain of dependent loads
// (sequence length, block ids, K/V tiles) before any arithmetic.  Here the attention
// work groups are appended to the QKV product's grid: they are dispatched as product
// work groups retire, load their block ids and first K/V tile (positions written by
// earlier steps), and wait only for the product work groups of their own kv head.  This
// is the kernel-fusion study's point that a kernel boundary between producer and
// consumer costs a drain and a ramp ("Kernels, Fusion & CUDA Graphs", Fix 1: kernel
// fusion), applied to the one boundary of the layer whose consumer is latency-bound.
//
// Product part (work groups 0 .. n_groups - 1): the norm-fused matrix-vector product
// with the QKV epilogue (RoPE, q to the fp32 buffer, the new token's K/V into the paged
// cache), written device-coherently.  A work group's 2 IPW rows lie in one head (d_head
// is a multiple of 2 IPW), so after its stores complete it adds one to the counter of that
// head's kv head.  A kv head is complete at (g + 2) d_head / (2 IPW) work groups.
//
// Attention part (the rest, (split, kv head, sequence) with the split fastest): the
// split-K attention unit, waiting on that counter (bounded) before it reads q and the block
// of the new token.  Forward progress: the hardware dispatches a kernel's work groups
// in order of their index on each XCD, so an attention work group occupies a slot only
// after every product work group of its XCD was dispatched, and product work groups
// wait for nothing.
//
// Opt-in (DEC_FLAG_FUSED_QKV_ATTN): at the 8B shapes, batch 1, it measures 23 us against
// 10.7 + 9.4 us for the two kernels.  Per-work-group timestamps show why: after the last
// product work group of a kv head, the attention still runs a chain of dependent
// device-coherent round trips (the count, q and the new K/V, the partials, the combine)
// that costs about what the kernel boundary did, and the product part itself runs
// slower next to the resident attention work groups.

#include "attn_unit.h"
#include "gemv_norm.h"

namespace dec {

template <int BT, bool FP8, bool KVFP8, int U, int IPW, int DH, int G>
__global__ __launch_bounds__(WAVE * IPW) __attribute__((amdgpu_waves_per_eu(4))) void k_qkv_attn(MatmulParams mp, AttnParams ap, int n_items, int n_groups) {
  extern __shared__ __align__(16) uint8_t qa_smem[];
  const int grp = blockIdx.x;
  if (grp < n_groups) {
    gemv_norm_group<BT, FP8, EPI_QKV, KVFP8, U, IPW, true>(mp, n_items, grp, reinterpret_cast<uint16_t*>(qa_smem),
                                                           IPW);
    // every wave's stores complete, then the work group counts for its kv head
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    __syncthreads();
    if (threadIdx.x == 0) {
      const int r = 2 * IPW * grp, qrows = mp.Hq * DH, krows = mp.Hkv * DH;
      const int c = r < qrows ? r / DH / G : r < qrows + krows ? (r - qrows) / DH : (r - qrows - krows) / DH;
      __hip_atomic_fetch_add(ap.ready + (int64_t)c * COUNTER_STRIDE, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    return;
  }
  const int u = grp - n_groups;
  const int split = u % ap.n_split, c = (u / ap.n_split) % ap.Hkv, b = u / (ap.n_split * ap.Hkv);
  attn_unit<DH, KVFP8, G, IPW, true>(ap, split, c, b, *reinterpret_cast<AttnSmem<DH, G, IPW>*>(qa_smem));
}

namespace {

constexpr int QA_U = 4;  // weight loads per row per lane in flight (as the norm-fused kernel)

template <int DH, int G>
constexpr size_t attn_smem_bytes() {
  return sizeof(AttnSmem<DH, G, QKV_ATTN_IPW>);
}

size_t attn_smem_bytes_rt(int dh, int g) {
  // same layout as AttnSmem: G DH + 2 NW G + NW G DH + 2 G MAX_SPLIT + G floats, one int
  const size_t nw = QKV_ATTN_IPW;
  return ((size_t)g * dh + 2 * nw * g + nw * g * dh + 2 * (size_t)g * MAX_SPLIT + g + 1) * 4;
}

template <int BT, bool FP8, bool KVFP8, int DH, int G>
hipError_t qa_go(const MatmulParams& mp, const AttnParams& ap, hipStream_t s) {
  static_assert(attn_smem_bytes<DH, G>() ==
                    (G * DH + 2 * QKV_ATTN_IPW * G + QKV_ATTN_IPW * G * DH + 2 * G * MAX_SPLIT + G + 1) * 4,
                "AttnSmem layout");
  auto kern = k_qkv_attn<BT, FP8, KVFP8, QA_U, QKV_ATTN_IPW, DH, G>;
  const size_t lds = qkv_attn_lds_bytes(BT, mp.K, mp.Hq, mp.Hkv, DH);
  static size_t allowed = 64 * 1024;  // per instance: the dynamic LDS size enabled so far
  if (lds > allowed) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    allowed = lds;
  }
  const int n_items = mp.N / 2;
  const int n_groups = qkv_attn_groups(mp);
  const int grid = n_groups + ap.n_split * ap.Hkv * ap.Bp;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(WAVE * QKV_ATTN_IPW), lds, s, mp, ap, n_items, n_groups);
  return hipGetLastError();
}

template <int BT, bool FP8, bool KVFP8, int DH>
hipError_t qa_g(const MatmulParams& mp, const AttnParams& ap, hipStream_t s) {
  switch (ap.Hq / ap.Hkv) {
    case 1: return qa_go<BT, FP8, KVFP8, DH, 1>(mp, ap, s);
    case 2: return qa_go<BT, FP8, KVFP8, DH, 2>(mp, ap, s);
    case 3: return qa_go<BT, FP8, KVFP8, DH, 3>(mp, ap, s);
    case 4: return qa_go<BT, FP8, KVFP8, DH, 4>(mp, ap, s);
    default: return hipErrorInvalidValue;  // wider groups: QKV_ATTN_MAX_GROUP
  }
}

template <int BT, bool FP8, bool KVFP8>
hipError_t qa_dh(const MatmulParams& mp, const AttnParams& ap, hipStream_t s) {
  if (ap.dh == 64) return qa_g<BT, FP8, KVFP8, 64>(mp, ap, s);
  if (ap.dh == 128) return qa_g<BT, FP8, KVFP8, 128>(mp, ap, s);
  return hipErrorInvalidValue;
}

template <bool FP8, bool KVFP8>
hipError_t qa_bt(const MatmulParams& mp, const AttnParams& ap, hipStream_t s) {
  if (mp.Bp <= 1) return qa_dh<1, FP8, KVFP8>(mp, ap, s);
  if (mp.Bp <= 2) return qa_dh<2, FP8, KVFP8>(mp, ap, s);
  if (mp.Bp <= 4) return qa_dh<4, FP8, KVFP8>(mp, ap, s);
  if (mp.Bp <= 8) return qa_dh<8, FP8, KVFP8>(mp, ap, s);
  return hipErrorInvalidValue;
}

}  // namespace

int qkv_attn_groups(const MatmulParams& mp) { return (mp.N / 2 + QKV_ATTN_IPW - 1) / QKV_ATTN_IPW; }

unsigned qkv_attn_ready_target(int Hq, int Hkv, int dh) {
  return (unsigned)((Hq / Hkv + 2) * dh / (2 * QKV_ATTN_IPW));
}

size_t qkv_attn_lds_bytes(int Bp, int K, int Hq, int Hkv, int dh) {
  const size_t x = (size_t)Bp * K * 2, a = attn_smem_bytes_rt(dh, Hq / Hkv);
  return x > a ? x : a;
}

hipError_t launch_qkv_attn(const MatmulParams& mp, const AttnParams& ap, bool w_fp8, bool kv_fp8, hipStream_t s) {
  if (!mp.nh || mp.Bp > 8 || mp.Bp != ap.Bp || mp.dh != ap.dh || ap.dh % (2 * QKV_ATTN_IPW) != 0 ||
      mp.N != (ap.Hq + 2 * ap.Hkv) * ap.dh || ap.Hq / ap.Hkv > QKV_ATTN_MAX_GROUP ||
      qkv_attn_lds_bytes(mp.Bp, mp.K, ap.Hq, ap.Hkv, ap.dh) > 160 * 1024 - 1024)
    return hipErrorInvalidValue;
  if (w_fp8) return kv_fp8 ? qa_bt<true, true>(mp, ap, s) : qa_bt<true, false>(mp, ap, s);
  return kv_fp8 ? qa_bt<false, true>(mp, ap, s) : qa_bt<false, false>(mp, ap, s);
}

}  // namespace dec
