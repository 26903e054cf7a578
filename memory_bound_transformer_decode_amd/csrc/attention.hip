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
// k_attn_split: work group (split j, kv head c, sequence b), 8 waves.  The blocks
// of positions 0..p are divided evenly between n_split work groups (one, unless the
// context is long and the batch small); wave w of a work group takes blocks w, w + 8,
// ..., with the next block's loads in flight while it works on the current one (the
// physical block ids are fetched once, one per lane).  A lane holds 8 elements of one
// position's K and V row; scores are reduced over the lanes of a row, then the
// running max m, sum l and output o are updated (base-2 exponentials with log2(e)
// folded into q).  The waves merge in LDS; with one split the work group writes o.
// The last work group of a (sequence, kv head) to finish -- counted by a
// self-resetting arrival counter -- combines the splits:
// o = sum_j 2^(m_j - M) o_j / sum_j 2^(m_j - M) l_j, M = max_j m_j, as bf16; a
// sequence with no positions (a padded row) gets o = 0.  Partials go through
// device-coherent stores and loads, since the work groups of one (sequence, kv
// head) run on different XCDs, whose L2 caches are not coherent with each other.

#include "attn_unit.h"

namespace dec {

template <int DH, bool FP8, int G, int NW>
__global__ __launch_bounds__(WAVE * NW) void k_attn_split(AttnParams p) {
  __shared__ AttnSmem<DH, G, NW> S;
  attn_unit<DH, FP8, G, NW>(p, blockIdx.x, blockIdx.y, blockIdx.z, S);
}

// The same work with each wave's blocks on the matrix cores (attn_wave_mfma): for batches
// where the per-position arithmetic of the vector form is what the kernel waits on.
template <int DH, bool FP8, int G, int NW>
__global__ __launch_bounds__(WAVE * NW) void k_attn_mfma(AttnParams p) {
  __shared__ AttnSmem<DH, G, NW> S;
  __shared__ __align__(16) uint8_t vt[NW * attn_wave_lds<DH>()];
  attn_unit<DH, FP8, G, NW, true>(p, blockIdx.x, blockIdx.y, blockIdx.z, S, vt);
}

namespace {

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Work groups per attention launch to aim for (one per CU of MI355X), and the context
// blocks one work group takes before the context is split further.  A split costs a
// round of partial stores, an arrival counter and a combine; a longer split costs more
// blocks per wave in sequence (splits of 16 or 24 blocks, and target grids of 512 or
// 1024 work groups, measured slower).
constexpr int ATTN_TARGET_GROUPS = 256;
constexpr int ATTN_BLOCKS_PER_SPLIT = 8;

template <int DH, bool FP8, int G>
hipError_t attn_g(const AttnParams& p, hipStream_t s) {
  const dim3 grid(p.n_split, p.Hkv, p.Bp);
  if (p.mfma)
    hipLaunchKernelGGL((k_attn_mfma<DH, FP8, G, ATTN_WAVES>), grid, dim3(WAVE * ATTN_WAVES), 0, s, p);
  else
    hipLaunchKernelGGL((k_attn_split<DH, FP8, G, ATTN_WAVES>), grid, dim3(WAVE * ATTN_WAVES), 0, s, p);
  return hipGetLastError();
}

template <int DH, bool FP8>
hipError_t attn_go(const AttnParams& p, hipStream_t s) {
  switch (p.Hq / p.Hkv) {
    case 1: return attn_g<DH, FP8, 1>(p, s);
    case 2: return attn_g<DH, FP8, 2>(p, s);
    case 3: return attn_g<DH, FP8, 3>(p, s);
    case 4: return attn_g<DH, FP8, 4>(p, s);
    case 5: return attn_g<DH, FP8, 5>(p, s);
    case 6: return attn_g<DH, FP8, 6>(p, s);
    case 7: return attn_g<DH, FP8, 7>(p, s);
    case 8: return attn_g<DH, FP8, 8>(p, s);
    default: return hipErrorInvalidValue;
  }
}
}  // namespace

// Split only past ATTN_BLOCKS_PER_SPLIT blocks (of the longest context the block table
// holds), and only while there are few (sequence, kv head) groups; every wave holds the
// ids of its blocks in its 64 lanes, which sets the fewest splits.
int attn_splits(const AttnShape& c, int Bp) {
  int ns = (ATTN_TARGET_GROUPS + Bp * c.Hkv - 1) / (Bp * c.Hkv);
  const int by_len = (c.bps + ATTN_BLOCKS_PER_SPLIT - 1) / ATTN_BLOCKS_PER_SPLIT;
  if (ns > by_len) ns = by_len;
  const int min_ns = (c.bps + WAVE * ATTN_WAVES - 1) / (WAVE * ATTN_WAVES);
  if (ns < min_ns) ns = min_ns;
  if (ns > ATTN_MAX_SPLIT) ns = ATTN_MAX_SPLIT;
  return ns < 1 ? 1 : ns;
}

AttnScratch attn_scratch(const AttnShape& c, int Bp) {
  const size_t rows = (size_t)Bp * attn_splits(c, Bp);
  AttnScratch a{};
  size_t off = 0;
  a.part_o = off;
  off = align256(off + rows * c.Hq * c.dh * 4);
  a.part_ml = off;
  off = align256(off + rows * c.Hq * 2 * 4);
  a.cnt = off;
  off = align256(off + (size_t)Bp * c.Hkv * 4);
  a.total = off;
  return a;
}

hipError_t launch_attention(const AttnParams& p, bool kv_fp8, hipStream_t s) {
  if (p.n_split < 1 || p.n_split > ATTN_MAX_SPLIT || p.bps > p.n_split * WAVE * ATTN_WAVES) return hipErrorInvalidValue;
  if (p.dh == 64) return kv_fp8 ? attn_go<64, true>(p, s) : attn_go<64, false>(p, s);
  if (p.dh == 128) return kv_fp8 ? attn_go<128, true>(p, s) : attn_go<128, false>(p, s);
  return hipErrorInvalidValue;
}

}  // namespace dec

namespace dec {

// zero n counters (a kernel rather than a memset, so that a captured graph replays it)
__global__ void k_zero_u32(unsigned* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

hipError_t launch_zero_u32(unsigned* p, int n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_zero_u32, dim3((n + 255) / 256), dim3(256), 0, s, p, n);
  return hipGetLastError();
}

}  // namespace dec
