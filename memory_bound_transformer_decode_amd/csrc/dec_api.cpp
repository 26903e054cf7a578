// Host runtime behind include/dec.h: validation, workspace layout, pinned staging
// of the per-step inputs, the kernel plan of one step, and one captured hipGraph
// per batch-size bucket.
//
// The engine step the pages describe has the CPU prepare the batch, block tables
// and metadata, copy them into static device buffers, and replay a graph captured
// once per batch size, padding the live batch up to the nearest captured size
// (ladder 1, 2, 4, then every 8); eager launches stay available for debugging and
// measurement ("Kernels, Fusion & CUDA Graphs", Fix 2: CUDA graphs and The serving
// engine's kernel stack; "CUDA graphs & kernel fusion", Direct answer and Deep
// dive).  Everything that varies per step is read by the kernels from device
// buffers, so one graph per bucket serves every step.

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "dec.h"
#include "kernels.h"

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

constexpr int LADDER[] = {1, 2, 4, 8, 16, 24, 32, 40, 48, 56, 64};
constexpr int N_BUCKETS = sizeof(LADDER) / sizeof(LADDER[0]);
constexpr int MAX_SPLIT = 64;
#ifndef DEC_ATTN_GROUPS
#define DEC_ATTN_GROUPS 256
#endif
constexpr int ATTN_TARGET_GROUPS = DEC_ATTN_GROUPS;  // work groups per attention launch to aim for
constexpr int ATTN_BLOCKS_PER_SPLIT = 8;  // context blocks one attention work group takes alone
constexpr int ATTN_WAVES_ = 8;            // waves per attention work group (attention.hip)
constexpr int WAVE_ = 64;
constexpr uint32_t KNOWN_FLAGS = DEC_FLAG_EAGER | DEC_FLAG_UNFUSED | DEC_FLAG_NO_MFMA | DEC_FLAG_CAPTURE_ALL |
                                 DEC_FLAG_PERSISTENT | DEC_FLAG_FUSED_QKV_ATTN;
constexpr int N_MODES = 16;  // plan-changing flag combinations (UNFUSED, NO_MFMA, PERSISTENT, FUSED_QKV_ATTN)
constexpr int PERSIST_MAX_BATCH = 8;
constexpr size_t PERSIST_XS_BUDGET = 128 * 1024;  // LDS for one layer input block
constexpr int PERSIST_ASSUMED_WAVES = 256 * 8;    // sizes the attention split count
constexpr double BARRIER_TIMEOUT_S = 0.25;

int mode_of(uint32_t flags) {
  return (int)(((flags & DEC_FLAG_UNFUSED) ? 1 : 0) | ((flags & DEC_FLAG_NO_MFMA) ? 2 : 0) |
               ((flags & DEC_FLAG_PERSISTENT) ? 4 : 0) | ((flags & DEC_FLAG_FUSED_QKV_ATTN) ? 8 : 0));
}

int bucket_index(int n) {
  for (int i = 0; i < N_BUCKETS; ++i)
    if (LADDER[i] >= n) return i;
  return -1;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

int blocks_per_seq(const dec_config& c) { return (c.max_seq_len + 15) / 16; }

// Context splits per (sequence, kv head) of the attention kernel.  A split costs a
// round of partial stores, an arrival counter and a combine; a longer split costs
// more blocks per wave in sequence.  Split only past ATTN_BLOCKS_PER_SPLIT blocks
// (at the longest context), and only while there are few (sequence, head) groups.
int n_split_for(const dec_config& c, int Bp) {
  int ns = (ATTN_TARGET_GROUPS + Bp * c.n_kv_heads - 1) / (Bp * c.n_kv_heads);
  const int bps = blocks_per_seq(c), by_len = (bps + ATTN_BLOCKS_PER_SPLIT - 1) / ATTN_BLOCKS_PER_SPLIT;
  if (ns > by_len) ns = by_len;
  // a wave holds the block ids of its share in its 64 lanes
  const int min_ns = (bps + WAVE_ * ATTN_WAVES_ - 1) / (WAVE_ * ATTN_WAVES_);
  if (ns < min_ns) ns = min_ns;
  if (ns > MAX_SPLIT) ns = MAX_SPLIT;
  return ns < 1 ? 1 : ns;
}

// context splits of the persistent step's attention: about two (sequence, head, split)
// units per wave
int n_split_persistent(const dec_config& c, int Bp) {
  int ns = (2 * PERSIST_ASSUMED_WAVES + Bp * c.n_q_heads - 1) / (Bp * c.n_q_heads);
  const int bps = blocks_per_seq(c);
  if (ns > bps) ns = bps;
  if (ns > MAX_SPLIT) ns = MAX_SPLIT;
  return ns < 1 ? 1 : ns;
}

// the persistent step holds one layer input block [Bp][K] of bf16 in LDS
bool persistent_fits(const dec_config& c, int Bp) {
  size_t k = (size_t)c.d_model;
  if ((size_t)c.n_q_heads * c.d_head > k) k = (size_t)c.n_q_heads * c.d_head;
  if ((size_t)c.d_ff > k) k = (size_t)c.d_ff;
  return Bp <= PERSIST_MAX_BATCH && (size_t)Bp * k * 2 <= PERSIST_XS_BUDGET;
}

struct Layout {
  size_t ids, lens, bt, static_bytes;  // static region: ids | lens | block tables
  size_t h, x, q, part_o, part_ml, o, a, rope;
  size_t uf;                           // unfused step: fp32 product rows [MB][max(N)]
  size_t mats, bar, attn_cnt, err;     // persistent-step state
  size_t ready;                        // QKV + attention kernel: [n_kv_heads] counters, 256 B apart
  size_t ssq;                          // folded RMSNorm: row-block sums of squares
  size_t gpart, gcnt;                  // MFMA products split over K: partial tiles, row-block counters
  size_t gpart_floats, gcnt_n;
  size_t total;
};

Layout layout_of(const dec_config& c) {
  Layout L{};
  const size_t MB = (size_t)c.max_batch;
  const size_t bps = (size_t)blocks_per_seq(c);
  size_t off = 0;
  L.ids = off;
  off += MB * 4;
  L.lens = off;
  off += MB * 4;
  L.bt = off;
  off += MB * bps * 4;
  L.static_bytes = off;
  off = align256(off);
  L.h = off;
  off = align256(off + MB * c.d_model * 4);
  L.x = off;
  off = align256(off + MB * c.d_model * 2);
  L.q = off;
  off = align256(off + MB * c.n_q_heads * c.d_head * 4);
  size_t rows_split = 0;  // max over buckets of Bp * n_split
  for (int i = 0; i < N_BUCKETS && LADDER[i] <= c.max_batch; ++i) {
    size_t r = (size_t)LADDER[i] * n_split_for(c, LADDER[i]);
    if (r > rows_split) rows_split = r;
    r = (size_t)LADDER[i] * n_split_persistent(c, LADDER[i]);
    if (persistent_fits(c, LADDER[i]) && r > rows_split) rows_split = r;
  }
  L.part_o = off;
  off = align256(off + rows_split * c.n_q_heads * c.d_head * 4);
  L.part_ml = off;
  off = align256(off + rows_split * c.n_q_heads * 2 * 4);
  L.o = off;
  off = align256(off + MB * c.n_q_heads * c.d_head * 2);
  L.a = off;
  off = align256(off + MB * c.d_ff * 2);
  L.rope = off;
  off = align256(off + (size_t)c.max_seq_len * (c.d_head / 2) * 8);
  L.uf = off;  // largest product row: QKV, gate+up or d_model
  {
    size_t n = (size_t)(c.n_q_heads + 2 * c.n_kv_heads) * c.d_head;
    if ((size_t)2 * c.d_ff > n) n = (size_t)2 * c.d_ff;
    if ((size_t)c.d_model > n) n = c.d_model;
    off = align256(off + MB * n * 4);
  }
  // MFMA products: the largest partial-tile buffer and row-block count over the step's
  // matrices (gate+up also as one plain matrix, as the unfused step runs it) and the
  // buckets (every bucket, so that the size does not depend on which run on MFMA)
  size_t part_floats = 0, n_rb = 0;
  for (int i = 0; i < N_BUCKETS && LADDER[i] <= c.max_batch; ++i) {
    const int Bp = LADDER[i];
    const int qkv_rows = (c.n_q_heads + 2 * c.n_kv_heads) * c.d_head;
    const int shapes[6][3] = {{qkv_rows, 1, c.d_model}, {c.d_model, 1, c.n_q_heads * c.d_head},
                              {c.d_ff, 2, c.d_model},   {2 * c.d_ff, 1, c.d_model},
                              {c.d_model, 1, c.d_ff},   {c.vocab, 1, c.d_model}};
    for (const auto& sh : shapes) {
      const dec::GemmPlan gp = dec::gemm_plan(sh[0], sh[1], sh[2], Bp, c.weight_dtype == DEC_FP8_E4M3);
      if (gp.part_floats > part_floats) part_floats = gp.part_floats;
      if (gp.ks > 1 && (size_t)gp.n_rb > n_rb) n_rb = gp.n_rb;
    }
  }
  L.gpart = off;
  L.gpart_floats = part_floats;
  L.gcnt_n = n_rb;
  off = align256(off + part_floats * 4);
  L.mats = off;  // device copies of the per-layer weight pointers: 4 arrays of n_layers
  off = align256(off + (size_t)4 * (c.n_layers > 0 ? c.n_layers : 1) * sizeof(dec::DevMat));
  L.bar = off;
  off = align256(off + 2 * 4);
  L.attn_cnt = off;
  off = align256(off + MB * c.n_q_heads * 4);
  L.err = off;
  off = align256(off + 4);
  L.ready = off;
  off = align256(off + (size_t)c.n_kv_heads * dec::COUNTER_STRIDE * 4);
  L.ssq = off;
  off = align256(off + (size_t)dec::GEMM_SSQ_MAX * dec::GEMM_SSQ_STRIDE * 4);
  L.gcnt = off;
  off = align256(off + n_rb * dec::COUNTER_STRIDE * 4);
  L.total = off;
  return L;
}

int validate_config(const dec_config* c) {
  if (!c) return fail(DEC_E_INVALID, "config is NULL");
  if (c->n_layers < 0) return fail(DEC_E_INVALID, "n_layers must be >= 0 (got %d)", c->n_layers);
  if (c->d_model <= 0 || c->d_model % 16) return fail(DEC_E_INVALID, "d_model must be a positive multiple of 16 (got %d)", c->d_model);
  if (c->d_ff <= 0 || c->d_ff % 16) return fail(DEC_E_INVALID, "d_ff must be a positive multiple of 16 (got %d)", c->d_ff);
  if (c->n_kv_heads <= 0 || c->n_q_heads <= 0 || c->n_q_heads % c->n_kv_heads)
    return fail(DEC_E_INVALID, "n_q_heads (%d) must be a positive multiple of n_kv_heads (%d)", c->n_q_heads, c->n_kv_heads);
  if (c->n_q_heads / c->n_kv_heads > 8)
    return fail(DEC_E_UNSUPPORTED, "query heads per KV head must be <= 8 (got %d)", c->n_q_heads / c->n_kv_heads);
  if (c->d_head != 64 && c->d_head != 128) return fail(DEC_E_UNSUPPORTED, "d_head must be 64 or 128 (got %d)", c->d_head);
  if (c->vocab <= 0 || c->vocab % 2) return fail(DEC_E_INVALID, "vocab must be positive and even (got %d)", c->vocab);
  if (!(c->rms_eps > 0.f) || !std::isfinite(c->rms_eps)) return fail(DEC_E_INVALID, "rms_eps must be a positive finite number");
  if (!(c->rope_theta > 1.f) || !std::isfinite(c->rope_theta)) return fail(DEC_E_INVALID, "rope_theta must be finite and > 1");
  if ((c->weight_dtype != DEC_BF16 && c->weight_dtype != DEC_FP8_E4M3) || (c->kv_dtype != DEC_BF16 && c->kv_dtype != DEC_FP8_E4M3))
    return fail(DEC_E_INVALID, "weight_dtype / kv_dtype must be DEC_BF16 or DEC_FP8_E4M3");
  if (c->block_size != 16) return fail(DEC_E_UNSUPPORTED, "block_size must be 16 (got %d)", c->block_size);
  if (c->num_blocks <= 0) return fail(DEC_E_INVALID, "num_blocks must be positive (got %d)", c->num_blocks);
  if (bucket_index(c->max_batch) < 0 || LADDER[bucket_index(c->max_batch)] != c->max_batch)
    return fail(DEC_E_INVALID, "max_batch must be one of 1, 2, 4, 8, 16, 24, ..., 64 (got %d)", c->max_batch);
  if (c->max_seq_len <= 0) return fail(DEC_E_INVALID, "max_seq_len must be positive (got %d)", c->max_seq_len);
  if (c->flags & ~KNOWN_FLAGS) return fail(DEC_E_INVALID, "unknown flag bits 0x%x", c->flags & ~KNOWN_FLAGS);
  return DEC_OK;
}

// waves of one work group that share a row pair's K range in a persistent product
// phase: the smallest S in {1, 2, 4, 8} that spreads the rows evenly over the waves
int choose_split(int items, int groups) {
  const int pw = dec::step_waves_per_group();
  int best = 1;
  double best_eff = 0.0;
  for (int S = 1; S <= pw; S *= 2) {
    const int wg_items = (items + groups - 1) / groups;
    const int slots = pw / S;
    const int per_slot = (wg_items + slots - 1) / slots;
    if (S > 1 && per_slot > dec::step_max_rounds()) continue;
    const double work = (double)per_slot / S;
    const double eff = ((double)items / ((double)groups * pw)) / work;
    if (eff > best_eff + 1e-9) {
      best_eff = eff;
      best = S;
    }
  }
  return best;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

}  // namespace

struct dec_ctx {
  dec_config cfg{};
  hipStream_t stream = nullptr;
  hipStream_t cap_stream = nullptr;
  int device = 0;
  void* pool = nullptr;
  uint8_t* ws = nullptr;
  float* logits = nullptr;
  Layout L{};
  bool loaded = false;
  bool failed = false;
  int last_n = 0;  // sequences of the last enqueued step (0: none yet)
  // weights
  dec_mat embed{}, lm{};
  std::vector<dec_mat> qkv, o, gu, down;
  const float* attn_norm = nullptr;
  const float* mlp_norm = nullptr;
  const float* final_norm = nullptr;
  // host staging of the per-step inputs (double-buffered, pinned)
  uint8_t* pinned[2] = {nullptr, nullptr};
  hipEvent_t slot_ev[2] = {nullptr, nullptr};
  bool slot_pending[2] = {false, false};
  int slot = 0;
  // graphs per (bucket, plan flags)
  hipGraphExec_t graphs[N_BUCKETS][N_MODES] = {};
  dec_info info{};
  // persistent step
  int n_cu = 0;
  uint64_t timeout_ticks = 0;
  unsigned* err_host = nullptr;      // pinned, written by the device on a barrier timeout
  unsigned* err_host_dev = nullptr;  // its device address
};

namespace {

template <typename T>
T* ws_ptr(dec_ctx* c, size_t off) {
  return reinterpret_cast<T*>(c->ws + off);
}

int hip_fail(dec_ctx* c, hipError_t e, const char* what) {
  if (c) c->failed = true;
  return fail(DEC_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

#define HIPCHK(ctx, call, what)                       \
  do {                                                \
    hipError_t e_ = (call);                           \
    if (e_ != hipSuccess) return hip_fail(ctx, e_, what); \
  } while (0)

// Parameters of the matrix kernel `which` (dec_matrix) of layer l for a padded batch Bp.
dec::MatmulParams matmul_params(dec_ctx* c, int which, int l, int Bp, int* epi) {
  const dec_config& g = c->cfg;
  const int d = g.d_model, dh = g.d_head, Hq = g.n_q_heads, Hkv = g.n_kv_heads;
  dec::MatmulParams p{};
  p.Bp = Bp;
  p.seq_lens = ws_ptr<int32_t>(c, c->L.lens);
  p.bt = ws_ptr<int32_t>(c, c->L.bt);
  p.rope = ws_ptr<float2>(c, c->L.rope);
  p.pool = c->pool;
  p.q = ws_ptr<float>(c, c->L.q);
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.dh = dh;
  p.num_blocks = g.num_blocks;
  p.bps = blocks_per_seq(g);
  p.d_ff = g.d_ff;
  p.layer = l;
  p.gpart = ws_ptr<float>(c, c->L.gpart);
  p.gcnt = ws_ptr<unsigned>(c, c->L.gcnt);
  p.gpart_floats = c->L.gpart_floats;
  p.gcnt_n = (int)c->L.gcnt_n;
  uint16_t* x = ws_ptr<uint16_t>(c, c->L.x);
  float* h = ws_ptr<float>(c, c->L.h);
  switch (which) {
    case DEC_MAT_QKV:  // [q; k; v] = W_qkv x, RoPE, K/V -> cache
      p.W = c->qkv[l].w;
      p.scale = c->qkv[l].scale;
      p.N = (Hq + 2 * Hkv) * dh;
      p.K = d;
      p.x = x;
      p.ldx = d;
      *epi = dec::EPI_QKV;
      break;
    case DEC_MAT_O:  // h += W_o o
      p.W = c->o[l].w;
      p.scale = c->o[l].scale;
      p.N = d;
      p.K = Hq * dh;
      p.x = ws_ptr<uint16_t>(c, c->L.o);
      p.ldx = Hq * dh;
      p.out = h;
      p.ldo = d;
      // clears the wait counters of the QKV + attention kernel that precedes it
      p.rearm = ws_ptr<unsigned>(c, c->L.ready);
      p.n_rearm = Hkv;
      *epi = dec::EPI_RESID;
      break;
    case DEC_MAT_GATE_UP:  // a = silu(W_gate x) * (W_up x)
      p.W = c->gu[l].w;
      p.scale = c->gu[l].scale;
      p.N = 2 * g.d_ff;
      p.K = d;
      p.x = x;
      p.ldx = d;
      p.act = ws_ptr<uint16_t>(c, c->L.a);
      p.ldact = g.d_ff;
      *epi = dec::EPI_SILU;
      break;
    case DEC_MAT_DOWN:  // h += W_down a
      p.W = c->down[l].w;
      p.scale = c->down[l].scale;
      p.N = d;
      p.K = g.d_ff;
      p.x = ws_ptr<uint16_t>(c, c->L.a);
      p.ldx = g.d_ff;
      p.out = h;
      p.ldo = d;
      *epi = dec::EPI_RESID;
      break;
    default:  // logits = W_lm x
      p.W = c->lm.w;
      p.scale = c->lm.scale;
      p.N = g.vocab;
      p.K = d;
      p.x = x;
      p.ldx = d;
      p.out = c->logits;
      p.ldo = g.vocab;
      *epi = dec::EPI_LOGITS;
      break;
  }
  return p;
}

// Buckets from 8 rows (bf16 weights) or 4 rows (E4M3 weights) up run the products on
// the matrix cores (unless DEC_FLAG_NO_MFMA); smaller ones run the matrix-vector
// kernels.  Measured on the 8B and 32B shapes: the vector kernels' activation reads from
// LDS (Bp per weight vector) and, for E4M3, the widening of every weight once per batch
// row make them slower than the MFMA tiles from these batches on; the MFMA tiles pad the
// batch to 16 columns at no extra HBM traffic.
constexpr int MFMA_MIN_BATCH_BF16 = 8;
constexpr int MFMA_MIN_BATCH_FP8 = 4;
bool use_mfma(const dec_config& g, int Bp) {
  return !(g.flags & DEC_FLAG_NO_MFMA) &&
         Bp >= (g.weight_dtype == DEC_FP8_E4M3 ? MFMA_MIN_BATCH_FP8 : MFMA_MIN_BATCH_BF16);
}

// Row blocks of a residual product on the MFMA tiles -- O (K = Hq dh) or down (K = d_ff)
// -- : the number of row-block sums of squares it writes for the folded RMSNorm that
// follows it.
int residual_row_blocks(const dec_config& g, int Bp, int which) {
  const int K = which == DEC_MAT_O ? g.n_q_heads * g.d_head : g.d_ff;
  return dec::gemm_plan(g.d_model, 1, K, Bp, g.weight_dtype == DEC_FP8_E4M3).n_rb;
}

// The MFMA plan folds the two RMSNorms of a layer and the final one into the products:
// O and down write the next norm's input times its gain (x) and their row blocks' sums of
// squares of h; QKV (past layer 0, whose x the embedding kernel normalizes), gate+up and
// the LM head scale their sums by 1 / rms.  Up to GEMM_SSQ_MAX row blocks; not in the
// unfused step, which runs the norms as kernels of their own.
bool fold_norm(const dec_config& g, int Bp) {
  return use_mfma(g, Bp) && !(g.flags & DEC_FLAG_UNFUSED) &&
         residual_row_blocks(g, Bp, DEC_MAT_O) <= dec::GEMM_SSQ_MAX &&
         residual_row_blocks(g, Bp, DEC_MAT_DOWN) <= dec::GEMM_SSQ_MAX;
}

void set_fold_norm(dec_ctx* c, int which, int l, int Bp, dec::MatmulParams& p) {
  const dec_config& g = c->cfg;
  const int d = g.d_model;
  float* ssq = ws_ptr<float>(c, c->L.ssq);
  p.eps = g.rms_eps;
  if (which == DEC_MAT_O || which == DEC_MAT_DOWN) {
    p.xout = ws_ptr<uint16_t>(c, c->L.x);
    p.ldxo = d;
    p.xg = which == DEC_MAT_O ? c->mlp_norm + (size_t)l * d
           : l + 1 < g.n_layers ? c->attn_norm + (size_t)(l + 1) * d : c->final_norm;
    p.ssq_out = ssq;
  } else if (which == DEC_MAT_GATE_UP || (which == DEC_MAT_QKV && l > 0) ||
             (which == DEC_MAT_LM_HEAD && g.n_layers > 0)) {
    // the sums of the residual product before it: O before gate+up, down before the
    // next layer's QKV and before the LM head
    p.ssq_in = ssq;
    p.ssq_n = residual_row_blocks(g, Bp, which == DEC_MAT_GATE_UP ? DEC_MAT_O : DEC_MAT_DOWN);
  }
}

// Attention's arithmetic on the matrix cores (k_attn_mfma) from buckets of
// ATTN_MFMA_MIN_BATCH rows (unless DEC_FLAG_NO_MFMA).  Measured, with q and P split into
// bf16 parts by the hardware conversion: as fast or faster than the vector form from
// one row (8B batch 1 2.82 against 2.86 ms per step, 32B 6.38 against 6.50), as the
// vector form's per-position arithmetic sits on each wave's chain of blocks.
#ifndef DEC_ATTN_MFMA_MIN_BATCH
#define DEC_ATTN_MFMA_MIN_BATCH 1
#endif
constexpr int ATTN_MFMA_MIN_BATCH = DEC_ATTN_MFMA_MIN_BATCH;
bool attn_mfma(const dec_config& g, int Bp) { return !(g.flags & DEC_FLAG_NO_MFMA) && Bp >= ATTN_MFMA_MIN_BATCH; }

// norm_gain: when set, the kernel computes x = RMSNorm(h) norm_gain itself (fused_norm)
hipError_t run_matmul(dec_ctx* c, int which, int l, int Bp, hipStream_t s, const float* norm_gain = nullptr) {
  const dec_config& g = c->cfg;
  int epi = 0;
  dec::MatmulParams p = matmul_params(c, which, l, Bp, &epi);
  if (norm_gain) {
    p.nh = ws_ptr<float>(c, c->L.h);
    p.ng = norm_gain;
    p.eps = g.rms_eps;
  }
  if (fold_norm(g, Bp)) set_fold_norm(c, which, l, Bp, p);
  return dec::launch_matmul(p, epi, g.weight_dtype == DEC_FP8_E4M3, g.kv_dtype == DEC_FP8_E4M3, use_mfma(g, Bp), s);
}

// Batches of <= 8 rows on the matrix-vector kernels normalize their own input in LDS
// ([Bp][d] bf16 must fit in 128 KB)
bool fused_norm(const dec_config& g, int Bp) {
  return !use_mfma(g, Bp) && Bp <= 8 && (size_t)Bp * g.d_model * 2 <= 128 * 1024;
}

// QKV projection and attention in one kernel (opt-in): the norm-fused batches, for head
// sizes whose QKV work groups each lie in one head, groups of up to QKV_ATTN_MAX_GROUP
// query heads, and while the product's activations or the attention state fit the LDS
// of a work group
bool fuse_qkv_attn(const dec_ctx* c, int Bp) {
  const dec_config& g = c->cfg;
  return fused_norm(g, Bp) && (g.flags & DEC_FLAG_FUSED_QKV_ATTN) && g.d_head % (2 * dec::QKV_ATTN_IPW) == 0 &&
         (g.d_head == 64 || g.d_head == 128) && g.n_q_heads / g.n_kv_heads <= dec::QKV_ATTN_MAX_GROUP &&
         dec::qkv_attn_lds_bytes(Bp, g.d_model, g.n_q_heads, g.n_kv_heads, g.d_head) <= 160 * 1024 - 1024;
}

bool use_persistent(const dec_ctx* c, int Bp) {
  return (c->cfg.flags & DEC_FLAG_PERSISTENT) && !(c->cfg.flags & DEC_FLAG_UNFUSED) && persistent_fits(c->cfg, Bp);
}

// The whole step as one persistent kernel (Bp <= 8).
hipError_t enqueue_persistent(dec_ctx* c, int Bp, hipStream_t s) {
  const dec_config& g = c->cfg;
  dec::StepParams p{};
  p.L = g.n_layers;
  p.d = g.d_model;
  p.Hq = g.n_q_heads;
  p.Hkv = g.n_kv_heads;
  p.dh = g.d_head;
  p.dff = g.d_ff;
  p.V = g.vocab;
  p.Bp = Bp;
  p.num_blocks = g.num_blocks;
  p.bps = blocks_per_seq(g);
  p.n_split = n_split_persistent(g, Bp);
  p.eps = g.rms_eps;
  const int G = c->n_cu;
  p.split[0] = choose_split((g.n_q_heads + 2 * g.n_kv_heads) * g.d_head / 2, G);
  p.split[1] = choose_split(g.d_model / 2, G);
  p.split[2] = choose_split(g.d_ff, G);
  p.split[3] = choose_split(g.d_model / 2, G);
  p.split[4] = choose_split(g.vocab / 2, G);
  size_t k = (size_t)g.d_model;
  if ((size_t)g.n_q_heads * g.d_head > k) k = (size_t)g.n_q_heads * g.d_head;
  if ((size_t)g.d_ff > k) k = (size_t)g.d_ff;
  p.xs_bytes = (int)(((size_t)Bp * k * 2 + 15) & ~(size_t)15);
  const dec::DevMat* mats = ws_ptr<dec::DevMat>(c, c->L.mats);
  const int Ls = g.n_layers > 0 ? g.n_layers : 1;
  p.w_qkv = mats;
  p.w_o = mats + Ls;
  p.w_gu = mats + 2 * Ls;
  p.w_down = mats + 3 * Ls;
  p.embed = dec::DevMat{c->embed.w, c->embed.scale};
  p.lm = dec::DevMat{c->lm.w, c->lm.scale};
  p.attn_norm = c->attn_norm;
  p.mlp_norm = c->mlp_norm;
  p.final_norm = c->final_norm;
  p.ids = ws_ptr<int32_t>(c, c->L.ids);
  p.lens = ws_ptr<int32_t>(c, c->L.lens);
  p.bt = ws_ptr<int32_t>(c, c->L.bt);
  p.h = ws_ptr<float>(c, c->L.h);
  p.q = ws_ptr<float>(c, c->L.q);
  p.part_o = ws_ptr<float>(c, c->L.part_o);
  p.part_ml = ws_ptr<float>(c, c->L.part_ml);
  p.o = ws_ptr<uint16_t>(c, c->L.o);
  p.a = ws_ptr<uint16_t>(c, c->L.a);
  p.rope = ws_ptr<float2>(c, c->L.rope);
  p.pool = c->pool;
  p.logits = c->logits;
  p.bar = ws_ptr<unsigned>(c, c->L.bar);
  p.attn_cnt = ws_ptr<unsigned>(c, c->L.attn_cnt);
  p.err_dev = ws_ptr<unsigned>(c, c->L.err);
  p.err_host = c->err_host_dev;
  p.timeout_ticks = c->timeout_ticks;
  return dec::launch_step(p, g.weight_dtype == DEC_FP8_E4M3, g.kv_dtype == DEC_FP8_E4M3, G, s);
}

// Enqueue the plan of one step for a padded batch of Bp rows on stream s.
// The unfused step (DEC_FLAG_UNFUSED, measurement only): RMSNorm kernels, the matrix
// kernels with a plain fp32 output, and the elementwise work as kernels of its own.
hipError_t enqueue_unfused(dec_ctx* c, int Bp, hipStream_t s) {
  const dec_config& g = c->cfg;
  const bool wfp8 = g.weight_dtype == DEC_FP8_E4M3, kvfp8 = g.kv_dtype == DEC_FP8_E4M3;
  const bool mfma = use_mfma(g, Bp);
  const int d = g.d_model;
  float* h = ws_ptr<float>(c, c->L.h);
  float* uf = ws_ptr<float>(c, c->L.uf);
  hipError_t e;
  dec::NormParams np{};
  np.h = h;
  np.h_out = h;
  np.x = ws_ptr<uint16_t>(c, c->L.x);
  np.d = d;
  np.Bp = Bp;
  np.eps = g.rms_eps;
  np.E = c->embed.w;
  np.E_scale = c->embed.scale;
  np.ids = ws_ptr<int32_t>(c, c->L.ids);
  np.gain = g.n_layers > 0 ? c->attn_norm : c->final_norm;
  if ((e = dec::launch_embed_norm(np, wfp8, s)) != hipSuccess) return e;
  // the product of `which` with its rows written plainly to uf [Bp][N]
  auto plain = [&](int which, int l, dec::MatmulParams* keep) -> hipError_t {
    int epi = 0;
    dec::MatmulParams p = matmul_params(c, which, l, Bp, &epi);
    if (keep) *keep = p;
    p.out = uf;
    p.ldo = p.N;
    return dec::launch_matmul(p, dec::EPI_LOGITS, wfp8, kvfp8, mfma, s);
  };
  dec::AttnParams ap{};
  ap.q = ws_ptr<float>(c, c->L.q);
  ap.pool = c->pool;
  ap.seq_lens = ws_ptr<int32_t>(c, c->L.lens);
  ap.bt = ws_ptr<int32_t>(c, c->L.bt);
  ap.part_o = ws_ptr<float>(c, c->L.part_o);
  ap.part_ml = ws_ptr<float>(c, c->L.part_ml);
  ap.o = ws_ptr<uint16_t>(c, c->L.o);
  ap.cnt = ws_ptr<unsigned>(c, c->L.attn_cnt);
  ap.Bp = Bp;
  ap.Hq = g.n_q_heads;
  ap.Hkv = g.n_kv_heads;
  ap.dh = g.d_head;
  ap.num_blocks = g.num_blocks;
  ap.bps = blocks_per_seq(g);
  ap.n_split = n_split_for(g, Bp);
  ap.mfma = attn_mfma(g, Bp) ? 1 : 0;
  for (int l = 0; l < g.n_layers; ++l) {
    if (l > 0) {
      np.gain = c->attn_norm + (size_t)l * d;
      if ((e = dec::launch_rmsnorm(np, s)) != hipSuccess) return e;
    }
    dec::MatmulParams qp{};
    if ((e = plain(DEC_MAT_QKV, l, &qp)) != hipSuccess) return e;
    if ((e = dec::launch_rope_kv(qp, uf, kvfp8, s)) != hipSuccess) return e;
    ap.layer = l;
    if ((e = dec::launch_attention(ap, kvfp8, s)) != hipSuccess) return e;
    if ((e = plain(DEC_MAT_O, l, nullptr)) != hipSuccess) return e;
    if ((e = dec::launch_add(h, uf, Bp * d, s)) != hipSuccess) return e;
    np.gain = c->mlp_norm + (size_t)l * d;
    if ((e = dec::launch_rmsnorm(np, s)) != hipSuccess) return e;
    if ((e = plain(DEC_MAT_GATE_UP, l, nullptr)) != hipSuccess) return e;
    if ((e = dec::launch_silu_mul(uf, g.d_ff, Bp, ws_ptr<uint16_t>(c, c->L.a), g.d_ff, s)) != hipSuccess) return e;
    if ((e = plain(DEC_MAT_DOWN, l, nullptr)) != hipSuccess) return e;
    if ((e = dec::launch_add(h, uf, Bp * d, s)) != hipSuccess) return e;
  }
  if (g.n_layers > 0) {
    np.gain = c->final_norm;
    if ((e = dec::launch_rmsnorm(np, s)) != hipSuccess) return e;
  }
  return run_matmul(c, DEC_MAT_LM_HEAD, 0, Bp, s);
}

hipError_t enqueue_step(dec_ctx* c, int Bp, hipStream_t s) {
  if (use_persistent(c, Bp)) return enqueue_persistent(c, Bp, s);
  if (c->cfg.flags & DEC_FLAG_UNFUSED) return enqueue_unfused(c, Bp, s);
  const dec_config& g = c->cfg;
  const bool wfp8 = g.weight_dtype == DEC_FP8_E4M3, kvfp8 = g.kv_dtype == DEC_FP8_E4M3;
  const int bps = blocks_per_seq(g);
  int32_t* ids = ws_ptr<int32_t>(c, c->L.ids);
  int32_t* lens = ws_ptr<int32_t>(c, c->L.lens);
  int32_t* bt = ws_ptr<int32_t>(c, c->L.bt);
  float* h = ws_ptr<float>(c, c->L.h);
  uint16_t* x = ws_ptr<uint16_t>(c, c->L.x);
  float* q = ws_ptr<float>(c, c->L.q);
  uint16_t* o = ws_ptr<uint16_t>(c, c->L.o);
  const int d = g.d_model, dh = g.d_head, Hq = g.n_q_heads, Hkv = g.n_kv_heads;
  hipError_t e;

  dec::NormParams np{};
  np.h = h;
  np.h_out = h;
  np.x = x;
  np.d = d;
  np.Bp = Bp;
  np.eps = g.rms_eps;
  np.E = c->embed.w;
  np.E_scale = c->embed.scale;
  np.ids = ids;
  np.gain = g.n_layers > 0 ? c->attn_norm : c->final_norm;
  if ((e = dec::launch_embed_norm(np, wfp8, s)) != hipSuccess) return e;

  dec::AttnParams ap{};
  ap.q = q;
  ap.pool = c->pool;
  ap.seq_lens = lens;
  ap.bt = bt;
  ap.part_o = ws_ptr<float>(c, c->L.part_o);
  ap.part_ml = ws_ptr<float>(c, c->L.part_ml);
  ap.o = o;
  ap.Bp = Bp;
  ap.Hq = Hq;
  ap.Hkv = Hkv;
  ap.dh = dh;
  ap.num_blocks = g.num_blocks;
  ap.bps = bps;
  ap.n_split = n_split_for(g, Bp);
  ap.mfma = attn_mfma(g, Bp) ? 1 : 0;
  ap.cnt = ws_ptr<unsigned>(c, c->L.attn_cnt);

  // the matrix-vector kernels normalize their own input (no RMSNorm kernels)
  const bool fn = fused_norm(g, Bp);
  const bool fqa = fuse_qkv_attn(c, Bp);
  if (fqa) {
    unsigned* ready = ws_ptr<unsigned>(c, c->L.ready);
    ap.ready = ready;
    ap.ready_target = dec::qkv_attn_ready_target(Hq, Hkv, dh);
    ap.err_dev = ws_ptr<unsigned>(c, c->L.err);
    ap.err_host = c->err_host_dev;
    ap.timeout_ticks = c->timeout_ticks;
  }
  // no RMSNorm kernels: the matrix-vector kernels normalize their own input (fn), or the
  // MFMA products fold the norms (fold)
  const bool nk = !fn && !fold_norm(g, Bp);
  for (int l = 0; l < g.n_layers; ++l) {
    const float* an = c->attn_norm + (size_t)l * d;
    if (l > 0 && nk) {
      np.gain = an;
      if ((e = dec::launch_rmsnorm(np, s)) != hipSuccess) return e;
    }
    ap.layer = l;
    if (fqa) {
      // [q; k; v] = W_qkv RMSNorm(h) g_attn with RoPE and the cache write, and attention
      // over positions 0..p, in one kernel
      int epi = 0;
      dec::MatmulParams mp = matmul_params(c, DEC_MAT_QKV, l, Bp, &epi);
      mp.nh = h;
      mp.ng = an;
      mp.eps = g.rms_eps;
      if ((e = dec::launch_qkv_attn(mp, ap, wfp8, kvfp8, s)) != hipSuccess) return e;
    } else {
      if ((e = run_matmul(c, DEC_MAT_QKV, l, Bp, s, fn ? an : nullptr)) != hipSuccess) return e;
      // attention over positions 0..p
      if ((e = dec::launch_attention(ap, kvfp8, s)) != hipSuccess) return e;
    }
    if ((e = run_matmul(c, DEC_MAT_O, l, Bp, s)) != hipSuccess) return e;
    // x = RMSNorm(h) g_mlp
    const float* mn = c->mlp_norm + (size_t)l * d;
    if (nk) {
      np.gain = mn;
      if ((e = dec::launch_rmsnorm(np, s)) != hipSuccess) return e;
    }
    if ((e = run_matmul(c, DEC_MAT_GATE_UP, l, Bp, s, fn ? mn : nullptr)) != hipSuccess) return e;
    if ((e = run_matmul(c, DEC_MAT_DOWN, l, Bp, s)) != hipSuccess) return e;
  }
  if (g.n_layers > 0 && nk) {
    np.gain = c->final_norm;
    if ((e = dec::launch_rmsnorm(np, s)) != hipSuccess) return e;
  }
  if ((e = run_matmul(c, DEC_MAT_LM_HEAD, 0, Bp, s, fn ? c->final_norm : nullptr)) != hipSuccess) return e;
  return hipSuccess;
}

void drop_graphs(dec_ctx* c) {
  for (auto& row : c->graphs)
    for (auto& ge : row)
      if (ge) {
        (void)hipGraphExecDestroy(ge);
        ge = nullptr;
      }
}

int capture(dec_ctx* c, int bi, int mode) {
  hipGraph_t graph = nullptr;
  HIPCHK(c, hipStreamBeginCapture(c->cap_stream, hipStreamCaptureModeThreadLocal), "hipStreamBeginCapture");
  hipError_t e = enqueue_step(c, LADDER[bi], c->cap_stream);
  hipError_t e2 = hipStreamEndCapture(c->cap_stream, &graph);
  if (e != hipSuccess) {
    if (graph) (void)hipGraphDestroy(graph);
    return hip_fail(c, e, "kernel launch during capture");
  }
  if (e2 != hipSuccess) return hip_fail(c, e2, "hipStreamEndCapture");
  hipGraphExec_t exec = nullptr;
  e = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0);
  (void)hipGraphDestroy(graph);
  if (e != hipSuccess) return hip_fail(c, e, "hipGraphInstantiate");
  c->graphs[bi][mode] = exec;
  return DEC_OK;
}

int check_mat(const dec_mat& m, bool fp8, const char* name, int layer) {
  if (!m.w) return fail(DEC_E_INVALID, "%s[%d].w is NULL", name, layer);
  if (!aligned16(m.w)) return fail(DEC_E_INVALID, "%s[%d].w is not 16-byte aligned", name, layer);
  if (fp8 && !m.scale) return fail(DEC_E_INVALID, "%s[%d].scale is NULL for E4M3 weights", name, layer);
  if (!fp8 && m.scale) return fail(DEC_E_INVALID, "%s[%d].scale must be NULL for bf16 weights", name, layer);
  return DEC_OK;
}

}  // namespace

extern "C" {

const char* dec_last_error(void) { return g_err.c_str(); }

size_t dec_workspace_bytes(const dec_config* cfg) {
  if (validate_config(cfg) != DEC_OK) return 0;
  return layout_of(*cfg).total;
}

int dec_create(const dec_config* cfg, void* hip_stream, void* kv_pool, void* workspace, size_t workspace_bytes,
               float* logits, dec_ctx** out) {
  if (!out) return fail(DEC_E_INVALID, "out is NULL");
  *out = nullptr;
  int rc = validate_config(cfg);
  if (rc != DEC_OK) return rc;
  if (!kv_pool || !workspace || !logits) return fail(DEC_E_INVALID, "kv_pool, workspace and logits must be non-NULL");
  if (!aligned16(kv_pool) || !aligned16(logits)) return fail(DEC_E_INVALID, "kv_pool and logits must be 16-byte aligned");
  if (((uintptr_t)workspace & 255u) != 0) return fail(DEC_E_INVALID, "workspace must be 256-byte aligned");
  const Layout L = layout_of(*cfg);
  if (workspace_bytes < L.total)
    return fail(DEC_E_INVALID, "workspace has %zu bytes, needs %zu", workspace_bytes, L.total);

  dec_ctx* c = new dec_ctx();
  c->cfg = *cfg;
  c->stream = static_cast<hipStream_t>(hip_stream);
  c->pool = kv_pool;
  c->ws = static_cast<uint8_t*>(workspace);
  c->logits = logits;
  c->L = L;
  hipError_t e;
  if ((e = hipGetDevice(&c->device)) != hipSuccess || (e = hipStreamCreateWithFlags(&c->cap_stream, hipStreamNonBlocking)) != hipSuccess) {
    rc = hip_fail(nullptr, e, "dec_create: device / capture stream");
    delete c;
    return rc;
  }
  int wall_khz = 0;
  if ((e = hipDeviceGetAttribute(&c->n_cu, hipDeviceAttributeMultiprocessorCount, c->device)) != hipSuccess ||
      (e = hipHostMalloc(reinterpret_cast<void**>(&c->err_host), 64, hipHostMallocMapped)) != hipSuccess ||
      (e = hipHostGetDevicePointer(reinterpret_cast<void**>(&c->err_host_dev), c->err_host, 0)) != hipSuccess) {
    rc = hip_fail(nullptr, e, "dec_create: device attributes / error word");
    dec_destroy(c);
    return rc;
  }
  *reinterpret_cast<volatile unsigned*>(c->err_host) = 0u;
  if (hipDeviceGetAttribute(&wall_khz, hipDeviceAttributeWallClockRate, c->device) != hipSuccess || wall_khz <= 0)
    wall_khz = 100000;  // the s_memrealtime counter runs at 100 MHz on this family
  c->timeout_ticks = (uint64_t)((double)wall_khz * 1e3 * BARRIER_TIMEOUT_S);
  for (int i = 0; i < 2; ++i) {
    if ((e = hipHostMalloc(reinterpret_cast<void**>(&c->pinned[i]), L.static_bytes, hipHostMallocDefault)) != hipSuccess ||
        (e = hipEventCreateWithFlags(&c->slot_ev[i], hipEventDisableTiming)) != hipSuccess) {
      rc = hip_fail(nullptr, e, "dec_create: pinned staging");
      dec_destroy(c);
      return rc;
    }
    std::memset(c->pinned[i], 0, L.static_bytes);
  }
  // RoPE table once; static region starts zeroed (ids 0, every row padded until set)
  if ((e = dec::launch_rope_table(ws_ptr<float2>(c, L.rope), cfg->max_seq_len, cfg->d_head, (double)cfg->rope_theta,
                                  c->stream)) != hipSuccess ||
      (e = hipMemsetAsync(c->ws, 0, L.static_bytes, c->stream)) != hipSuccess ||
      (e = hipMemsetAsync(c->ws + L.bar, 0, L.total - L.bar, c->stream)) != hipSuccess ||
      (e = hipStreamSynchronize(c->stream)) != hipSuccess) {
    rc = hip_fail(nullptr, e, "dec_create: initialising the workspace");
    dec_destroy(c);
    return rc;
  }
  c->info.flags = cfg->flags;
  *out = c;
  return DEC_OK;
}

int dec_load_weights(dec_ctx* c, const dec_weights* w) {
  if (!c || !w) return fail(DEC_E_INVALID, "ctx or weights is NULL");
  if (c->failed) return fail(DEC_E_STATE, "context has failed; destroy it");
  const dec_config& g = c->cfg;
  const bool fp8 = g.weight_dtype == DEC_FP8_E4M3;
  int rc;
  if ((rc = check_mat(w->embed, fp8, "embed", 0)) != DEC_OK) return rc;
  if ((rc = check_mat(w->lm_head, fp8, "lm_head", 0)) != DEC_OK) return rc;
  if (!w->final_norm) return fail(DEC_E_INVALID, "final_norm is NULL");
  if (g.n_layers > 0) {
    if (!w->attn_norm || !w->mlp_norm || !w->qkv || !w->o || !w->gate_up || !w->down)
      return fail(DEC_E_INVALID, "per-layer weight arrays must be non-NULL");
    for (int l = 0; l < g.n_layers; ++l) {
      if ((rc = check_mat(w->qkv[l], fp8, "qkv", l)) != DEC_OK || (rc = check_mat(w->o[l], fp8, "o", l)) != DEC_OK ||
          (rc = check_mat(w->gate_up[l], fp8, "gate_up", l)) != DEC_OK ||
          (rc = check_mat(w->down[l], fp8, "down", l)) != DEC_OK)
        return rc;
    }
  }
  drop_graphs(c);
  c->embed = w->embed;
  c->lm = w->lm_head;
  c->attn_norm = w->attn_norm;
  c->mlp_norm = w->mlp_norm;
  c->final_norm = w->final_norm;
  c->qkv.assign(w->qkv, w->qkv + g.n_layers);
  c->o.assign(w->o, w->o + g.n_layers);
  c->gu.assign(w->gate_up, w->gate_up + g.n_layers);
  c->down.assign(w->down, w->down + g.n_layers);
  // device copies of the per-layer pointers for the persistent step
  if (g.n_layers > 0) {
    std::vector<dec::DevMat> host(4 * (size_t)g.n_layers);
    for (int l = 0; l < g.n_layers; ++l) {
      host[l] = dec::DevMat{c->qkv[l].w, c->qkv[l].scale};
      host[g.n_layers + l] = dec::DevMat{c->o[l].w, c->o[l].scale};
      host[2 * g.n_layers + l] = dec::DevMat{c->gu[l].w, c->gu[l].scale};
      host[3 * g.n_layers + l] = dec::DevMat{c->down[l].w, c->down[l].scale};
    }
    hipError_t e = hipMemcpyAsync(c->ws + c->L.mats, host.data(), host.size() * sizeof(dec::DevMat),
                                  hipMemcpyHostToDevice, c->stream);
    if (e == hipSuccess) e = hipStreamSynchronize(c->stream);
    if (e != hipSuccess) return hip_fail(c, e, "dec_load_weights: uploading layer pointers");
  }
  c->loaded = true;
  c->info.graphs_captured = 0;
  return DEC_OK;
}

int dec_set_flags(dec_ctx* c, uint32_t flags) {
  if (!c) return fail(DEC_E_INVALID, "ctx is NULL");
  if (flags & ~KNOWN_FLAGS) return fail(DEC_E_INVALID, "unknown flag bits 0x%x", flags & ~KNOWN_FLAGS);
  c->cfg.flags = flags;
  c->info.flags = flags;
  return DEC_OK;
}

int dec_step(dec_ctx* c, const dec_step_args* a) {
  if (!c || !a) return fail(DEC_E_INVALID, "ctx or args is NULL");
  if (c->failed) return fail(DEC_E_STATE, "context has failed; destroy it");
  if (!c->loaded) return fail(DEC_E_STATE, "dec_step before dec_load_weights");
  if (*reinterpret_cast<volatile unsigned*>(c->err_host) != 0u) {
    c->failed = true;
    return fail(DEC_E_HIP, "a bounded wait of an earlier step (grid barrier or attention wait) timed out; "
                            "the context is unusable");
  }
  const dec_config& g = c->cfg;
  const int n = a->n_seqs;
  if (n < 1) return fail(DEC_E_INVALID, "n_seqs must be >= 1 (got %d)", n);
  if (n > g.max_batch) return fail(DEC_E_CAPACITY, "n_seqs %d exceeds max_batch %d", n, g.max_batch);
  if (!a->token_ids || !a->seq_lens || !a->block_tables)
    return fail(DEC_E_INVALID, "token_ids, seq_lens and block_tables must be non-NULL");
  const int bps = blocks_per_seq(g);
  for (int b = 0; b < n; ++b) {
    const int t = a->token_ids[b], p = a->seq_lens[b];
    if (t < 0 || t >= g.vocab) return fail(DEC_E_INVALID, "token_ids[%d] = %d outside [0, %d)", b, t, g.vocab);
    if (p < 0) return fail(DEC_E_INVALID, "seq_lens[%d] = %d is negative", b, p);
    if (p >= g.max_seq_len) return fail(DEC_E_CAPACITY, "seq_lens[%d] = %d: position must be < max_seq_len %d", b, p, g.max_seq_len);
    for (int k = 0; k <= p / 16; ++k) {
      const int blk = a->block_tables[(size_t)b * bps + k];
      if (blk < 0 || blk >= g.num_blocks)
        return fail(DEC_E_CAPACITY, "block_tables[%d][%d] = %d outside [0, %d)", b, k, blk, g.num_blocks);
    }
  }
  const int bi = bucket_index(n);
  const int Bp = LADDER[bi];

  // stage into the pinned slot (wait until the copy that last used it has finished)
  const int s = c->slot;
  c->slot ^= 1;
  if (c->slot_pending[s]) HIPCHK(c, hipEventSynchronize(c->slot_ev[s]), "waiting for a staging slot");
  uint8_t* st = c->pinned[s];
  int32_t* ids = reinterpret_cast<int32_t*>(st + c->L.ids);
  int32_t* lens = reinterpret_cast<int32_t*>(st + c->L.lens);
  int32_t* bt = reinterpret_cast<int32_t*>(st + c->L.bt);
  std::memcpy(ids, a->token_ids, (size_t)n * 4);
  std::memcpy(lens, a->seq_lens, (size_t)n * 4);
  std::memcpy(bt, a->block_tables, (size_t)n * bps * 4);
  for (int b = n; b < Bp; ++b) {  // padded rows: token 0, position -1 (no cache write, no attention)
    ids[b] = 0;
    lens[b] = -1;
    std::memset(bt + (size_t)b * bps, 0, (size_t)bps * 4);
  }
  HIPCHK(c, hipMemcpyAsync(c->ws, st, c->L.static_bytes, hipMemcpyHostToDevice, c->stream), "staging copy");
  HIPCHK(c, hipEventRecord(c->slot_ev[s], c->stream), "hipEventRecord");
  c->slot_pending[s] = true;

  const int mode = mode_of(g.flags);
  if (g.flags & DEC_FLAG_EAGER) {
    hipError_t e = enqueue_step(c, Bp, c->stream);
    if (e != hipSuccess) return hip_fail(c, e, "kernel launch");
    c->info.used_graph = 0;
  } else {
    if (g.flags & DEC_FLAG_CAPTURE_ALL) {
      for (int i = 0; i < N_BUCKETS && LADDER[i] <= g.max_batch; ++i)
        if (!c->graphs[i][mode]) {
          int rc = capture(c, i, mode);
          if (rc != DEC_OK) return rc;
        }
    }
    if (!c->graphs[bi][mode]) {
      int rc = capture(c, bi, mode);
      if (rc != DEC_OK) return rc;
    }
    HIPCHK(c, hipGraphLaunch(c->graphs[bi][mode], c->stream), "hipGraphLaunch");
    c->info.used_graph = 1;
  }
  int ncap = 0;
  for (auto& row : c->graphs)
    for (auto& ge : row) ncap += ge != nullptr;
  const bool persist = use_persistent(c, Bp);
  const bool mfma = !persist && use_mfma(g, Bp);
  const int slices = (!mfma && Bp > 8) ? Bp / 8 : 1;
  const int L = g.n_layers;
  // per layer: QKV, attention, O, gate+up, down, and two RMSNorm kernels unless the
  // matrix-vector kernels fuse them or the MFMA products fold them (and QKV + attention
  // as one kernel where fuse_qkv_attn holds); unfused: also RoPE + KV write, SiLU x mul
  // and two residual adds
  const bool unfused = (g.flags & DEC_FLAG_UNFUSED) != 0;
  const int per_layer = unfused ? 11 : fuse_qkv_attn(c, Bp) ? 4 : fused_norm(g, Bp) || fold_norm(g, Bp) ? 5 : 7;
  c->info.kernels_per_step = persist ? 1 : 2 + per_layer * L + (slices - 1) * (4 * L + 1);
  c->info.bucket = Bp;
  c->last_n = n;
  c->info.attn_splits = persist ? n_split_persistent(g, Bp) : n_split_for(g, Bp);
  c->info.used_mfma = mfma ? 1 : 0;
  c->info.persistent = persist ? 1 : 0;
  c->info.graphs_captured = ncap;
  c->info.flags = g.flags;
  return DEC_OK;
}

int dec_launch_matmul(dec_ctx* c, int which, int layer) {
  if (!c) return fail(DEC_E_INVALID, "ctx is NULL");
  if (c->failed) return fail(DEC_E_STATE, "context has failed; destroy it");
  if (!c->loaded || c->info.bucket == 0) return fail(DEC_E_STATE, "dec_launch_matmul needs a previous dec_step");
  if (which < DEC_MAT_O || which > DEC_MAT_LM_HEAD)
    return fail(DEC_E_INVALID, "which must be DEC_MAT_O, DEC_MAT_GATE_UP, DEC_MAT_DOWN or DEC_MAT_LM_HEAD");
  if (which != DEC_MAT_LM_HEAD && (layer < 0 || layer >= c->cfg.n_layers))
    return fail(DEC_E_INVALID, "layer %d outside [0, %d)", layer, c->cfg.n_layers);
  // the same kernel as in the step: a fused RMSNorm where the step fuses it
  const float* ng = nullptr;
  if (fused_norm(c->cfg, c->info.bucket)) {
    if (which == DEC_MAT_GATE_UP) ng = c->mlp_norm + (size_t)layer * c->cfg.d_model;
    if (which == DEC_MAT_LM_HEAD) ng = c->final_norm;
  }
  hipError_t e = run_matmul(c, which, which == DEC_MAT_LM_HEAD ? 0 : layer, c->info.bucket, c->stream, ng);
  if (e != hipSuccess) return hip_fail(c, e, "kernel launch");
  return DEC_OK;
}

int dec_sample_greedy(dec_ctx* c, int32_t* token_ids) {
  if (!c || !token_ids) return fail(DEC_E_INVALID, "ctx or token_ids is NULL");
  if (((uintptr_t)token_ids & 3u) != 0) return fail(DEC_E_INVALID, "token_ids is not 4-byte aligned");
  if (c->failed) return fail(DEC_E_STATE, "context has failed; destroy it");
  if (!c->loaded || c->last_n <= 0) return fail(DEC_E_STATE, "dec_sample_greedy needs a previous dec_step");
  hipError_t e = dec::launch_argmax(c->logits, c->cfg.vocab, c->cfg.vocab, c->last_n, token_ids, c->stream);
  if (e != hipSuccess) return hip_fail(c, e, "kernel launch");
  return DEC_OK;
}

int dec_sample(dec_ctx* c, const float* uniforms, float temperature, int32_t top_k, float top_p,
               int32_t* token_ids) {
  if (!c || !token_ids || !uniforms) return fail(DEC_E_INVALID, "ctx, uniforms or token_ids is NULL");
  if (((uintptr_t)token_ids & 3u) != 0 || ((uintptr_t)uniforms & 3u) != 0)
    return fail(DEC_E_INVALID, "token_ids or uniforms is not 4-byte aligned");
  if (!(temperature > 0.f) || !std::isfinite(temperature))
    return fail(DEC_E_INVALID, "temperature must be positive and finite");
  if (top_k < 1 || top_k > dec::SAMPLE_MAX_K)
    return fail(DEC_E_INVALID, "top_k must be in [1, %d] (got %d)", dec::SAMPLE_MAX_K, top_k);
  if (!(top_p > 0.f) || top_p > 1.f) return fail(DEC_E_INVALID, "top_p must be in (0, 1]");
  if (c->failed) return fail(DEC_E_STATE, "context has failed; destroy it");
  if (!c->loaded || c->last_n <= 0) return fail(DEC_E_STATE, "dec_sample needs a previous dec_step");
  hipError_t e = dec::launch_sample_topkp(c->logits, c->cfg.vocab, c->cfg.vocab, c->last_n, uniforms, temperature,
                                          top_k, top_p, token_ids, c->stream);
  if (e != hipSuccess) return hip_fail(c, e, "kernel launch");
  return DEC_OK;
}

int dec_get_info(const dec_ctx* c, dec_info* out) {
  if (!c || !out) return fail(DEC_E_INVALID, "ctx or out is NULL");
  *out = c->info;
  return DEC_OK;
}

int dec_destroy(dec_ctx* c) {
  if (!c) return DEC_OK;
  int rc = DEC_OK;
  if (c->stream || c->cap_stream) {
    hipError_t e = hipStreamSynchronize(c->stream);
    if (e != hipSuccess) rc = fail(DEC_E_HIP, "dec_destroy: %s", hipGetErrorString(e));
  }
  drop_graphs(c);
  for (int i = 0; i < 2; ++i) {
    if (c->slot_ev[i]) (void)hipEventDestroy(c->slot_ev[i]);
    if (c->pinned[i]) (void)hipHostFree(c->pinned[i]);
  }
  if (c->cap_stream) (void)hipStreamDestroy(c->cap_stream);
  if (c->err_host) (void)hipHostFree(c->err_host);
  delete c;
  return rc;
}

int dec_bw_probe(const void* buf, size_t bytes, int reps, void* hip_stream, double* out) {
  if (!buf || !out || reps < 1 || bytes < 16 || bytes % 16 || !aligned16(buf))
    return fail(DEC_E_INVALID, "dec_bw_probe: need a 16-byte aligned buffer, bytes a positive multiple of 16, reps >= 1");
  hipStream_t s = static_cast<hipStream_t>(hip_stream);
  hipEvent_t e0 = nullptr, e1 = nullptr;
  hipError_t e;
  double best = 0.0;
  if ((e = hipEventCreate(&e0)) != hipSuccess || (e = hipEventCreate(&e1)) != hipSuccess) goto done;
  for (int r = 0; r < reps + 1; ++r) {
    if ((e = hipEventRecord(e0, s)) != hipSuccess) goto done;
    if ((e = dec::launch_bw_probe(buf, bytes, nullptr, s)) != hipSuccess) goto done;
    if ((e = hipEventRecord(e1, s)) != hipSuccess) goto done;
    if ((e = hipEventSynchronize(e1)) != hipSuccess) goto done;
    float ms = 0.f;
    if ((e = hipEventElapsedTime(&ms, e0, e1)) != hipSuccess) goto done;
    if (r > 0 && ms > 0.f && bytes / (ms * 1e-3) > best) best = bytes / (ms * 1e-3);  // first run warms up
  }
done:
  if (e0) (void)hipEventDestroy(e0);
  if (e1) (void)hipEventDestroy(e1);
  if (e != hipSuccess) return fail(DEC_E_HIP, "dec_bw_probe: %s", hipGetErrorString(e));
  *out = best;
  return DEC_OK;
}

}  // extern "C"
