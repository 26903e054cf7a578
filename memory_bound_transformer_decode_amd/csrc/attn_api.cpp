// The attention step of decode as a call of its own: split-K paged GQA attention of
// query rows over a paged KV cache, with the caller's workspace (dec_attention) or a
// statically allocated scratch area (dec_attention_noalloc, for callers that cannot
// allocate device memory).
//
// Exact softmax attention computed tile by tile over a paged cache (FlashAttention and
// PagedAttention as cited by "GPU Inference Internals", Kernels: FlashAttention and the
// Memory Hierarchy); the same kernels as the attention of dec_step.

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>

#include "dec.h"
#include "kernels.h"

namespace {

// Scratch of dec_attention_noalloc: attention partials and split counters, one copy per
// GPU the library runs on, held until the process ends.  Host code never uses the
// array's name as an address: each device's address comes from hipGetSymbolAddress.
constexpr size_t NOALLOC_SCRATCH_BYTES = DEC_ATTN_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[NOALLOC_SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[MAX_DEVICES] = {};

int afail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  dec::set_last_error(buf);
  return code;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int check_desc(const dec_attn_desc* d) {
  if (!d) return afail(DEC_E_INVALID, "attention descriptor is NULL");
  if (d->n_rows < 1 || d->n_rows > DEC_ATTN_MAX_ROWS)
    return afail(DEC_E_INVALID, "n_rows must be in [1, %d] (got %d)", DEC_ATTN_MAX_ROWS, d->n_rows);
  if (d->n_kv_heads <= 0 || d->n_q_heads <= 0 || d->n_q_heads % d->n_kv_heads)
    return afail(DEC_E_INVALID, "n_q_heads (%d) must be a positive multiple of n_kv_heads (%d)", d->n_q_heads,
                 d->n_kv_heads);
  if (d->n_q_heads / d->n_kv_heads > 8)
    return afail(DEC_E_UNSUPPORTED, "query heads per KV head must be <= 8 (got %d)", d->n_q_heads / d->n_kv_heads);
  if (d->d_head != 64 && d->d_head != 128) return afail(DEC_E_UNSUPPORTED, "d_head must be 64 or 128 (got %d)", d->d_head);
  if (d->kv_dtype != DEC_BF16 && d->kv_dtype != DEC_FP8_E4M3)
    return afail(DEC_E_INVALID, "kv_dtype must be DEC_BF16 or DEC_FP8_E4M3");
  if (d->num_blocks <= 0 || d->n_layers <= 0 || d->layer < 0 || d->layer >= d->n_layers)
    return afail(DEC_E_INVALID, "need num_blocks > 0 and 0 <= layer < n_layers (got %d, %d, %d)", d->num_blocks,
                 d->layer, d->n_layers);
  if (d->max_blocks_per_seq <= 0 || d->max_blocks_per_seq > dec::ATTN_MAX_SPLIT * dec::ATTN_WAVES * 64)
    return afail(DEC_E_UNSUPPORTED, "max_blocks_per_seq must be in [1, %d] (got %d)",
                 dec::ATTN_MAX_SPLIT * dec::ATTN_WAVES * 64, d->max_blocks_per_seq);
  return DEC_OK;
}

dec::AttnShape shape_of(const dec_attn_desc* d) {
  return dec::AttnShape{d->n_q_heads, d->n_kv_heads, d->d_head, d->max_blocks_per_seq};
}

int check_ptrs(const float* q, const void* kv_pool, const int32_t* seq_lens, const int32_t* block_tables,
               const uint16_t* o) {
  if (!q || !kv_pool || !seq_lens || !block_tables || !o)
    return afail(DEC_E_INVALID, "q, kv_pool, seq_lens, block_tables and o must be non-NULL");
  if (!aligned16(q) || !aligned16(kv_pool) || !aligned16(o) || ((uintptr_t)seq_lens & 3u) ||
      ((uintptr_t)block_tables & 3u))
    return afail(DEC_E_INVALID, "q, kv_pool and o must be 16-byte aligned, seq_lens and block_tables 4-byte aligned");
  return DEC_OK;
}

// Clear the split counters, then run the attention kernel, with the scratch at `ws`.
int enqueue(const dec_attn_desc* d, const float* q, const void* kv_pool, const int32_t* seq_lens,
            const int32_t* block_tables, uint16_t* o, uint8_t* ws, hipStream_t s) {
  const dec::AttnShape sh = shape_of(d);
  const dec::AttnScratch sc = dec::attn_scratch(sh, d->n_rows);
  dec::AttnParams p{};
  p.q = q;
  p.pool = kv_pool;
  p.layer = d->layer;
  p.seq_lens = seq_lens;
  p.bt = block_tables;
  p.part_o = reinterpret_cast<float*>(ws + sc.part_o);
  p.part_ml = reinterpret_cast<float*>(ws + sc.part_ml);
  p.o = o;
  p.cnt = reinterpret_cast<unsigned*>(ws + sc.cnt);
  p.Bp = d->n_rows;
  p.Hq = d->n_q_heads;
  p.Hkv = d->n_kv_heads;
  p.dh = d->d_head;
  p.num_blocks = d->num_blocks;
  p.bps = d->max_blocks_per_seq;
  p.n_split = dec::attn_splits(sh, d->n_rows);
  p.mfma = 1;
  hipError_t e = dec::launch_zero_u32(p.cnt, d->n_rows * d->n_kv_heads, s);
  if (e == hipSuccess) e = dec::launch_attention(p, d->kv_dtype == DEC_FP8_E4M3, s);
  if (e != hipSuccess) return afail(DEC_E_HIP, "attention launch: %s", hipGetErrorString(e));
  return DEC_OK;
}

}  // namespace

extern "C" {

size_t dec_attention_workspace_bytes(const dec_attn_desc* d) {
  if (check_desc(d) != DEC_OK) return 0;
  return dec::attn_scratch(shape_of(d), d->n_rows).total;
}

int dec_attention(const dec_attn_desc* d, const float* q, const void* kv_pool, const int32_t* seq_lens,
                  const int32_t* block_tables, uint16_t* o, void* workspace, size_t workspace_bytes,
                  void* hip_stream) {
  int rc = check_desc(d);
  if (rc != DEC_OK) return rc;
  if ((rc = check_ptrs(q, kv_pool, seq_lens, block_tables, o)) != DEC_OK) return rc;
  const size_t need = dec::attn_scratch(shape_of(d), d->n_rows).total;
  if (!workspace || ((uintptr_t)workspace & 255u))
    return afail(DEC_E_INVALID, "workspace must be non-NULL and 256-byte aligned");
  if (workspace_bytes < need) return afail(DEC_E_INVALID, "workspace has %zu bytes, needs %zu", workspace_bytes, need);
  return enqueue(d, q, kv_pool, seq_lens, block_tables, o, static_cast<uint8_t*>(workspace),
                 static_cast<hipStream_t>(hip_stream));
}

int dec_attention_noalloc(const dec_attn_desc* d, const float* q, const void* kv_pool, const int32_t* seq_lens,
                          const int32_t* block_tables, uint16_t* o, void* hip_stream) {
  int rc = check_desc(d);
  if (rc != DEC_OK) return rc;
  if ((rc = check_ptrs(q, kv_pool, seq_lens, block_tables, o)) != DEC_OK) return rc;
  const size_t need = dec::attn_scratch(shape_of(d), d->n_rows).total;
  if (need > NOALLOC_SCRATCH_BYTES)
    return afail(DEC_E_CAPACITY, "this shape needs %zu bytes of scratch; the static area holds %zu", need,
                 NOALLOC_SCRATCH_BYTES);
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return afail(DEC_E_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= MAX_DEVICES) return afail(DEC_E_UNSUPPORTED, "device %d beyond %d", dev, MAX_DEVICES);
  void* ptr = nullptr;
  {
    // the device's own address of its copy of the array, looked up once per device
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
      e = hipGetSymbolAddress(&g_scratch_ptr[dev], HIP_SYMBOL(scratch));
      if (e != hipSuccess) {
        g_scratch_ptr[dev] = nullptr;
        return afail(DEC_E_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
      }
    }
    ptr = g_scratch_ptr[dev];
  }
  return enqueue(d, q, kv_pool, seq_lens, block_tables, o, static_cast<uint8_t*>(ptr),
                 static_cast<hipStream_t>(hip_stream));
}

}  // extern "C"
