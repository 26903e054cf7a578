// Device helpers shared by the decode-step kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace dec {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int WAVE = 64;
constexpr int KV_BLOCK = 16;  // positions per paged KV block

// ---------------------------------------------------------------- loads

// Global-memory accesses through pointers the compiler cannot place (read from
// memory, or passed around generically) would become flat instructions, which also
// count against the LDS counter and so make every LDS read wait for in-flight global
// loads.  These helpers address global memory explicitly.
#define DEC_GLOBAL __attribute__((address_space(1)))

template <typename T>
__device__ __forceinline__ T gld(const T* p) { return *(const DEC_GLOBAL T*)p; }
template <typename T>
__device__ __forceinline__ void gst(T* p, T v) { *(DEC_GLOBAL T*)p = v; }

// Weights are read exactly once per step: stream them past the caches.
__device__ __forceinline__ u32x4 ld_stream(const u32x4* p) { return __builtin_nontemporal_load((const DEC_GLOBAL u32x4*)p); }
// 16 bytes from global memory
__device__ __forceinline__ u32x4 gld16(const void* p) { return gld(reinterpret_cast<const u32x4*>(p)); }
// 16 bytes from LDS or global memory (the caller's pointer decides)
__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

// Data one work group writes and another work group of the same kernel reads (attention
// partials, the split products' partial tiles) goes through device-coherent accesses:
// each L2 (one per XCD) is not coherent with the others, so these stores write through
// it and these loads bypass it.  The reader learns that the data is there from an
// arrival counter (see arrive_after_stores).
template <typename T>
__device__ __forceinline__ T cld(const T* p) { return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
template <typename T>
__device__ __forceinline__ void cst(T* p, T v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
__device__ __forceinline__ u32x4 cld16(const void* p) {
  const uint64_t* q = static_cast<const uint64_t*>(p);
  const uint64_t a = cld(q), b = cld(q + 1);
  return u32x4{(uint32_t)a, (uint32_t)(a >> 32), (uint32_t)b, (uint32_t)(b >> 32)};
}
__device__ __forceinline__ void cst_f2(float* p, float x, float y) {
  cst(reinterpret_cast<uint64_t*>(p), (uint64_t)__float_as_uint(x) | ((uint64_t)__float_as_uint(y) << 32));
}
__device__ __forceinline__ void cst_f4(float* p, float x, float y, float z, float w) {
  cst_f2(p, x, y);
  cst_f2(p + 2, z, w);
}
__device__ __forceinline__ f32x4 cld_f4(const float* p) {
  const u32x4 v = cld16(p);
  return f32x4{__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z), __uint_as_float(v.w)};
}

// Count this work group's arrival at *cnt once every thread's device-coherent stores
// have completed.  Returns, in every thread, whether this work group is the last of n
// to arrive; the last one resets the counter to zero for the next launch.
//
// Why the last arriver sees every other work group's stores:
//  1. each thread waits until its own stores are acknowledged (vmcnt(0): on this family
//     the vector-memory counter also counts stores, and a device-coherent store is
//     acknowledged once it has reached the memory side that every XCD shares).  The
//     compiler-only fences on both sides of the wait keep the compiler from moving the
//     atomic stores below it or the counter update above it;
//  2. the work-group barrier orders every thread's wait before thread 0's update;
//  3. the update is one agent-scope atomic add, so the work group that reads n - 1 has
//     seen the n - 1 earlier updates, each made after its work group's stores completed;
//  4. the last arriver then reads with device-coherent loads, which bypass the
//     non-coherent L2 and cannot return a stale line.
// `flag`: one int of LDS.
__device__ __forceinline__ bool arrive_after_stores(unsigned* cnt, unsigned n, int* flag) {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0), expcnt and lgkmcnt not waited on
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned prev = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const bool last = prev == n - 1;
    *flag = last;
    if (last) cst(cnt, 0u);  // ready for the next launch
  }
  __syncthreads();
  return *flag != 0;
}

// ---------------------------------------------------------------- number formats

// bf16 bits -> fp32 (exact)
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// fp32 -> bf16 bits, round to nearest even (NaN stays a quiet NaN)
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// fp32 -> fp16 bits, round to nearest even; magnitudes beyond the largest finite fp16
// (65504) saturate to it (NaN stays NaN)
__device__ __forceinline__ uint16_t f32_to_f16(float f) {
  const float c = __builtin_fminf(__builtin_fmaxf(f, -65504.0f), 65504.0f);
  return __builtin_bit_cast(uint16_t, (_Float16)(f != f ? f : c));
}

// fp32 -> OCP E4M3 code: round to nearest even, finite values saturate to +-448.
__device__ __forceinline__ uint32_t f32_to_e4m3(float f) {
  uint32_t u = __float_as_uint(f);
  uint32_t sign = (u >> 24) & 0x80u;
  uint32_t a = u & 0x7FFFFFFFu;
  if (a > 0x7F800000u) return sign | 0x7Fu;           // NaN
  float af = __uint_as_float(a);
  if (af >= 448.0f) return sign | 0x7Eu;              // saturate (incl. inf)
  if (af < 0.015625f) {                               // below 2^-6: multiples of 2^-9
    return sign | (uint32_t)__builtin_rintf(af * 512.0f);  // rint: ties to even; 8 -> 2^-6 (code 8)
  }
  uint32_t r = (a + 0x7FFFFu + ((a >> 20) & 1u)) >> 20;  // (biased exp << 3) | 3-bit mantissa, RNE
  uint32_t code = r - ((127u - 7u) << 3);
  return sign | (code > 0x7Eu ? 0x7Eu : code);
}

// two E4M3 codes (bytes 0,1 or bytes 2,3 of w) -> two bf16 (exact: E4M3 values are bf16 values)
template <bool HI>
__device__ __forceinline__ bf16x2 e4m3x2_to_bf16x2(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI);
}

// two E4M3 codes -> two fp32 (exact)
template <bool HI>
__device__ __forceinline__ f32x2 e4m3x2_to_f32x2(uint32_t w) {
  return __builtin_amdgcn_cvt_pk_f32_fp8(w, HI);
}

// two int8 codes (bytes 0,1 or bytes 2,3 of w) -> two fp32 / two bf16 (exact: |v| <= 128
// has at most 8 significant bits).  Each byte is sign-extended and converted by one
// instruction (a byte-select on the conversion's source), the pair packed by another.
template <bool HI>
__device__ __forceinline__ f32x2 i8x2_to_f32x2(uint32_t w) {
  // written so that each conversion selects its byte directly (no shifts)
  if constexpr (HI) return f32x2{(float)(int8_t)(w >> 16), (float)((int32_t)w >> 24)};
  else return f32x2{(float)(int8_t)w, (float)(int8_t)(w >> 8)};
}
template <bool HI>
__device__ __forceinline__ bf16x2 i8x2_to_bf16x2(uint32_t w) {
  const f32x2 f = i8x2_to_f32x2<HI>(w);
  return bf16x2{(__bf16)f.x, (__bf16)f.y};
}

// two one-byte codes of format WQ -> two bf16 / two fp32
template <int WQ, bool HI>
__device__ __forceinline__ bf16x2 b8x2_to_bf16x2(uint32_t w) {
  if constexpr (WQ == W_I8) return i8x2_to_bf16x2<HI>(w);
  else return e4m3x2_to_bf16x2<HI>(w);
}
template <int WQ, bool HI>
__device__ __forceinline__ f32x2 b8x2_to_f32x2(uint32_t w) {
  if constexpr (WQ == W_I8) return i8x2_to_f32x2<HI>(w);
  else return e4m3x2_to_f32x2<HI>(w);
}

// Weights as fp16 operands.  E4M3 and int8 values are fp16 values (exact).  bf16 values
// are exact in fp16 from 2^-14 to 65504 in magnitude (8 significant bits fit fp16's 11);
// smaller ones are cut to a multiple of 2^-24 (the conversion rounds toward zero), an
// absolute change below 2^-24.
__device__ __forceinline__ f16x2 bf16x2_to_f16x2(uint32_t w) {
  return __builtin_bit_cast(f16x2, __builtin_amdgcn_cvt_pkrtz(bf16_lo(w), bf16_hi(w)));
}
template <int WQ, bool HI>
__device__ __forceinline__ f16x2 b8x2_to_f16x2(uint32_t w) {
  if constexpr (WQ == W_I8) {
    const f32x2 f = i8x2_to_f32x2<HI>(w);
    return __builtin_bit_cast(f16x2, __builtin_amdgcn_cvt_pkrtz(f.x, f.y));
  } else {
    return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, HI);
  }
}

// ---------------------------------------------------------------- dot products

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b),
                                         acc, false);
}
__device__ __forceinline__ float dot2_bf16v(bf16x2 a, uint32_t b, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(a, __builtin_bit_cast(bf16x2, b), acc, false);
}

// 8 bf16 weights . 8 bf16 activations
__device__ __forceinline__ float dot8_bf16(const u32x4& w, const u32x4& x, float acc) {
  acc = dot2_bf16(w.x, x.x, acc);
  acc = dot2_bf16(w.y, x.y, acc);
  acc = dot2_bf16(w.z, x.z, acc);
  acc = dot2_bf16(w.w, x.w, acc);
  return acc;
}

// 4 one-byte weights (one u32) . 4 bf16 activations (two u32)
template <int WQ>
__device__ __forceinline__ float dot4_b8(uint32_t w, uint32_t x01, uint32_t x23, float acc) {
  acc = dot2_bf16v(b8x2_to_bf16x2<WQ, false>(w), x01, acc);
  acc = dot2_bf16v(b8x2_to_bf16x2<WQ, true>(w), x23, acc);
  return acc;
}

// 16 one-byte codes -> 16 bf16 (exact): elements 0..7 in a, 8..15 in b
template <int WQ>
__device__ __forceinline__ void widen16_b8(const u32x4& w, u32x4& a, u32x4& b) {
  const uint32_t c[4] = {w.x, w.y, w.z, w.w};
  uint32_t o[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    o[2 * i] = __builtin_bit_cast(uint32_t, b8x2_to_bf16x2<WQ, false>(c[i]));
    o[2 * i + 1] = __builtin_bit_cast(uint32_t, b8x2_to_bf16x2<WQ, true>(c[i]));
  }
  a = u32x4{o[0], o[1], o[2], o[3]};
  b = u32x4{o[4], o[5], o[6], o[7]};
}

// 16 one-byte weights . 16 bf16 activations (xa: elements 0..7, xb: 8..15)
template <int WQ>
__device__ __forceinline__ float dot16_b8(const u32x4& w, const u32x4& xa, const u32x4& xb, float acc) {
  acc = dot4_b8<WQ>(w.x, xa.x, xa.y, acc);
  acc = dot4_b8<WQ>(w.y, xa.z, xa.w, acc);
  acc = dot4_b8<WQ>(w.z, xb.x, xb.y, acc);
  acc = dot4_b8<WQ>(w.w, xb.z, xb.w, acc);
  return acc;
}

// ---------------------------------------------------------------- reductions

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Sum over aligned groups of N = 8 or 16 lanes, every lane of a group receiving the
// group's sum, with DPP lane moves inside a 16-lane row (no trip through the LDS
// crossbar that __shfl_xor takes): swap neighbours, swap pairs, mirror each half-row
// (lane i <-> 7 - i, which pairs the two quads of a half), and for 16 mirror the row
// (lane i <-> 15 - i, which pairs its two halves).  Each step adds a value that covers
// a disjoint set of lanes, and fp addition is commutative, so all lanes of a group end
// with the same bits.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
template <int N>
__device__ __forceinline__ float group_sum(float v) {
  static_assert(N == 8 || N == 16, "8- or 16-lane groups");
  v += dpp_mov<0xB1>(v);   // quad_perm [1, 0, 3, 2]
  v += dpp_mov<0x4E>(v);   // quad_perm [2, 3, 0, 1]
  v += dpp_mov<0x141>(v);  // row_half_mirror
  if (N == 16) v += dpp_mov<0x140>(v);  // row_mirror
  return v;
}

// 2^x by the hardware instruction (v_exp_f32, about 1 ulp): results below 2^-126 flush to
// zero, which softmax weights (x <= 0) lose nothing by; 2^-inf = 0.
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// Sum over the wave, the same value in every lane: 16-lane row sums by DPP, then the four
// row sums read into scalar registers and added in a fixed order.
__device__ __forceinline__ float wave_sum_rows(float v) {
  v = group_sum<16>(v);
  const float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float b = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float d = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return (a + b) + (c + d);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

// Sum over a 256-thread block; every thread gets the total.  `red` holds 4 floats.
__device__ __forceinline__ float block256_sum(float v, float* red) {
  v = wave_sum(v);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  return red[0] + red[1] + red[2] + red[3];
}

__device__ __forceinline__ int64_t kv_offset(int layer, int kv, int block, int head, int slot, int e,
                                             int num_blocks, int n_kv_heads, int d_head) {
  return ((((int64_t)layer * 2 + kv) * num_blocks + block) * n_kv_heads + head) * (int64_t)(KV_BLOCK * d_head) +
         (int64_t)slot * d_head + e;
}

}  // namespace dec
