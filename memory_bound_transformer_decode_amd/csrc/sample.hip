// Greedy sampling after the LM head: the argmax of each sequence's logits row, on the
// device, so that only the token ids -- not the vocabulary-sized logits -- need to leave
// the GPU ("Kernels, Fusion & CUDA Graphs", Fix 1: the sampling kernel keeps the logits
// on chip; "The serving engine's kernel stack": a sampling kernel turns logits into
// token ids before the small copy back to the CPU).
//
// One work group of 1024 threads per row; every thread scans a strided share of the row
// keeping the first largest value, then the work group reduces (value, index) pairs,
// larger value first, lower index on ties.  NaN never wins; a row with no number
// larger than -inf returns the first -inf, a row of NaN returns 0.

#include "common.h"
#include "kernels.h"

namespace dec {

namespace {
constexpr int AT = 1024;  // threads per row

__device__ __forceinline__ bool better(float v, int i, float bv, int bi) {
  // bi < 0: nothing held yet (then any non-NaN value is taken)
  return v > bv || (v == bv && (bi < 0 || (i >= 0 && i < bi)));
}
}  // namespace

__global__ __launch_bounds__(AT) void k_argmax(const float* logits, int ldl, int V, int32_t* out) {
  __shared__ float sv[AT / WAVE];
  __shared__ int si[AT / WAVE];
  const int row = blockIdx.x, tid = threadIdx.x, lane = tid % WAVE, w = tid / WAVE;
  const float* z = logits + (int64_t)row * ldl;
  float bv = -INFINITY;
  int bi = -1;
  for (int i = tid; i < V; i += AT) {
    const float v = gld(z + i);
    if (better(v, i, bv, bi)) { bv = v; bi = i; }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const float ov = __shfl_xor(bv, off);
    const int oi = __shfl_xor(bi, off);
    if (oi >= 0 && better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
  }
  if (lane == 0) { sv[w] = bv; si[w] = bi; }
  __syncthreads();
  if (tid == 0) {
    for (int k = 1; k < AT / WAVE; ++k)
      if (si[k] >= 0 && better(sv[k], si[k], bv, bi)) { bv = sv[k]; bi = si[k]; }
    gst(out + row, bi < 0 ? 0 : bi);
  }
}

// ---------------------------------------------------------------- top-k / top-p

// Sampling from the temperature-scaled softmax restricted to the top_k largest logits
// and then to the nucleus: the shortest prefix of them (largest first, lower index first
// on ties) whose probability reaches top_p.  The random draw is an input (u in [0, 1) per
// row): the token is the first candidate whose cumulative weight exceeds u times the
// nucleus weight.  One work group of 1024 threads per row:
//   1. the top_k-th largest logit by radix selection on an order-preserving 32-bit key
//      (four 8-bit passes over a 256-bin LDS histogram; NaN ranks as -inf);
//   2. the candidates gathered in index order: every key above it, and the lowest
//      indices among the keys equal to it;
//   3. each candidate's rank by counting the candidates before it;
//   4. one thread: weights exp((z - z_max) / T) in rank order, their running sums, the
//      nucleus cut and the draw.
namespace {
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) u = 0xFF800000u;  // NaN: as -inf
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_value(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}
}  // namespace

__global__ __launch_bounds__(AT) void k_sample_topkp(const float* logits, int ldl, int V, const float* uniforms,
                                                     float inv_temp, int top_k, float top_p, int32_t* out) {
  __shared__ unsigned hist[256];
  __shared__ uint32_t s_prefix, s_mask;
  __shared__ int s_need;  // candidates still to take among the keys under the prefix
  __shared__ int scan[AT / WAVE][2];
  __shared__ uint32_t ck[SAMPLE_MAX_K];
  __shared__ int ci[SAMPLE_MAX_K];
  __shared__ uint32_t sk[SAMPLE_MAX_K];
  __shared__ int si_[SAMPLE_MAX_K];
  __shared__ float cum_s[SAMPLE_MAX_K];
  const int row = blockIdx.x, tid = threadIdx.x, lane = tid % WAVE, w = tid / WAVE;
  const float* z = logits + (int64_t)row * ldl;
  const int K = min(top_k, V);
  if (tid == 0) {
    s_prefix = 0u;
    s_mask = 0u;
    s_need = K;
  }
  // 1. radix selection, most significant byte first
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    if (tid < 256) hist[tid] = 0u;
    __syncthreads();
    const uint32_t prefix = s_prefix, mask = s_mask;
    for (int i = tid; i < V; i += AT) {
      const uint32_t k = order_key(gld(z + i));
      if ((k & mask) == prefix) atomicAdd(&hist[(k >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (tid == 0) {
      int need = s_need, b = 255;
      for (; b > 0; --b) {
        if ((int)hist[b] >= need) break;
        need -= (int)hist[b];
      }
      s_need = need;
      s_prefix = prefix | ((uint32_t)b << shift);
      s_mask = mask | (255u << shift);
    }
    __syncthreads();
  }
  const uint32_t t = s_prefix;  // the K-th largest key
  const int need_eq = s_need;   // keys equal to t to take
  const int n_gt = K - need_eq;
  // 2. gather in index order: thread tid takes the contiguous indices [b0, b1)
  const int per = (V + AT - 1) / AT;
  const int b0 = min(V, tid * per), b1 = min(V, b0 + per);
  int gt = 0, eq = 0;
  for (int i = b0; i < b1; ++i) {
    const uint32_t k = order_key(gld(z + i));
    gt += k > t;
    eq += k == t;
  }
  // exclusive prefix sums over the threads (waves in order, then lanes in order)
  int xg = gt, xe = eq;
#pragma unroll
  for (int off = 1; off < WAVE; off <<= 1) {
    const int yg = __shfl_up(xg, off), ye = __shfl_up(xe, off);
    if (lane >= off) { xg += yg; xe += ye; }
  }
  if (lane == WAVE - 1) { scan[w][0] = xg; scan[w][1] = xe; }
  __syncthreads();
  int og = xg - gt, oe = xe - eq;
  for (int v = 0; v < w; ++v) { og += scan[v][0]; oe += scan[v][1]; }
  for (int i = b0; i < b1; ++i) {
    const uint32_t k = order_key(gld(z + i));
    if (k > t) {
      ck[og] = k;
      ci[og] = i;
      ++og;
    } else if (k == t) {
      if (oe < need_eq) {
        ck[n_gt + oe] = k;
        ci[n_gt + oe] = i;
      }
      ++oe;
    }
  }
  __syncthreads();
  // 3. rank: larger key first, lower index first
  if (tid < K) {
    const uint32_t k = ck[tid];
    const int i = ci[tid];
    int r = 0;
    for (int j = 0; j < K; ++j) r += ck[j] > k || (ck[j] == k && ci[j] < i);
    sk[r] = k;
    si_[r] = i;
  }
  __syncthreads();
  // 4. weights, nucleus and draw
  if (tid == 0) {
    const float zmax = key_value(sk[0]);
    float* cum = cum_s;  // running sums of the weights in rank order
    float c = 0.f;
    for (int j = 0; j < K; ++j) {
      const float zj = key_value(sk[j]);
      c += zj == -INFINITY ? 0.f : __expf((zj - zmax) * inv_temp);
      cum[j] = c;
    }
    int m = K - 1;  // last candidate of the nucleus
    for (int j = 0; j < K; ++j)
      if (cum[j] >= top_p * c) { m = j; break; }
    const float target = gld(uniforms + row) * cum[m];
    int pick = m;
    for (int j = 0; j <= m; ++j)
      if (cum[j] > target) { pick = j; break; }
    gst(out + row, si_[pick]);
  }
}

hipError_t launch_sample_topkp(const float* logits, int ldl, int V, int n, const float* uniforms, float temperature,
                               int top_k, float top_p, int32_t* out, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  if (top_k < 1 || top_k > SAMPLE_MAX_K || !(temperature > 0.f) || !(top_p > 0.f) || top_p > 1.f)
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_sample_topkp, dim3(n), dim3(AT), 0, s, logits, ldl, V, uniforms, 1.0f / temperature, top_k,
                     top_p, out);
  return hipGetLastError();
}

hipError_t launch_argmax(const float* logits, int ldl, int V, int n, int32_t* out, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_argmax, dim3(n), dim3(AT), 0, s, logits, ldl, V, out);
  return hipGetLastError();
}

}  // namespace dec
