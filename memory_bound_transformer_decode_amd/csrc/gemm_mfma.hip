// Weight-streaming products for batches of 4 to 64 rows on the matrix cores.
//
// At these batches y = s (.) (W x) is a real (if skinny) contraction: 2 Bp FLOP per
// weight element, more than the vector ALUs issue at HBM rate, so the products run on
// v_mfma_f32_16x16x32_bf16 tiles.  The kernel is still bound by HBM ("GPU Inference
// Internals", Roofline: Why Decode Is Memory-Bound: the intensity 2 Bp / b_w stays
// far below the chip's balance), so its design is about bytes, not FLOPs:
//
//  * Every weight byte is read once, with 16-byte non-temporal loads in which 16
//    lanes read 256 contiguous bytes of one row (a load instruction covers 4 rows).
//    The MFMA operand layout would have each instruction touch 16 rows with 64 bytes
//    each, which streams measurably slower from HBM; each wave instead passes its
//    loads through a small private LDS tile that hands every lane its operand.
//  * One-byte codes (E4M3 or int8) are widened to bf16 in registers (exact), and the
//    per-row scale is applied once in the epilogue (dequantization fused into the
//    matmul: kernel-fusion architecture study, section 11).
//  * QKV runs on v_mfma_f32_16x16x32_f16 instead: its input x comes as fp16 (more
//    significant bits for q and k, see MatmulParams::xl), and the weights are widened
//    to fp16 in registers (exact for E4M3 and int8; bf16 see bf16x2_to_f16x2).
//  * The activations x [Bp][K] are the other operand of every tile.  A work group owns
//    W 16-row tiles (one per wave) and stages x through LDS in chunks of KC k-values
//    shared by all of its waves, so its L2 reads of x are Bp / 16 W of the weight bytes
//    instead of Bp / 16 of them for a work group of one tile.
//  * Every wave keeps the next chunk's weights in flight while it multiplies the
//    current one.  For the compiler's waits to allow that, every path issues the same
//    loads in a fixed order and no loaded value is looked at before it is needed (a
//    select on the just-loaded x made each chunk wait for all loads in flight).
//  * Matrices with too few row blocks to fill the chip also split K over KS work
//    groups.  Each writes its partial tiles; the last one of a row block to arrive sums
//    the KS partials in split order (so the result does not depend on arrival order)
//    and applies the epilogue.
//
// Fused epilogues as in the matrix-vector kernels: QKV + RoPE + paged KV-cache write,
// gate+up + SiLU x mul (a tile holds 8 gate rows and the 8 up rows of the same
// intermediate indices), residual add (O, down), fp32 logits (LM head).

#include "common.h"
#include "epilogue.h"
#include "kernels.h"

namespace dec {

namespace {

constexpr int KC = 256;          // k-values per staged chunk of x
constexpr int XROW = KC + 8;     // LDS row of a staged x chunk, in bf16: 16 bytes of padding
                                 // move consecutive batch rows to different LDS banks
// Weight rows one load instruction covers (bf16; one-byte weights always 4): each row
// gets 64 / R lanes of 16 bytes, i.e. 4 rows x 256 bytes per instruction (2 rows x 512
// bytes measured within 1 % at 8 and 32 rows, 5 % slower at 64)
constexpr int RPL_BF16 = 4;
template <bool B8>
constexpr int tile_bytes() { return B8 ? 256 : 16 * (64 / RPL_BF16); }  // of a row per group
template <bool B8>
constexpr int tile_row() { return tile_bytes<B8>() + 16; }  // LDS row of a wave's weight tile (padded)
// x chunk buffers: two (the next chunk is staged while this one is read) up to 32 batch
// columns; one beyond, where two would hold the LDS to one work group per CU.
constexpr int x_buffers(int NT) { return NT >= 3 ? 1 : 2; }
// 16-row tiles per wave (measured on the 8B, 32B and 70B shapes at 48-64 rows): with
// one-byte (E4M3) weights each x operand read from LDS (NT per k-step) costs the LDS more than the
// weights do, so from 48 columns a wave takes two tiles that share those reads -- on
// matrices of at least TPW2_MIN_WEIGHTS weights; smaller ones would need twice the K
// split, which costs more than it saves.  bf16 weights: one tile (two take 256 registers
// per lane, one wave per SIMD).
constexpr size_t TPW2_MIN_WEIGHTS = (size_t)200 << 20;
int tiles_per_wave(int NT, bool byte_weights, int n_rows_total, int K) {
  return byte_weights && NT >= 3 && (size_t)n_rows_total * (size_t)K >= TPW2_MIN_WEIGHTS ? 2 : 1;
}

// Weight chunks each wave keeps in flight (the chunk being multiplied and D - 1 ahead).
// Measured at 8B and 70B widths, batches 8 to 64: two (one chunk ahead) beat three and
// four, whose registers cost more than their extra loads in flight bring.
constexpr int GEMM_DEPTH = 2;
constexpr int gemm_depth(int) { return GEMM_DEPTH; }

// v_mfma_f32_16x16x32_bf16: lane l supplies A[l % 16][8 k-values] and B[8 k-values][l % 16],
// the four lane groups l / 16 four disjoint sets of 8 k-values; lane l receives
// D[4 (l / 16) + j][l % 16], j = 0..3.  Which k-values a lane group covers is free as long
// as A and B agree: in k-step s of a group of GK k-values, lane group g takes the 8
// k-values s 32 + 8 g + [0, 8).  v_mfma_f32_16x16x32_f16 has the same operand layout.
// F16: x holds fp16 codes and the weights enter the products as fp16 (the QKV input).
template <int NT, int WQ, int EPI, bool KVFP8, int W, int TPW, bool F16>
__global__ __launch_bounds__(WAVE * W) void k_gemm_lds(MatmulParams p, int ks_n) {
  // x: [XBUFS][NT 16][XROW] bf16 or fp16; tiles: [W][TPW][16][TROW]
  extern __shared__ __align__(16) uint8_t lds[];
  constexpr bool B8 = WQ != W_BF16;  // one-byte weights (E4M3 or int8 codes)
  constexpr bool SILU = EPI == EPI_SILU;
  constexpr int RPL = B8 ? 4 : RPL_BF16;          // rows per weight load instruction
  constexpr int LPR = WAVE / RPL;                  // lanes per row of a load
  constexpr int TB = tile_bytes<B8>();            // bytes of a row per group
  constexpr int TROW = tile_row<B8>();
  constexpr int GK = B8 ? TB : TB / 2;            // k-values per group
  constexpr int NGRP = KC / GK;                    // groups per chunk (2 bf16, 1 one-byte)
  constexpr int NS = GK / 32;                      // MFMA k-steps per group
  constexpr int COLS = NT * 16;
  constexpr int XSEG = KC / 8;                     // 16-byte pieces per staged x row
  constexpr int XL = (COLS * XSEG + W * WAVE - 1) / (W * WAVE);  // x staging loads per thread
  constexpr int XBUF = COLS * XROW;                // elements per x buffer
  constexpr int XBUFS = x_buffers(NT);
  uint16_t* xs = reinterpret_cast<uint16_t*>(lds);
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / WAVE);
  const int lane = tid % WAVE, m = lane % 16, kg = lane / 16;
  uint8_t* tile = lds + (size_t)XBUFS * XBUF * 2 + (size_t)wave * TPW * 16 * tile_row<B8>();
  // rows: output rows of the product (d_ff intermediate indices for gate+up); a tile
  // covers TR of them, a wave TPW tiles (TPW > 1: each x operand read from LDS feeds
  // TPW tiles' products)
  constexpr int TR = SILU ? 8 : 16;
  const int rows = SILU ? p.d_ff : p.N;
  const int rb = blockIdx.x / ks_n, ks = blockIdx.x % ks_n;
  const int nch = (p.K + KC - 1) / KC;
  const int c0 = (int)((int64_t)nch * ks / ks_n), c1 = (int)((int64_t)nch * (ks + 1) / ks_n);
  const int row0 = (rb * W + wave) * TR * TPW;  // first output row of this wave's tiles

  // weight row of row i of tile tt (rows past the matrix are clamped: their results are
  // dropped)
  auto wrow = [&](int tt, int i) -> int {
    const int r0 = row0 + tt * TR;
    if (SILU) return (i < 8 ? 0 : p.d_ff) + min(r0 + (i & 7), rows - 1);
    return min(r0 + i, rows - 1);
  };
  const size_t rowbytes = B8 ? (size_t)p.K : (size_t)p.K * 2;
  // load q of a group: lane (r = lane / LPR, j = lane % LPR) reads 16 bytes at byte 16 j
  // of the group's TB bytes of tile row RPL q + r
  constexpr int NQ = 16 / RPL;
  const int lr = lane / LPR, lj = lane % LPR;
  const uint8_t* wp[TPW][NQ];
#pragma unroll
  for (int tt = 0; tt < TPW; ++tt)
#pragma unroll
    for (int q = 0; q < NQ; ++q)
      wp[tt][q] = static_cast<const uint8_t*>(p.W) + (size_t)wrow(tt, RPL * q + lr) * rowbytes;
  const int lastv = (int)rowbytes - 16;  // last 16-byte piece of a row

  // weight loads of chunk c, unconditional: pieces past K are read at the row's last
  // piece (x is zero there, so they add nothing)
  // A chunk past this work group's last (c >= c1) reads the matrix's first bytes instead,
  // the same few lines for every wave (cache hits), so that every path issues the same
  // loads: the compiler's waits for a chunk then let the later chunks' loads stay in
  // flight (a load issued on only some paths makes it wait for all of them).
  auto load_w = [&](int c, u32x4 (&wr)[TPW][NGRP][NQ]) {
    const bool real = c < c1;
#pragma unroll
    for (int gi = 0; gi < NGRP; ++gi) {
      const int off = min(c * KC * (B8 ? 1 : 2) + gi * TB + lj * 16, lastv);
#pragma unroll
      for (int tt = 0; tt < TPW; ++tt)
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
          const uint8_t* a = real ? wp[tt][q] + off : static_cast<const uint8_t*>(p.W) + lj * 16;
          wr[tt][gi][q] = ld_stream(reinterpret_cast<const u32x4*>(a));
        }
    }
  };
  // x loads of chunk c into registers (rows past Bp read row Bp - 1, k past K the row's
  // last piece).  The loaded values are not looked at before store_x: a use right after
  // the load would wait for it, and so for every weight load issued before it.
  auto load_x = [&](int c, u32x4 (&xr)[XL]) {
#pragma unroll
    for (int j = 0; j < XL; ++j) {
      const int i = tid + j * W * WAVE;
      const int b = min(i / XSEG, p.Bp - 1), k = c * KC + (i % XSEG) * 8;
      xr[j] = gld16(p.x + (int64_t)b * p.ldx + min(k, p.K - 8));
    }
  };
  // x of chunk c into LDS buffer buf, zero for k past K
  auto store_x = [&](int buf, int c, const u32x4 (&xr)[XL]) {
#pragma unroll
    for (int j = 0; j < XL; ++j) {
      const int i = tid + j * W * WAVE;
      const int k = c * KC + (i % XSEG) * 8;
      if (XL * W * WAVE == COLS * XSEG || i < COLS * XSEG)
        *reinterpret_cast<u32x4*>(xs + buf * XBUF + (i / XSEG) * XROW + (i % XSEG) * 8) =
            k < p.K ? xr[j] : u32x4{0u, 0u, 0u, 0u};
    }
  };

  f32x4 acc[TPW][NT];
#pragma unroll
  for (int tt = 0; tt < TPW; ++tt)
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[tt][t] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto mma_chunk = [&](int buf, const u32x4 (&wr)[TPW][NGRP][NQ]) {
#pragma unroll
    for (int gi = 0; gi < NGRP; ++gi) {
      // this wave's TPW 16 x TB-byte tiles of the group, then each lane's operands from them
#pragma unroll
      for (int tt = 0; tt < TPW; ++tt)
#pragma unroll
        for (int q = 0; q < NQ; ++q)
          *reinterpret_cast<u32x4*>(tile + (tt * 16 + RPL * q + lr) * TROW + lj * 16) = wr[tt][gi][q];
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        // the lane's 8 weights of each tile as bf16, or fp16 (F16), bits
        u32x4 av[TPW];
#pragma unroll
        for (int tt = 0; tt < TPW; ++tt) {
          const uint8_t* tr = tile + (tt * 16 + m) * TROW;
          if (B8) {
            const u32x2 c8 = *reinterpret_cast<const u32x2*>(tr + s * 32 + kg * 8);
            if constexpr (F16)
              av[tt] = u32x4{__builtin_bit_cast(uint32_t, b8x2_to_f16x2<WQ, false>(c8.x)),
                             __builtin_bit_cast(uint32_t, b8x2_to_f16x2<WQ, true>(c8.x)),
                             __builtin_bit_cast(uint32_t, b8x2_to_f16x2<WQ, false>(c8.y)),
                             __builtin_bit_cast(uint32_t, b8x2_to_f16x2<WQ, true>(c8.y))};
            else
              av[tt] = u32x4{__builtin_bit_cast(uint32_t, b8x2_to_bf16x2<WQ, false>(c8.x)),
                             __builtin_bit_cast(uint32_t, b8x2_to_bf16x2<WQ, true>(c8.x)),
                             __builtin_bit_cast(uint32_t, b8x2_to_bf16x2<WQ, false>(c8.y)),
                             __builtin_bit_cast(uint32_t, b8x2_to_bf16x2<WQ, true>(c8.y))};
          } else {
            const u32x4 wv = *reinterpret_cast<const u32x4*>(tr + s * 64 + kg * 16);
            if constexpr (F16)
              av[tt] = u32x4{__builtin_bit_cast(uint32_t, bf16x2_to_f16x2(wv.x)),
                             __builtin_bit_cast(uint32_t, bf16x2_to_f16x2(wv.y)),
                             __builtin_bit_cast(uint32_t, bf16x2_to_f16x2(wv.z)),
                             __builtin_bit_cast(uint32_t, bf16x2_to_f16x2(wv.w))};
            else
              av[tt] = wv;
          }
        }
        const uint16_t* xb = xs + buf * XBUF;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const u32x4 bv = ld16(xb + (t * 16 + m) * XROW + gi * GK + s * 32 + kg * 8);
#pragma unroll
          for (int tt = 0; tt < TPW; ++tt) {
            if constexpr (F16)
              acc[tt][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, av[tt]),
                                                                  __builtin_bit_cast(f16x8, bv), acc[tt][t], 0, 0, 0);
            else
              acc[tt][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av[tt]),
                                                                   __builtin_bit_cast(bf16x8, bv), acc[tt][t], 0, 0, 0);
          }
        }
      }
    }
  };

  // What the epilogue reads besides the sums, fetched at kernel start so that these loads
  // overlap the weight stream: for the lane's four rows er0 .. er0 + 3 of each tile (in
  // range: full) and each of its batch columns, the row scales, the residual rows (O,
  // down), and for QKV the token's position and cache block and the RoPE angles of the
  // lane's two row pairs (adjacent in the table: er0 is a multiple of 4, d_head of 64).
  int er0[TPW];
  bool full[TPW];
#pragma unroll
  for (int tt = 0; tt < TPW; ++tt) {
    er0[tt] = row0 + tt * TR + 4 * kg;
    full[tt] = er0[tt] + 4 <= rows;
  }
  f32x4 e_sc[TPW], e_su[TPW], e_g[TPW];  // e_g: the folded next norm's gain (O, down)
  f32x4 e_h[TPW][EPI == EPI_RESID ? NT : 1];
  f32x4 e_cs[TPW][EPI == EPI_QKV ? NT : 1];
  int e_pos[EPI == EPI_QKV ? NT : 1], e_blk[EPI == EPI_QKV ? NT : 1];
  // As with the weights, every path issues the same loads here (rows clamped into the
  // matrix, absent scale or gain arrays replaced by the matrix's first bytes), and the
  // values are looked at only in the epilogue, where they are selected.  The tokens'
  // positions, which the cache-block and RoPE addresses need, are loaded before the first
  // weights (pos_prefetch), so that waiting for them leaves the weight loads in flight.
  const float* fdummy = static_cast<const float*>(p.W);
  auto pos_prefetch = [&]() {
    if (EPI == EPI_QKV) {
#pragma unroll
      for (int t = 0; t < NT; ++t) e_pos[t] = gld(p.seq_lens + min(t * 16 + m, p.Bp - 1));
    }
  };
  auto epi_prefetch = [&]() {
#pragma unroll
    for (int tt = 0; tt < TPW; ++tt) {
      const int rc = min(er0[tt], rows - 4);
      e_sc[tt] = gld(reinterpret_cast<const f32x4*>(p.scale ? p.scale + rc : fdummy));
      if (SILU) e_su[tt] = gld(reinterpret_cast<const f32x4*>(p.scale ? p.scale + p.d_ff + rc : fdummy));
      if (EPI == EPI_RESID) {
        e_g[tt] = gld(reinterpret_cast<const f32x4*>(p.xout ? p.xg + rc : fdummy));
#pragma unroll
        for (int t = 0; t < NT; ++t)
          e_h[tt][t] = gld(reinterpret_cast<const f32x4*>(p.out + (int64_t)min(t * 16 + m, p.Bp - 1) * p.ldo + rc));
      }
    }
    if (EPI == EPI_QKV) {
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const int col = min(t * 16 + m, p.Bp - 1);
        const int pr = e_pos[t] < 0 ? 0 : e_pos[t];
        e_blk[t] = gld(p.bt + (int64_t)col * p.bps + pr / KV_BLOCK);  // used only where e_pos >= 0
#pragma unroll
        for (int tt = 0; tt < TPW; ++tt)
          e_cs[tt][t] = gld(reinterpret_cast<const f32x4*>(p.rope + (int64_t)pr * (p.dh / 2) +
                                                             ((min(er0[tt], rows - 4) % p.dh) >> 1)));
      }
    }
  };

  // folded RMSNorm (ssq_n > 0): thread (part, column) adds the producer's row-block sums
  // of squares i = part, part + W, ... of its batch column; loaded ahead of the first
  // chunk, added once those loads are out; combined per column in the epilogue
  __shared__ float ssq_s[W][GEMM_SSQ_STRIDE];
  constexpr int SPER = (GEMM_SSQ_MAX + W - 1) / W;
  {
    // weight chunks in flight: chunk c + D - 1 is requested before chunk c is multiplied
    constexpr int D = gemm_depth(TPW);
    u32x4 wr[D][TPW][NGRP][NQ], xr[XL];
    const int scol = tid % GEMM_SSQ_STRIDE, spart = tid / GEMM_SSQ_STRIDE;
    float sv[SPER];
    {
      const float* sp = p.ssq_n > 0 ? p.ssq_in + min(scol, p.Bp - 1) : fdummy;
      const int last = p.ssq_n > 0 ? p.ssq_n - 1 : 0;
#pragma unroll
      for (int j = 0; j < SPER; ++j) sv[j] = gld(sp + (size_t)min(spart + j * W, last) * GEMM_SSQ_STRIDE);
    }
    pos_prefetch();
    load_x(c0, xr);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j + 1 < D; ++j) load_w(c0 + j, wr[j]);
    __builtin_amdgcn_sched_barrier(0);
    epi_prefetch();
    __builtin_amdgcn_sched_barrier(0);
    if (p.ssq_n > 0) {
      float ss = 0.f;
#pragma unroll
      for (int j = 0; j < SPER; ++j) ss += spart + j * W < p.ssq_n ? sv[j] : 0.f;
      ssq_s[spart][scol] = ss;
    }
    store_x(0, c0, xr);
    __syncthreads();
    // chunk c = c0 + D i + j sits in weight buffer j and in x buffer (c - c0) % XBUFS.  The
    // x of chunk c + 1 is requested before the weights of chunk c + D - 1, so that storing
    // it to LDS (which waits for it) does not wait for those weights.
    for (int c = c0; c < c1; c += D) {
#pragma unroll
      for (int j = 0; j < D; ++j) {
        const int cc = c + j;
        if (cc >= c1) break;
        // the order of the loads (and that they precede the products) is kept by
        // scheduling barriers: the compiler would otherwise sink them past the products
        load_x(cc + 1, xr);
        __builtin_amdgcn_sched_barrier(0);
        load_w(cc + D - 1, wr[(j + D - 1) % D]);
        __builtin_amdgcn_sched_barrier(0);
        mma_chunk(XBUFS == 2 ? (cc - c0) & 1 : 0, wr[j]);
        if (cc + 1 >= c1) break;
        if (XBUFS == 1) __syncthreads();
        store_x(XBUFS == 2 ? (cc + 1 - c0) & 1 : 0, cc + 1, xr);
        __syncthreads();
      }
    }
  }

  if (ks_n > 1) {
    // partial tiles of this split: part[blockIdx.x][wave][tt][t][lane] (f32x4), written
    // device-coherently for the work group that combines them
    constexpr int PT = TPW * NT;
    float* part = p.gpart + ((int64_t)blockIdx.x * W + wave) * PT * (WAVE * 4);
#pragma unroll
    for (int tt = 0; tt < TPW; ++tt)
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const f32x4 v = acc[tt][t];
        cst_f4(part + ((tt * NT + t) * WAVE + lane) * 4, v.x, v.y, v.z, v.w);
      }
    __shared__ int last;
    if (!arrive_after_stores(p.gcnt + (int64_t)rb * COUNTER_STRIDE, (unsigned)ks_n, &last)) return;
    // sum the splits in order 0..ks_n-1 (this work group's own from registers)
    f32x4 tot[TPW][NT];
#pragma unroll
    for (int tt = 0; tt < TPW; ++tt)
#pragma unroll
      for (int t = 0; t < NT; ++t) tot[tt][t] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int sp = 0; sp < ks_n; ++sp) {
      const float* ps = p.gpart + ((int64_t)(rb * ks_n + sp) * W + wave) * PT * (WAVE * 4);
#pragma unroll
      for (int tt = 0; tt < TPW; ++tt)
#pragma unroll
        for (int t = 0; t < NT; ++t)
          tot[tt][t] += sp == ks ? acc[tt][t] : cld_f4(ps + ((tt * NT + t) * WAVE + lane) * 4);
    }
#pragma unroll
    for (int tt = 0; tt < TPW; ++tt)
#pragma unroll
      for (int t = 0; t < NT; ++t) acc[tt][t] = tot[tt][t];
  }

  // epilogue: lane holds rows 4 kg + j (j = 0..3) of each tile, batch column t 16 + m
  if (p.ssq_n > 0) {
    // the folded RMSNorm's 1 / rms of each batch column, on the sums
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int col = t * 16 + m;
      float ss = 0.f;
#pragma unroll
      for (int w = 0; w < W; ++w) ss += ssq_s[w][col];
      const float rinv = 1.0f / sqrtf(ss / (float)p.K + p.eps);
#pragma unroll
      for (int tt = 0; tt < TPW; ++tt) acc[tt][t] *= rinv;
    }
  }
  float sq[NT];  // residual products that fold the next norm: this lane's sum of h^2
#pragma unroll
  for (int t = 0; t < NT; ++t) sq[t] = 0.f;
#pragma unroll
  for (int tt = 0; tt < TPW; ++tt) {
    const int r0 = er0[tt];  // the lane's first row in tile tt (for gate+up: lane groups 0, 1)
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int col = t * 16 + m;
      if (SILU) {
        // gate rows are tile rows 0..7 (lane groups 0, 1), up rows 8..15 (lane groups 2,
        // 3): lane l pairs with lane l + 32
        f32x4 up;
#pragma unroll
        for (int j = 0; j < 4; ++j) up[j] = __shfl_xor(acc[tt][t][j], 32);
        if (kg >= 2 || col >= p.Bp) continue;
        uint16_t* o = p.act + (int64_t)col * p.ldact;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int r = r0 + j;
          if (r >= rows) break;
          const float sg = !p.scale ? 1.f : full[tt] ? e_sc[tt][j] : gld(p.scale + r);
          const float su = !p.scale ? 1.f : full[tt] ? e_su[tt][j] : gld(p.scale + p.d_ff + r);
          gst(o + r, f32_to_bf16(silu_f(acc[tt][t][j] * sg) * (up[j] * su)));
        }
        continue;
      }
      if (col >= p.Bp) continue;
      if (EPI == EPI_QKV) {
        if (full[tt]) {
          // rows r0 .. r0 + 3 lie in one head (r0 % 4 == 0, d_head % 4 == 0)
          const int qrows = p.Hq * p.dh, krows = p.Hkv * p.dh, dh = p.dh;
          float y[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) y[j] = acc[tt][t][j] * (p.scale ? e_sc[tt][j] : 1.f);
          if (r0 < qrows + krows) {  // q or k: rotate the adjacent pairs
            const f32x4 cs = e_cs[tt][t];
            const float a0 = y[0] * cs.x - y[1] * cs.y, a1 = y[0] * cs.y + y[1] * cs.x;
            const float b0 = y[2] * cs.z - y[3] * cs.w, b1 = y[2] * cs.w + y[3] * cs.z;
            y[0] = a0; y[1] = a1; y[2] = b0; y[3] = b1;
          }
          if (r0 < qrows) {
            float* qp = p.q + ((int64_t)col * p.Hq + r0 / dh) * dh + r0 % dh;
            cst_f2(qp, y[0], y[1]);
            cst_f2(qp + 2, y[2], y[3]);
          } else if (e_pos[t] >= 0) {  // padded rows write no cache slot
            const int kv = r0 < qrows + krows ? 0 : 1;
            const int rr = r0 - qrows - kv * krows;
            const int64_t off = kv_offset(p.layer, kv, e_blk[t], rr / dh, e_pos[t] % KV_BLOCK, rr % dh, p.num_blocks,
                                          p.Hkv, dh);
            if (KVFP8) {
              const uint32_t w = f32_to_e4m3(y[0]) | (f32_to_e4m3(y[1]) << 8) | (f32_to_e4m3(y[2]) << 16) |
                                 (f32_to_e4m3(y[3]) << 24);
              cst(reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(p.pool) + off), w);
            } else {
              const uint64_t w = (uint64_t)f32_to_bf16(y[0]) | ((uint64_t)f32_to_bf16(y[1]) << 16) |
                                 ((uint64_t)f32_to_bf16(y[2]) << 32) | ((uint64_t)f32_to_bf16(y[3]) << 48);
              cst(reinterpret_cast<uint64_t*>(static_cast<uint16_t*>(p.pool) + off), w);
            }
          }
          continue;
        }
#pragma unroll
        for (int j = 0; j < 4; j += 2) {
          const int r = r0 + j;  // even; rows is a multiple of d_head
          if (r >= rows) break;
          const float s0 = p.scale ? gld(p.scale + r) : 1.f, s1 = p.scale ? gld(p.scale + r + 1) : 1.f;
          qkv_pair_out(p, KVFP8, col, r, acc[tt][t][j] * s0, acc[tt][t][j + 1] * s1);
        }
      } else {
        float* o = p.out + (int64_t)col * p.ldo;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int r = r0 + j;
          if (r >= rows) break;
          const float y = acc[tt][t][j] * (!p.scale ? 1.f : full[tt] ? e_sc[tt][j] : gld(p.scale + r));
          if (EPI == EPI_RESID) {
            const float hn = (full[tt] ? e_h[tt][t][j] : gld(o + r)) + y;
            gst(o + r, hn);
            if (p.xout) {
              const float xv = hn * (full[tt] ? e_g[tt][j] : gld(p.xg + r));
              gst(p.xout + (int64_t)col * p.ldxo + r, p.xout_f16 ? f32_to_f16(xv) : f32_to_bf16(xv));
              sq[t] += hn * hn;
            }
          } else {
            gst(o + r, y);
          }
        }
      }
    }
  }
  if (EPI == EPI_RESID && p.xout) {
    // the row block's sum of h^2 per batch column: over the lane's rows (above), the four
    // lane groups, then the waves in order
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      sq[t] += __shfl_xor(sq[t], 16);
      sq[t] += __shfl_xor(sq[t], 32);
      if (kg == 0) ssq_s[wave][t * 16 + m] = sq[t];
    }
    __syncthreads();
    if (tid < p.Bp) {
      float ss = 0.f;
#pragma unroll
      for (int w = 0; w < W; ++w) ss += ssq_s[w][tid];
      gst(p.ssq_out + (int64_t)rb * GEMM_SSQ_STRIDE + tid, ss);
    }
  }
}

template <bool B8>
constexpr size_t lds_bytes(int NT, int W, int TPW) {
  return (size_t)x_buffers(NT) * NT * 16 * XROW * 2 + (size_t)W * TPW * 16 * tile_row<B8>();
}

template <int NT, int WQ, int EPI, bool KVFP8, int W, int TPW, bool F16>
hipError_t go_tpwx(const MatmulParams& p, const GemmPlan& g, hipStream_t s) {
  auto kern = k_gemm_lds<NT, WQ, EPI, KVFP8, W, TPW, F16>;
  constexpr size_t lds = lds_bytes<WQ != W_BF16>(NT, W, TPW);
  static_assert(lds <= 160 * 1024, "LDS of one work group");
  static bool attr = false;
  if (!attr && lds > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    attr = true;
  }
  hipLaunchKernelGGL(kern, dim3(g.n_rb * g.ks), dim3(WAVE * W), lds, s, p, g.ks);
  return hipGetLastError();
}

// QKV always takes an fp16 input; a plain product (the unfused step's QKV) does when
// p.x_f16 says so; the others never do
template <int NT, int WQ, int EPI, bool KVFP8, int W, int TPW>
hipError_t go_tpw(const MatmulParams& p, const GemmPlan& g, hipStream_t s) {
  if constexpr (EPI == EPI_QKV) {
    return go_tpwx<NT, WQ, EPI, KVFP8, W, TPW, true>(p, g, s);
  } else if constexpr (EPI == EPI_LOGITS) {
    return p.x_f16 ? go_tpwx<NT, WQ, EPI, KVFP8, W, TPW, true>(p, g, s)
                   : go_tpwx<NT, WQ, EPI, KVFP8, W, TPW, false>(p, g, s);
  } else {
    return go_tpwx<NT, WQ, EPI, KVFP8, W, TPW, false>(p, g, s);
  }
}

template <int NT, int WQ, int EPI, bool KVFP8, int W>
hipError_t go(const MatmulParams& p, const GemmPlan& g, hipStream_t s) {
  if constexpr (WQ != W_BF16 && NT >= 3)
    if (g.tpw == 2) return go_tpw<NT, WQ, EPI, KVFP8, W, 2>(p, g, s);
  return go_tpw<NT, WQ, EPI, KVFP8, W, 1>(p, g, s);
}

template <int WQ, int EPI, bool KVFP8>
hipError_t go_nt(const MatmulParams& p, const GemmPlan& g, hipStream_t s) {
  if constexpr (EPI == EPI_SILU) {
    if (g.waves == GEMM_WAVES_WIDE) {
      if (p.Bp <= 16) return go<1, WQ, EPI, KVFP8, GEMM_WAVES_WIDE>(p, g, s);
      if (p.Bp <= 32) return go<2, WQ, EPI, KVFP8, GEMM_WAVES_WIDE>(p, g, s);
      if (p.Bp <= 48) return go<3, WQ, EPI, KVFP8, GEMM_WAVES_WIDE>(p, g, s);
      return go<4, WQ, EPI, KVFP8, GEMM_WAVES_WIDE>(p, g, s);
    }
  }
  if (g.waves != GEMM_WAVES) return hipErrorInvalidValue;
  if (p.Bp <= 16) return go<1, WQ, EPI, KVFP8, GEMM_WAVES>(p, g, s);
  if (p.Bp <= 32) return go<2, WQ, EPI, KVFP8, GEMM_WAVES>(p, g, s);
  if (p.Bp <= 48) return go<3, WQ, EPI, KVFP8, GEMM_WAVES>(p, g, s);
  return go<4, WQ, EPI, KVFP8, GEMM_WAVES>(p, g, s);
}

template <int WQ>
hipError_t go_epi(const MatmulParams& p, const GemmPlan& g, int epi, bool kv_fp8, hipStream_t s) {
  switch (epi) {
    case EPI_LOGITS: return go_nt<WQ, EPI_LOGITS, false>(p, g, s);
    case EPI_RESID: return go_nt<WQ, EPI_RESID, false>(p, g, s);
    case EPI_SILU: return go_nt<WQ, EPI_SILU, false>(p, g, s);
    default: return kv_fp8 ? go_nt<WQ, EPI_QKV, true>(p, g, s) : go_nt<WQ, EPI_QKV, false>(p, g, s);
  }
}

}  // namespace

// Row blocks of GEMM_WAVES tiles and the K split: where the row blocks alone would leave
// the chip under-filled (fewer than GEMM_TARGET_GROUPS work groups for MI355X's 256
// CUs), K is split, at least two chunks per work group and at most one work group per
// CU.  A pure function of the shape: the workspace is sized with it.
GemmPlan gemm_plan(int rows, int n_groups, int K, int Bp, bool byte_weights) {
  GemmPlan g{};
  const int NT = (Bp + 15) / 16;
  const int tpw = tiles_per_wave(NT, byte_weights, rows * n_groups, K);
  const int tile_rows = (n_groups == 2 ? 8 : 16) * tpw;  // gate+up tiles hold 8 of each
  g.waves = GEMM_WAVES;
  g.n_rb = (rows + tile_rows * GEMM_WAVES - 1) / (tile_rows * GEMM_WAVES);
  const int nch = (K + KC - 1) / KC;
  if (n_groups == 2 && g.n_rb >= GEMM_TARGET_GROUPS) {
    // gate+up without a K split: the row-block size whose busiest CU streams the fewest
    // wave tiles (work groups past a multiple of the CU count double up on some CUs)
    const int units = (rows + tile_rows - 1) / tile_rows;
    auto busiest = [&](int w) {
      const int n = (units + w - 1) / w;
      return ((n + GEMM_TARGET_GROUPS - 1) / GEMM_TARGET_GROUPS) * w;
    };
    if (busiest(GEMM_WAVES_WIDE) < busiest(GEMM_WAVES)) {
      g.waves = GEMM_WAVES_WIDE;
      g.n_rb = (units + GEMM_WAVES_WIDE - 1) / GEMM_WAVES_WIDE;
    }
  }
  int ks = 1;
  if (g.n_rb < GEMM_TARGET_GROUPS) {
    // as many splits as fit the CUs without a second work group on any of them: a grid
    // just past a multiple of the CU count doubles the work of some CUs while the others
    // wait (8B QKV at 32 rows: 3 splits, 288 work groups, measured slower than 2)
    ks = GEMM_TARGET_GROUPS / g.n_rb;
    const int cap = nch / 2 > 1 ? nch / 2 : 1;
    if (ks > cap) ks = cap;
    if (ks > GEMM_MAX_SPLIT) ks = GEMM_MAX_SPLIT;
  }
  g.ks = ks;
  g.tpw = tpw;
  g.part_floats = ks > 1 ? (size_t)g.n_rb * ks * g.waves * tpw * NT * WAVE * 4 : 0;
  return g;
}

hipError_t launch_gemm_mfma(const MatmulParams& p, int epi, WFmt wq, bool kv_fp8, hipStream_t s) {
  const int rows = epi == EPI_SILU ? p.d_ff : p.N;
  if (rows <= 0 || p.Bp <= 0) return hipSuccess;
  if (p.Bp > 64 || p.K < 16 || p.K % 16) return hipErrorInvalidValue;
  const GemmPlan g = gemm_plan(rows, epi == EPI_SILU ? 2 : 1, p.K, p.Bp, wq != W_BF16);
  if (g.ks > 1 && (!p.gpart || !p.gcnt || g.part_floats > p.gpart_floats || g.n_rb > p.gcnt_n))
    return hipErrorInvalidValue;
  // the folded RMSNorm: row-block sums within GEMM_SSQ_MAX x GEMM_SSQ_STRIDE
  if (p.ssq_n > GEMM_SSQ_MAX || (p.ssq_n > 0 && !p.ssq_in) ||
      (p.xout && (epi != EPI_RESID || !p.xg || !p.ssq_out || g.n_rb > GEMM_SSQ_MAX)))
    return hipErrorInvalidValue;
  switch (wq) {
    case W_E4M3: return go_epi<W_E4M3>(p, g, epi, kv_fp8, s);
    case W_I8: return go_epi<W_I8>(p, g, epi, kv_fp8, s);
    default: return go_epi<W_BF16>(p, g, epi, kv_fp8, s);
  }
}

}  // namespace dec
