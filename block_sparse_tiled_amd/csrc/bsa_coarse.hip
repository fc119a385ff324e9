// Coarse stage of video sparse attention for gfx950 (AMD Instinct MI355X):
// the choice of each query tile's key tiles (q2k_idx, q2k_num) and the coarse
// output, and the gated sum of the coarse and fine outputs.
//
// FastVideo fastvideo-kernel commit list, page 3: the hardening commit names
// the block-sparse kernel the "fine" attention (its fine-attention override)
// and the fused-layout commit scatters a gate into the tile buffer with Q, K
// and V; neither says how the tile lists are chosen.  The definition taken is
// the coarse stage of Video Sparse Attention (Zhang et al., 2025):
//   - every tile becomes one token, the mean of its valid rows;
//   - the pooled queries attend to the pooled keys; each query tile keeps the
//     topk key tiles with the largest coarse logits (a NaN logit ranks as
//     -inf, -0 as +0, equal logits by ascending index), listed by ascending
//     index, unused list entries -1; an empty query tile keeps nothing;
//   - the coarse output of a query tile is that pooled attention's result,
//     over every non-empty key tile;
//   - the layer output is the fine output plus the gate times the coarse
//     output of the token's tile.
// The pooled means and the logits are binary32 in a fixed order (rows summed
// in order then one division; one fused multiply-add per term over d
// ascending), so the selection is a fixed function of the inputs, reproducible
// bit for bit by a plain CPU loop.
//
// Kernels (all memory- or latency-bound; the stage is small next to the fine
// attention: for the video shape it reads Q, K and V once):
//   - coarse_pool_kernel: one thread per (tensor, head, tile, 16-byte chunk
//     of a row), summing the tile's valid rows in order (8 columns each);
//   - coarse_logits_kernel: the NT x NT logits per head, 64 x 64 per
//     workgroup, each thread a 4 x 4 block of them, d ascending through LDS,
//     one fused multiply-add per term;
//   - coarse_select_kernel: one wave per query tile; the row's keys in
//     registers, the k-th largest found by a 32-step bisection on their
//     order-preserving integer images (one ballot count per step), then the
//     kept tiles written in ascending order through ballot prefix counts;
//     also turns the row into softmax weights for the coarse output;
//   - coarse_out_kernel: those weights times the pooled values, on fp32 MFMA
//     (the weight rows staged in LDS, one wave per 32 columns);
//   - coarse_combine_kernel: out += gate * coarse output, valid rows only.
#include <hip/hip_runtime.h>

#include "bsa_fwd_common.h"
#include "bsa_launch.h"

namespace {

using namespace bsa::detail;

// ---- pooling ------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void coarse_pool_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const int32_t* __restrict__ vbs, int num_tiles, int tile, int64_t tiles_all,
    float* __restrict__ pooled) {
  constexpr int kChunks = D / 8;
  const int64_t total = 3 * tiles_all * kChunks;
  for (int64_t g = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; g < total;
       g += static_cast<int64_t>(gridDim.x) * 256) {
  const int64_t u = g / kChunks;  // (tensor, bh, t)
  const int c = static_cast<int>(g - u * kChunks);
  const int x = static_cast<int>(u / tiles_all);
  const int64_t rest = u - x * tiles_all;  // bh * NT + t
  const int t = static_cast<int>(rest % num_tiles);
  const uint16_t* src = (x == 0 ? q : (x == 1 ? k : v)) + rest * tile * D + 8 * c;
  const int n = clampi(vbs[t], 0, tile);
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.0f;
#pragma unroll 8
  for (int s = 0; s < n; ++s) {
    const uint4 w = *reinterpret_cast<const uint4*>(src + static_cast<int64_t>(s) * D);
    const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc[2 * e] = __fadd_rn(acc[2 * e], __uint_as_float(ww[e] << 16));
      acc[2 * e + 1] = __fadd_rn(acc[2 * e + 1], __uint_as_float(ww[e] & 0xffff0000u));
    }
  }
  float* dst = pooled + u * D + 8 * c;
#pragma unroll
  for (int e = 0; e < 8; ++e) dst[e] = n > 0 ? __fdiv_rn(acc[e], static_cast<float>(n)) : 0.0f;
  }
}

// ---- logits: g[bh][i][j] = sum_d qm[bh][i][d] * km[bh][j][d], d ascending, one fused -------
// ---- multiply-add per term (a single rounding each, as C's fmaf) ------------------------
// 64 x 64 logits per workgroup of 256 threads; thread (ty, tx) owns the 4 x 4 block of
// rows 4 ty .. 4 ty + 3 and columns 4 tx .. 4 tx + 3, each logit summed by that one
// thread over d ascending.  The pooled rows pass through LDS 32 columns of d at a time,
// transposed (d-major), so that a thread's four rows (columns) are one 16-byte read.
template <int D>
__global__ __launch_bounds__(256) void coarse_logits_kernel(const float* __restrict__ qm,
                                                            const float* __restrict__ km,
                                                            int num_tiles,
                                                            float* __restrict__ logits) {
  __shared__ __attribute__((aligned(16))) float qs[32][68];
  __shared__ __attribute__((aligned(16))) float ks[32][68];
  const int bh = blockIdx.z;
  const int i0 = blockIdx.y * 64, j0 = blockIdx.x * 64;
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const float* qh = qm + static_cast<int64_t>(bh) * num_tiles * D;
  const float* kh = km + static_cast<int64_t>(bh) * num_tiles * D;
  float acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = 0.0f;
  // 64 rows x 32 columns of each operand per round, 8 values per thread, the
  // next round's loaded into registers while the current one is computed
  float qv_next[8], kv_next[8];
  auto load = [&](int d0) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int idx = tid + 256 * e;  // 0 .. 2047
      const int row = idx >> 5, dd = idx & 31;
      const int i = i0 + row, j = j0 + row;
      qv_next[e] = i < num_tiles ? qh[static_cast<int64_t>(i) * D + d0 + dd] : 0.0f;
      kv_next[e] = j < num_tiles ? kh[static_cast<int64_t>(j) * D + d0 + dd] : 0.0f;
    }
  };
  load(0);
  for (int d0 = 0; d0 < D; d0 += 32) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int idx = tid + 256 * e;
      qs[idx & 31][idx >> 5] = qv_next[e];
      ks[idx & 31][idx >> 5] = kv_next[e];
    }
    __syncthreads();
    if (d0 + 32 < D) load(d0 + 32);
#pragma unroll 4
    for (int dd = 0; dd < 32; ++dd) {
      const float4 qa = *reinterpret_cast<const float4*>(&qs[dd][4 * ty]);
      const float4 kb = *reinterpret_cast<const float4*>(&ks[dd][4 * tx]);
      const float qv[4] = {qa.x, qa.y, qa.z, qa.w}, kv[4] = {kb.x, kb.y, kb.z, kb.w};
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = __fmaf_rn(qv[a], kv[b], acc[a][b]);
    }
    __syncthreads();
  }
  float* out = logits + static_cast<int64_t>(bh) * num_tiles * num_tiles;
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    const int i = i0 + 4 * ty + a;
    if (i >= num_tiles) continue;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int j = j0 + 4 * tx + b;
      if (j < num_tiles) out[static_cast<int64_t>(i) * num_tiles + j] = acc[a][b];
    }
  }
}

// ---- selection ------------------------------------------------------------------------
// Order-preserving image of a logit as an unsigned integer: a NaN ranks as -inf and -0
// as +0, and larger logits map to larger integers (0 is below every logit's image).
__device__ __forceinline__ uint32_t rank_image(float g) {
  if (g != g) g = -INFINITY;
  if (g == 0.0f) g = 0.0f;
  const uint32_t b = __float_as_uint(g);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ __forceinline__ int popc(uint64_t m) { return __popcll(m); }

__device__ __forceinline__ int lanes_below(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(m >> 32),
                                   __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m), 0));
}

// One wave per (bh, query tile i); key tile j = lane + 64 r is held in register r.
// Writes the list and the count, and (when weights are wanted) overwrites the logits
// row with the softmax weights of the coarse output: p_j / l over the non-empty key
// tiles, 0 elsewhere (all 0 for an empty query tile or one without candidates).
template <int KPL>
__global__ __launch_bounds__(256) void coarse_select_kernel(
    float* __restrict__ logits, const int32_t* __restrict__ vbs, int num_tiles, int64_t rows,
    int topk, int max_sel, float scale, int32_t* __restrict__ q2k_idx,
    int32_t* __restrict__ q2k_num, int weights) {
  const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;  // whole waves leave together
  const int i = static_cast<int>(row % num_tiles);
  float* grow = logits + row * num_tiles;
  int32_t* list = q2k_idx + row * max_sel;
  const bool q_valid = vbs[i] > 0;

  float gv[KPL];
  uint32_t key[KPL];
  int n_valid = 0;
#pragma unroll
  for (int r = 0; r < KPL; ++r) {
    const int j = lane + 64 * r;
    const bool ok = q_valid && j < num_tiles && vbs[j] > 0;
    gv[r] = ok ? grow[j] : 0.0f;
    key[r] = ok ? rank_image(gv[r]) : 0u;
    n_valid += popc(__ballot(ok));
  }
  const int k = topk < n_valid ? topk : n_valid;

  int written = 0;
  if (k > 0) {
    // the k-th largest image: the largest tau with #{key >= tau} >= k
    uint32_t tau = 0;
    for (int bit = 31; bit >= 0; --bit) {
      const uint32_t cand = tau | (1u << bit);
      int cnt = 0;
#pragma unroll
      for (int r = 0; r < KPL; ++r) cnt += popc(__ballot(key[r] >= cand));
      if (cnt >= k) tau = cand;
    }
    int above = 0;
#pragma unroll
    for (int r = 0; r < KPL; ++r) above += popc(__ballot(key[r] > tau));
    const int need = k - above;  // >= 1: how many of the tiles at tau are kept
    int eq_before = 0;
#pragma unroll
    for (int r = 0; r < KPL; ++r) {
      const bool eq = key[r] == tau;  // tau > 0, so never an empty or absent tile
      const uint64_t meq = __ballot(eq);
      const bool sel = key[r] > tau || (eq && eq_before + lanes_below(meq) < need);
      eq_before += popc(meq);
      const uint64_t msel = __ballot(sel);
      if (sel) list[written + lanes_below(msel)] = lane + 64 * r;
      written += popc(msel);
    }
  }
  for (int n = written + lane; n < max_sel; n += 64) list[n] = -1;
  if (lane == 0) q2k_num[row] = written;

  if (!weights) return;
  // softmax weights over the non-empty key tiles (a NaN logit is NaN here, as the
  // plain formula propagates it)
  float m = -INFINITY;
#pragma unroll
  for (int r = 0; r < KPL; ++r)
    if (key[r] != 0u) m = fmaxf(m, scale * gv[r]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  float p[KPL], l = 0.0f;
#pragma unroll
  for (int r = 0; r < KPL; ++r) {
    p[r] = key[r] != 0u ? __expf(scale * gv[r] - m) : 0.0f;
    l += p[r];
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) l += __shfl_xor(l, off);
  const bool any = n_valid > 0;
#pragma unroll
  for (int r = 0; r < KPL; ++r) {
    const int j = lane + 64 * r;
    if (j < num_tiles) grow[j] = any ? p[r] / l : 0.0f;
  }
}

// ---- coarse output: oc[bh][i][:] = sum_j w[bh][i][j] * vm[bh][j][:] -----------------------
// fp32 MFMA (v_mfma_f32_32x32x2_f32): a workgroup of 4 waves per 32 query tiles x 32
// columns, each wave a quarter of the key-tile range, the four partial blocks added in
// LDS.  Lane l feeds A[l % 32][l / 32] = w[i0 + l % 32][j] and B[l / 32][l % 32] =
// vm[j][c0 + l % 32] with j = jq + (l / 32) * half + step for the wave's quarter
// starting at jq: the two halves of the quarter run side by side in the instruction's
// two k slots, and each lane reads its weights row contiguously.  C (32 x 32): lane l,
// register r holds C[8 (r / 4) + 4 (l / 32) + r % 4][l % 32].  The order of the sum is
// free here (the output is compared within a tolerance); the logits, which decide the
// lists, are formed apart in a fixed order.
// Coarse output rows i0 .. i0 + 31 of one head: wave c computes columns
// 32c .. 32c + 31 over every key tile with v_mfma_f32_32x32x2f32 (A: 32 weight
// rows x 2 key tiles, one value per lane; B: 2 pooled-value rows x 32
// columns).  The weight rows and the pooled values of 128 key tiles at a time
// are staged in LDS with coalesced loads, the next chunk's issued before the
// current chunk's products (a lane's A value is one float of a different row,
// so reading it from memory directly would leave each MFMA waiting on
// scattered loads).
template <int D>
__global__ __launch_bounds__(256) void coarse_out_kernel(const float* __restrict__ w,
                                                         const float* __restrict__ vm,
                                                         int num_tiles, float* __restrict__ oc) {
  constexpr int kChunk = 128, kStride = kChunk + 1;  // padded weight rows: no bank conflicts
  constexpr int kWLoads = 32 * kChunk / 256;         // weight floats per thread and chunk
  constexpr int kVLoads = kChunk * D / 4 / 256;      // pooled-value float4s per thread and chunk
  __shared__ float ws[32 * kStride];
  __shared__ float4 vs[kChunk * D / 4];
  const int bh = blockIdx.z;
  const int i0 = blockIdx.x * 32;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 31, h = lane >> 5;
  const int c0 = 32 * wave;
  const float* wh = w + static_cast<int64_t>(bh) * num_tiles * num_tiles;
  const float4* vh = reinterpret_cast<const float4*>(vm + static_cast<int64_t>(bh) * num_tiles * D);
  const float* vsf = reinterpret_cast<const float*>(vs);
  f32x16_t acc = {};
  float wl[kWLoads];
  float4 vl[kVLoads];
  // chunk jc's loads into registers; they land while the previous chunk's
  // products run
  auto load = [&](int jc) {
    const int n = num_tiles - jc < kChunk ? num_tiles - jc : kChunk;
#pragma unroll
    for (int u = 0; u < kWLoads; ++u) {
      const int e = tid + 256 * u, rr = e / kChunk, cc = e % kChunk, i = i0 + rr;
      wl[u] = i < num_tiles && cc < n ? wh[static_cast<int64_t>(i) * num_tiles + jc + cc] : 0.0f;
    }
#pragma unroll
    for (int u = 0; u < kVLoads; ++u) {
      const int e = tid + 256 * u, jj = e / (D / 4);
      vl[u] = jj < n ? vh[static_cast<int64_t>(jc) * (D / 4) + e] : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    }
  };
  load(0);
  for (int jc = 0; jc < num_tiles; jc += kChunk) {
    __syncthreads();  // every wave is done with the previous chunk
#pragma unroll
    for (int u = 0; u < kWLoads; ++u) {
      const int e = tid + 256 * u;
      ws[(e / kChunk) * kStride + e % kChunk] = wl[u];
    }
#pragma unroll
    for (int u = 0; u < kVLoads; ++u) vs[tid + 256 * u] = vl[u];
    __syncthreads();
    if (jc + kChunk < num_tiles) load(jc + kChunk);
    if (c0 < D) {
      // operands read from LDS one batch of kB steps ahead of the MFMAs that use
      // them; step t takes key tile 2t + h (zeros past the chunk's end)
      constexpr int kB = 8, kSteps = kChunk / 2;
      float a[2][kB], b[2][kB];
      auto read = [&](int t0, int x) {
#pragma unroll
        for (int u = 0; u < kB; ++u) {
          const int j = 2 * (t0 + u) + h;
          a[x][u] = ws[r * kStride + j];
          b[x][u] = vsf[j * D + c0 + r];
        }
      };
      read(0, 0);
#pragma unroll
      for (int t0 = 0; t0 < kSteps; t0 += kB) {
        const int x = (t0 / kB) & 1;
        if (t0 + kB < kSteps) read(t0 + kB, x ^ 1);
#pragma unroll
        for (int u = 0; u < kB; ++u)
          acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[x][u], b[x][u], acc, 0, 0, 0);
      }
    }
  }
  if (c0 >= D) return;
#pragma unroll
  for (int g = 0; g < 16; ++g) {
    const int row = i0 + 8 * (g >> 2) + 4 * h + (g & 3);
    if (row < num_tiles) oc[(static_cast<int64_t>(bh) * num_tiles + row) * D + c0 + r] = acc[g];
  }
}

// 8 bf16 outputs of one row, out + gate * coarse output in fp32, then one
// rounding (RNE) to bf16: the combine's arithmetic, shared by both kernels
// that apply it so that they give the same bits.
__device__ __forceinline__ uint4 combine_chunk(uint4 o, uint4 gt, const float* __restrict__ cv) {
  const uint32_t ow[4] = {o.x, o.y, o.z, o.w}, gw[4] = {gt.x, gt.y, gt.z, gt.w};
  uint32_t res[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float lo = __uint_as_float(ow[e] << 16) + __uint_as_float(gw[e] << 16) * cv[2 * e];
    const float hi = __uint_as_float(ow[e] & 0xffff0000u) +
                     __uint_as_float(gw[e] & 0xffff0000u) * cv[2 * e + 1];
    res[e] = __builtin_bit_cast(uint32_t, to_bf16x2(lo, hi));
  }
  return make_uint4(res[0], res[1], res[2], res[3]);
}

// ---- out += gate * coarse output of the row's tile (valid rows only) ----------------------
template <int D>
__global__ __launch_bounds__(256) void coarse_combine_kernel(uint16_t* __restrict__ out,
                                                             const uint16_t* __restrict__ gate,
                                                             const float* __restrict__ oc,
                                                             const int32_t* __restrict__ vbs,
                                                             int num_tiles, int tile,
                                                             int64_t rows) {
  constexpr int kChunks = D / 8;
  const int64_t total = rows * kChunks;
  for (int64_t g = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; g < total;
       g += static_cast<int64_t>(gridDim.x) * 256) {
  const int64_t row = g / kChunks;
  const int c = static_cast<int>(g - row * kChunks);
  const int64_t bht = row / tile;  // bh * NT + t
  const int t = static_cast<int>(bht % num_tiles);
  if (static_cast<int>(row - bht * tile) >= clampi(vbs[t], 0, tile)) continue;  // padding stays +0
  uint4* po = reinterpret_cast<uint4*>(out + row * D + 8 * c);
  const uint4 o = *po;
  const uint4 gt = *reinterpret_cast<const uint4*>(gate + row * D + 8 * c);
  const float* cv = oc + bht * D + 8 * c;
  *po = combine_chunk(o, gt, cv);
  }
}

// The combine and the way back in one pass: token-major output row n of head h
// is tile row r = token_row[n] of the fine output, combined as above when r is
// a valid row of its tile and passed through otherwise (the padding rows the
// combine leaves alone), or +0 when r is out of range: the bits bsa_tile_unlayout
// gives after bsa_coarse_combine, without writing the tile buffer back.  One
// 16-byte chunk per thread, chunk index fastest, then head, then token.
template <int D>
__global__ __launch_bounds__(256) void unlayout_combine_kernel(
    const uint16_t* __restrict__ out, const uint16_t* __restrict__ gate,
    const float* __restrict__ oc, const int32_t* __restrict__ vbs,
    const int32_t* __restrict__ token_row, int64_t tokens, int64_t heads, int num_tiles, int tile,
    uint16_t* __restrict__ dst) {
  constexpr int kChunks = D / 8;
  const int64_t b = blockIdx.y;
  const int64_t chunks = tokens * heads * kChunks;  // per batch
  const int64_t rows_per_head = static_cast<int64_t>(num_tiles) * tile;
  for (int64_t g = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; g < chunks;
       g += static_cast<int64_t>(gridDim.x) * 256) {
    const int c = static_cast<int>(g % kChunks);
    const int64_t th = g / kChunks;  // token * heads + head
    const int64_t n = th / heads;
    const int64_t h = th - n * heads;
    const int32_t r = token_row[n];
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (r >= 0 && r < rows_per_head) {
      const int64_t bh = b * heads + h;
      const int64_t off = (bh * rows_per_head + r) * D + 8 * c;
      v = *reinterpret_cast<const uint4*>(out + off);
      const int t = r / tile;
      if (r - t * tile < clampi(vbs[t], 0, tile))
        v = combine_chunk(v, *reinterpret_cast<const uint4*>(gate + off),
                          oc + (bh * num_tiles + t) * D + 8 * c);
    }
    *reinterpret_cast<uint4*>(dst + (b * chunks + g) * 8) = v;
  }
}

// Grid of a grid-stride launch over `threads` work items, 256 per workgroup.
unsigned stride_grid(int64_t threads) {
  const int64_t blocks = (threads + 255) / 256;
  return static_cast<unsigned>(blocks < (int64_t{1} << 20) ? (blocks > 0 ? blocks : 1) : (int64_t{1} << 20));
}

template <int D>
hipError_t launch_coarse_d(const bsa::CoarseProblem& p, hipStream_t stream) {
  const int64_t tiles_all = p.batch_heads * p.num_tiles;
  // pooled rows: formed here (in the workspace, before the logits), or given
  const float* qm = p.pooled ? p.pooled : p.ws;
  const float* km = qm + tiles_all * D;
  const float* vm = km + tiles_all * D;
  float* logits = p.pooled ? p.ws : p.ws + 3 * tiles_all * D;
  if (!p.pooled) {
    const int64_t threads = 3 * tiles_all * (D / 8);
    hipLaunchKernelGGL(coarse_pool_kernel<D>, dim3(stride_grid(threads)),
                       dim3(256), 0, stream, p.q, p.k, p.v, p.block_sizes, p.num_tiles, p.tile,
                       tiles_all, p.ws);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  const unsigned nb = static_cast<unsigned>((p.num_tiles + 63) / 64);
  hipLaunchKernelGGL(coarse_logits_kernel<D>, dim3(nb, nb, static_cast<unsigned>(p.batch_heads)),
                     dim3(256), 0, stream, qm, km, p.num_tiles, logits);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const float scale = static_cast<float>(1.0 / __builtin_sqrt(static_cast<double>(D)));
  const int weights = p.coarse_out != nullptr ? 1 : 0;
  const dim3 sgrid(static_cast<unsigned>((tiles_all + 3) / 4));
  if (p.num_tiles <= 256)
    hipLaunchKernelGGL(coarse_select_kernel<4>, sgrid, dim3(256), 0, stream, logits,
                       p.block_sizes, p.num_tiles, tiles_all, p.topk, p.max_sel, scale, p.q2k_idx,
                       p.q2k_num, weights);
  else if (p.num_tiles <= 512)
    hipLaunchKernelGGL(coarse_select_kernel<8>, sgrid, dim3(256), 0, stream, logits,
                       p.block_sizes, p.num_tiles, tiles_all, p.topk, p.max_sel, scale, p.q2k_idx,
                       p.q2k_num, weights);
  else if (p.num_tiles <= 1024)
    hipLaunchKernelGGL(coarse_select_kernel<16>, sgrid, dim3(256), 0, stream, logits,
                       p.block_sizes, p.num_tiles, tiles_all, p.topk, p.max_sel, scale, p.q2k_idx,
                       p.q2k_num, weights);
  else
    hipLaunchKernelGGL(coarse_select_kernel<64>, sgrid, dim3(256), 0, stream, logits,
                       p.block_sizes, p.num_tiles, tiles_all, p.topk, p.max_sel, scale, p.q2k_idx,
                       p.q2k_num, weights);
  err = hipGetLastError();
  if (err != hipSuccess || !weights) return err;
  hipLaunchKernelGGL(coarse_out_kernel<D>,
                     dim3(static_cast<unsigned>((p.num_tiles + 31) / 32), 1,
                          static_cast<unsigned>(p.batch_heads)),
                     dim3(256), 0, stream, logits, vm, p.num_tiles, p.coarse_out);
  return hipGetLastError();
}

}  // namespace

namespace bsa {

size_t coarse_workspace_bytes(int64_t batch_heads, int64_t num_tiles, int32_t head_dim) {
  return static_cast<size_t>(batch_heads) * static_cast<size_t>(num_tiles) *
         (3 * static_cast<size_t>(head_dim) + static_cast<size_t>(num_tiles)) * sizeof(float);
}

hipError_t launch_coarse(const CoarseProblem& p, hipStream_t stream) {
  return p.head_dim == 128 ? launch_coarse_d<128>(p, stream) : launch_coarse_d<64>(p, stream);
}

hipError_t launch_unlayout_combine(const UnlayoutCombineProblem& p, hipStream_t stream) {
  const int64_t chunks = p.tokens * p.heads * (p.head_dim / 8);
  const int64_t want = (chunks + 255) / 256;
  const dim3 grid(static_cast<unsigned>(want < 65536 ? want : 65536), static_cast<unsigned>(p.batch));
  if (p.head_dim == 128)
    hipLaunchKernelGGL(unlayout_combine_kernel<128>, grid, dim3(256), 0, stream, p.out, p.gate,
                       p.coarse_out, p.block_sizes, p.token_row, p.tokens, p.heads, p.num_tiles,
                       p.tile, p.dst);
  else
    hipLaunchKernelGGL(unlayout_combine_kernel<64>, grid, dim3(256), 0, stream, p.out, p.gate,
                       p.coarse_out, p.block_sizes, p.token_row, p.tokens, p.heads, p.num_tiles,
                       p.tile, p.dst);
  return hipGetLastError();
}

hipError_t launch_coarse_combine(const CombineProblem& p, hipStream_t stream) {
  const dim3 grid(stride_grid(p.rows * (p.head_dim / 8)));
  if (p.head_dim == 128)
    hipLaunchKernelGGL(coarse_combine_kernel<128>, grid, dim3(256), 0, stream, p.out, p.gate,
                       p.coarse_out, p.block_sizes, p.num_tiles, p.tile, p.rows);
  else
    hipLaunchKernelGGL(coarse_combine_kernel<64>, grid, dim3(256), 0, stream, p.out, p.gate,
                       p.coarse_out, p.block_sizes, p.num_tiles, p.tile, p.rows);
  return hipGetLastError();
}

}  // namespace bsa
