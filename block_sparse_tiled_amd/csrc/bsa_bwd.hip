// Block-sparse tiled attention backward for gfx950 (AMD Instinct MI355X).
//
// FastVideo fastvideo-kernel commit list, page 3: the 128-token sm_121a
// forward commit keeps its binding to the forward because another route's
// log-sum-exp output feeds an autograd path; the Attn-QAT commit describes a
// backward of 64x128 dQ and dK/dV tiles.  The pages print no backward
// formulas; these kernels compute the gradients of the plain forward
// definition (softmax over the listed tiles' valid keys), per query row r:
//   P = exp(scale * q_r K^T - lse_r),  dP = dO_r V^T,  D_r = dO_r . out_r,
//   dS = P * (dP - D_r),  dq_r = scale * dS K,  dK += scale * dS^T q_r,
//   dV += P^T dO_r.
//
// Kernels (all bf16 MFMA 32x32x16 with fp32 accumulation, operands staged in
// LDS by LDS DMA with the forward's K-tile swizzle):
//   - k2q_count_kernel / k2q_kernel: the transposed lists (for each key
//     tile, the query tiles whose lists name it, ascending, a tile listed
//     twice appearing twice), built deterministically: counted in LDS per
//     (head, range of key tiles) and written by a parallel walk, or, for
//     heads too large to count, one wave per key tile scanning the lists in
//     order with a ballot-ordered append.
//   - delta_kernel: D_r = dO_r . o_r in fp32 (0 for padding rows), with o_r
//     the forward's fp32 result rebuilt as out + out_lo (the stored bf16
//     output plus its bf16 rounding residual).  On a peaked row dS = P(dP - D)
//     is a small difference of nearly equal terms, and D from the bf16 out
//     alone would carry an error of 2^-9 of |dO||o|, which then dominates dq
//     and dk.
//   - dq_kernel: one workgroup per query tile, T/32 waves of 32 query rows;
//     per listed key tile, in halves of 64 keys: S^T = K Q^T, P^T, dP^T =
//     V dO^T, dS^T, then dQ^T += K^T dS^T (the K^T operand through the LDS
//     transpose read).  Q and dO stay in registers as B operands.  K and V
//     are copied in the same 64-key halves, each half of the next tile as
//     soon as every wave is done with that half of the current one.
//   - dkv_kernel: one workgroup per key tile, T/32 waves of 32 key rows;
//     per query tile of its transposed list, in blocks of 32 queries: S =
//     Q K^T, P, dP = dO V^T, dS, then dV^T += dO^T P and dK^T += Q^T dS (dO^T
//     and Q^T through the LDS transpose read).  K and V stay in registers.
//     The blocks are software-pipelined (kDkvPipe): at D = 128, with two
//     register sets for S/dP and P/dS, one block's dV/dK products, a later
//     block's S/dP products and the next block's softmax share each period;
//     at D = 64 the next block's S/dP products go between the current block's
//     dV/dK products.  At D = 128 the next query tile's copies are issued one
//     instruction at a time among the products.
//   The C-layout-to-B-operand reuse and the key (query) order within a
//   16-wide chunk are those of the forward (bsa_fwd_common.h).
//
// Padding and special values: padding key rows (K, V) and padding query rows
// (Q, dO) are zeroed in LDS after their copy lands, so NaN or Inf there never
// meets a zero weight; padding query rows get P = 0 in dkv_kernel (their
// staged lse is +inf); rows without keys have no tiles in dq_kernel and appear
// in no transposed list; every gradient row of a padding token is written +0.
// A row whose softmax sum is NaN (lse NaN, or -inf with keys present)
// propagates NaN, as the plain formula does.
#include <hip/hip_runtime.h>

#include <type_traits>
#include <utility>

#include "bsa_fwd_common.h"
#include "bsa_launch.h"

namespace {

using namespace bsa::detail;

// ---- transposed lists ---------------------------------------------------------------------
// One wave per (head, key tile j) scans the head's lists in order (ascending
// query tile, then list position) and appends i for every live entry equal
// to j through a ballot-ordered prefix.  The scan is bound by load latency,
// so lists of up to 256 positions are read as one flat range of [NT][MS]
// entries, eight 64-entry loads (and their rows' counts) issued at a time
// before any of them is used.  Wider lists, whose counts may be far below
// their width, are read row by row (the count read once per row, only the
// positions below it loaded).
__device__ __forceinline__ void k2q_append(bool hit, int value, int& count, int32_t* dst, int max_k,
                                           int lane) {
  const uint64_t m = __ballot(hit);
  if (hit) {
    (void)lane;
    const int at = count + __builtin_amdgcn_mbcnt_hi(
                               static_cast<uint32_t>(m >> 32),
                               __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m), 0));
    if (at < max_k) dst[at] = value;
  }
  count += __popcll(m);
}

__global__ __launch_bounds__(256) void k2q_kernel(const int32_t* __restrict__ q2k_idx,
                                                  const int32_t* __restrict__ q2k_num,
                                                  int num_tiles, int max_sel, int64_t n_lists,
                                                  int32_t* __restrict__ k2q_idx,
                                                  int32_t* __restrict__ k2q_num, int max_k) {
  constexpr int kU = 8;
  const int64_t wid = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (wid >= n_lists) return;  // whole waves leave together
  const int64_t bh = wid / num_tiles;
  const int j = static_cast<int>(wid - bh * num_tiles);
  const int64_t entries = static_cast<int64_t>(num_tiles) * max_sel;
  const int32_t* idx_h = q2k_idx + bh * entries;
  const int32_t* num_h = q2k_num + bh * num_tiles;
  int32_t* dst = k2q_idx + wid * max_k;
  int count = 0;
  if (max_sel > 256 || entries + 64 * kU >= (int64_t{1} << 31)) {
    for (int i = 0; i < num_tiles; ++i) {
      const int n = clampi(num_h[i], 0, max_sel);
      for (int base = 0; base < n; base += 64) {
        const int e = base + lane;
        k2q_append(e < n && idx_h[static_cast<int64_t>(i) * max_sel + e] == j, i, count, dst, max_k,
                   lane);
      }
    }
  } else {
    const uint32_t ms = static_cast<uint32_t>(max_sel);  // entries < 2^31 here
    const uint32_t last = static_cast<uint32_t>(entries - 1);
    for (uint32_t base = 0; base < entries; base += 64 * kU) {
      // every load first, at positions clamped into the head's range, so that
      // they are in flight together; positions past the range never hit
      int x[kU], n[kU], row[kU], e[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const uint32_t pos = base + 64 * u + lane;
        const uint32_t pc = pos < entries ? pos : last;
        row[u] = static_cast<int>(pc / ms);
        e[u] = static_cast<int>(pc - row[u] * ms);
        x[u] = idx_h[pc];
        n[u] = num_h[row[u]];
      }
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const bool hit =
            base + 64 * u + lane < entries && e[u] < clampi(n[u], 0, max_sel) && x[u] == j;
        k2q_append(hit, row[u], count, dst, max_k, lane);
      }
    }
  }
  if (lane == 0) k2q_num[wid] = count;  // the true count (the list holds the first max_k)
}

// The same lists by counting, for heads whose lists fit: one workgroup per
// (head, range of J key tiles) counts in LDS, with 16-bit counters two to a
// word, how often each list i names each key tile j of its range; then thread
// jj walks i = 0 .. NT-1 and appends i as often as list i names j0 + jj.  The
// counts fix the output, so the atomic increments leave it deterministic, and
// it equals the scan's: ascending i, a tile named twice appearing twice.  The
// pass over the lists is bound by load latency: each thread issues eight
// loads, 1024 entries apart, before it uses any.
constexpr int kCountWords = 16384;     // 64 KiB of counter pairs
constexpr int kCountMaxTiles = 4096;   // the clamped list lengths staged in LDS
constexpr int kCountThreads = 1024;
__global__ __launch_bounds__(kCountThreads) void k2q_count_kernel(
    const int32_t* __restrict__ q2k_idx, const int32_t* __restrict__ q2k_num, int num_tiles,
    int max_sel, int span, int groups, int32_t* __restrict__ k2q_idx, int32_t* __restrict__ k2q_num,
    int max_k) {
  constexpr int kU = 8;
  __shared__ uint32_t cnt[kCountWords];
  __shared__ int nums[kCountMaxTiles];
  const int64_t bh = blockIdx.x / groups;
  const int j0 = static_cast<int>(blockIdx.x - bh * groups) * span;
  const int tid = threadIdx.x;
  const int NT = num_tiles, MS = max_sel, J = span;
  const int words = NT * (J / 2);
  for (int w = tid; w < words; w += kCountThreads) cnt[w] = 0;
  const int32_t* num_h = q2k_num + bh * NT;
  for (int i = tid; i < NT; i += kCountThreads) nums[i] = clampi(num_h[i], 0, MS);
  __syncthreads();
  if (MS > 0) {
    // entry e = i * MS + pos; the thread's entries lie kCountThreads apart, so
    // (i, pos) advances by (di, dp) with at most one carry
    const int32_t* idx_h = q2k_idx + bh * static_cast<int64_t>(NT) * MS;
    const uint32_t total = static_cast<uint32_t>(NT) * static_cast<uint32_t>(MS);
    const uint32_t last = total - 1;
    const int di = kCountThreads / MS, dp = kCountThreads % MS;
    int i = tid / MS, pos = tid % MS;
    for (uint32_t base = tid; base < total; base += kU * kCountThreads) {
      int x[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const uint32_t e = base + u * kCountThreads;
        x[u] = idx_h[e < total ? e : last];
      }
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        if (base + u * kCountThreads < total && pos < nums[i] && x[u] >= j0 && x[u] < j0 + J &&
            x[u] < NT) {
          const int jj = x[u] - j0;
          atomicAdd(&cnt[(i * J + jj) >> 1], 1u << (16 * (jj & 1)));
        }
        pos += dp;
        i += di;
        if (pos >= MS) {
          pos -= MS;
          ++i;
        }
      }
    }
  }
  __syncthreads();
  // The walk, in parallel: key tile j0 + jj's rows are cut into R blocks,
  // thread (r, jj) taking block r.  Pass 1 sums each block's counts (into the
  // space of the list lengths, no longer needed); each thread's start is the
  // sum over the blocks before it; pass 2 writes its entries from there.
  const int R = kCountThreads / J;
  const int jj = tid % J, r = tid / J, j = j0 + jj;
  const bool walker = r < R && j < NT;
  const int rows_per = (NT + R - 1) / R;
  const int i_begin = r * rows_per < NT ? r * rows_per : NT;
  const int i_end = i_begin + rows_per < NT ? i_begin + rows_per : NT;
  const int shift = 16 * (jj & 1);
  auto count_at = [&](int i) { return static_cast<int>((cnt[(i * J + jj) >> 1] >> shift) & 0xFFFFu); };
  int sum = 0;
  if (walker)
#pragma unroll 4
    for (int i = i_begin; i < i_end; ++i) sum += count_at(i);
  __syncthreads();  // every thread is done with nums[]
  int* part = nums;  // [R][J] block sums
  if (r < R) part[r * J + jj] = walker ? sum : 0;
  __syncthreads();
  if (walker) {
    int at = 0, total = 0;
    for (int q = 0; q < R; ++q) {
      const int v = part[q * J + jj];
      at += q < r ? v : 0;
      total += v;
    }
    if (r == 0) k2q_num[bh * NT + j] = total;
    int32_t* dst = k2q_idx + (bh * NT + j) * static_cast<int64_t>(max_k);
    for (int i = i_begin; i < i_end && at < max_k; ++i)
      for (int c = count_at(i); c > 0; --c, ++at)
        if (at < max_k) dst[at] = i;
  }
}

// ---- D = rowsum(dO * (out + out_lo)) ------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void delta_kernel(const uint16_t* __restrict__ out,
                                                    const uint16_t* __restrict__ out_lo,
                                                    const uint16_t* __restrict__ dout,
                                                    const int32_t* __restrict__ vbs, int num_tiles,
                                                    int tile, int64_t rows,
                                                    float* __restrict__ delta, int sub_shift) {
  constexpr int kLanes = D / 8;  // lanes per row, 8 bf16 each
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t row = gid / kLanes;
  const int part = static_cast<int>(gid % kLanes);
  float acc = 0.0f;
  bool valid = false;
  if (row < rows) {
    const int64_t r = row % (static_cast<int64_t>(num_tiles) * tile);
    const int t = static_cast<int>(r / tile);
    const int vq = clampi(vbs[t >> sub_shift] - tile * (t & ((1 << sub_shift) - 1)), 0, tile);
    valid = static_cast<int>(r % tile) < vq;
    if (valid) {
      const uint4 o = *reinterpret_cast<const uint4*>(out + row * D + 8 * part);
      const uint4 ol = *reinterpret_cast<const uint4*>(out_lo + row * D + 8 * part);
      const uint4 g = *reinterpret_cast<const uint4*>(dout + row * D + 8 * part);
      const uint32_t ow[4] = {o.x, o.y, o.z, o.w}, lw[4] = {ol.x, ol.y, ol.z, ol.w};
      const uint32_t gw[4] = {g.x, g.y, g.z, g.w};
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        acc += (__uint_as_float(ow[x] << 16) + __uint_as_float(lw[x] << 16)) *
               __uint_as_float(gw[x] << 16);
        acc += (__uint_as_float(ow[x] & 0xffff0000u) + __uint_as_float(lw[x] & 0xffff0000u)) *
               __uint_as_float(gw[x] & 0xffff0000u);
      }
    }
  }
#pragma unroll
  for (int off = kLanes / 2; off >= 1; off >>= 1) acc += __shfl_xor(acc, off);
  if (row < rows && part == 0) delta[row] = valid ? acc : 0.0f;
}

// ---- LDS operand reads shared by the two gradient kernels --------------------------------
// A operand (32 rows x 16 of the D axis) from rows [row0, row0 + 32) of a
// K-swizzled tile: lane l reads row row0 + l % 32, columns 16*kk + 8*half ..
template <int D>
__device__ __forceinline__ bf16x8_t read_rows(const uint16_t* tile, int row0, int kk, int col,
                                              int half) {
  const int row = row0 + col;
  const int chunk = (2 * kk + half) ^ swz_k<D>(row);
  return __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(tile + row * D + 8 * chunk));
}

// A operand (32 of the D axis x 16 rows) = the transpose of rows [16c, 16c + 16)
// of a K-swizzled tile, columns 32*db .. 32*db + 31, rows in the forward's
// order within a 16-wide chunk (element e of half h is row 8*(e/4) + 4*h + e%4).
template <int D>
__device__ __forceinline__ bf16x8_t read_rows_t(const uint16_t* tile, int c, int db, int lane) {
  const int tr_i = lane & 15, tr_g = (lane >> 4) & 1, half = lane >> 5;
  const int row_lo = 16 * c + 4 * half + (tr_i >> 2);
  const int row_hi = row_lo + 8;
  const int colv = 32 * db + 16 * tr_g + 4 * (tr_i & 3);
  const int off_lo = ((colv >> 3) ^ swz_k<D>(row_lo)) * 8 + (colv & 7);
  const int off_hi = ((colv >> 3) ^ swz_k<D>(row_hi)) * 8 + (colv & 7);
  const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(tile + row_lo * D + off_lo));
  const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(tile + row_hi * D + off_hi));
  return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// bf16 B operand from eight fp32 values of an accumulator (registers e0 .. e0+7).
__device__ __forceinline__ bf16x8_t pack8(const f32x16_t& x, int e0) {
  const bf16x2_t a = to_bf16x2(x[e0 + 0], x[e0 + 1]);
  const bf16x2_t b = to_bf16x2(x[e0 + 2], x[e0 + 3]);
  const bf16x2_t c = to_bf16x2(x[e0 + 4], x[e0 + 5]);
  const bf16x2_t d = to_bf16x2(x[e0 + 6], x[e0 + 7]);
  return __builtin_shufflevector(__builtin_shufflevector(a, b, 0, 1, 2, 3),
                                 __builtin_shufflevector(c, d, 0, 1, 2, 3), 0, 1, 2, 3, 4, 5, 6, 7);
}

// Store a D^T x 32 accumulator set (lane = row col, register r of block db =
// column 32*db + 8*(r/4) + 4*half + r%4) as bf16 rows, times `mul`; +0 rows
// where `zero`.
template <int D>
__device__ __forceinline__ void store_t(uint16_t* dst_row, const f32x16_t* acc, float mul,
                                        bool zero, int half) {
  constexpr int NDB = D / 32;
  uint16_t* dst = dst_row + 4 * half;
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      float x[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] = zero ? 0.0f : acc[db][4 * g + e] * mul;
      uint2 pk;
      pk.x = __builtin_bit_cast(unsigned, to_bf16x2(x[0], x[1]));
      pk.y = __builtin_bit_cast(unsigned, to_bf16x2(x[2], x[3]));
      *reinterpret_cast<uint2*>(dst + 32 * db + 8 * g) = pk;
    }
}

// Work item of linear workgroup id L (whole set only), XCD-aware as in the
// forward: XCD x = L % 8 receives a contiguous run of items.
__device__ __forceinline__ int item_of(int L, int n_padded) {
  return (L & 7) * (n_padded >> 3) + (L >> 3);
}

// Instructions [kLo, kHi) of a dma_tile copy of the first `rows` rows of a
// T x D tile (every one issued; lanes past `rows` fail the range check and
// read nothing), and the zeroing of padding-row slots those instructions
// filled: instruction it of a wave fills 1 KiB block it*kWaves + wave, so a
// contiguous range of instructions covers a contiguous range of rows.
template <int T, int D, int kLo, int kHi>
__device__ __forceinline__ void dma_tile_part(const uint16_t* __restrict__ src, uint16_t* lds, int wave,
                                              const DmaLane<T, D, false>& dl, int rows) {
  using C = Cfg<T, D>;
  using DL = DmaLane<T, D, false>;
  const uint32_t base = launder_s(__builtin_amdgcn_readfirstlane(lds_address(lds)) + wave * 1024);
  const uint64_t g = reinterpret_cast<uintptr_t>(src);
  const i32x4_t srd = {static_cast<int>(static_cast<uint32_t>(g)),
                       static_cast<int>(static_cast<uint32_t>(g >> 32)), rows * D * 2, 0x00020000};
#pragma unroll
  for (int it = kLo; it < kHi; ++it) {
    const uint32_t soff = it * C::kWaves * 1024;
    dma16(srd, dl.off[it % DL::kN], soff, base + soff);
  }
}
// The copy dma_tile<T, D, kIsV, kSkip> makes, one instruction at a time:
// set() takes the tile's source, LDS buffer and valid rows; one<it, kSkip>()
// issues instruction `it` of this wave (with kSkip, not when its whole block
// lies past the valid rows), so that a caller can spread a tile's copies over
// other work.
template <int T, int D, bool kIsV>
struct TileCopy {
  i32x4_t srd;
  uint32_t base;
  int rows;
  __device__ __forceinline__ void set(const uint16_t* __restrict__ src, uint16_t* lds, int wave,
                                      int valid_rows) {
    base = launder_s(__builtin_amdgcn_readfirstlane(lds_address(lds)) + wave * 1024);
    const uint64_t g = reinterpret_cast<uintptr_t>(src);
    srd = i32x4_t{static_cast<int>(static_cast<uint32_t>(g)),
                  static_cast<int>(static_cast<uint32_t>(g >> 32)), valid_rows * D * 2, 0x00020000};
    rows = valid_rows;
  }
  template <int it, bool kSkip>
  __device__ __forceinline__ void one(const DmaLane<T, D, kIsV>& dl, int wave) const {
    using C = Cfg<T, D>;
    constexpr int kRowsPerBlock = 512 / D;
    constexpr uint32_t soff = it * C::kWaves * 1024;
    if (!kSkip || (it * C::kWaves + wave) * kRowsPerBlock < rows)
      dma16(srd, dl.off[it % DmaLane<T, D, kIsV>::kN], soff, base + soff);
  }
};

template <int T, int D, int kLo, int kHi>
__device__ __forceinline__ void zero_padding_part(uint16_t* lds, int vk, int wave, int lane) {
  using C = Cfg<T, D>;
  constexpr int kRowsPerBlock = 64 / C::kChunks;
  const int lane_row = launder(lane) / C::kChunks;
  uint4* slot = reinterpret_cast<uint4*>(lds) + lane;
#pragma unroll
  for (int it = kLo; it < kHi; ++it) {
    const int blk = it * C::kWaves + wave;
    if (vk < (blk + 1) * kRowsPerBlock && lane_row >= vk - blk * kRowsPerBlock)  // uniform test first
      slot[blk * 64] = make_uint4(0u, 0u, 0u, 0u);
  }
}

// Calls f(std::integral_constant<int, P>) for P = 0 .. N-1, in order.
template <typename F, int... P>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, P...>) {
  (f(std::integral_constant<int, P>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}
// ---- dQ -----------------------------------------------------------------------------------
template <int T, int D>
__global__ __launch_bounds__(2 * T) __attribute__((amdgpu_waves_per_eu(2, T == 128 ? 2 : 4)))
void dq_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
               const uint16_t* __restrict__ v, const uint16_t* __restrict__ dout,
               const float* __restrict__ lse, const float* __restrict__ delta,
               const int32_t* __restrict__ q2k_idx, const int32_t* __restrict__ q2k_num,
               const int32_t* __restrict__ vbs, uint16_t* __restrict__ dq, int num_tiles,
               int max_sel, int n_items, int n_padded, float c, float scale, int sub_shift) {
  using C = Cfg<T, D>;
  constexpr int NDB = C::kDBlocks;
  __shared__ __attribute__((aligned(1024))) uint16_t ks[T * D];
  __shared__ __attribute__((aligned(1024))) uint16_t vs[T * D];
  // the steps of the current list chunk (compact_steps, as in the forward): a
  // tile, or, at T = 128, two tiles that fit in T rows together (at T = 64 the
  // pair's copy code made the compiler schedule the S/dP products worse)
  constexpr bool kPairs = T == 128;
  __shared__ int2 st[2 * (T == 128 ? 2 : 1) * C::kThreads];
  __shared__ int2 srt[kPairs ? 2 * C::kThreads : 1];
  __shared__ int wave_scratch[5 * C::kWaves];

  const int item = item_of(blockIdx.x, n_padded);
  if (item >= n_items) return;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31;
  const int half = lane >> 5;
  const int qrow = wave * 32 + col;
  const int64_t bh = item / num_tiles;
  const int tile_i = item - static_cast<int>(bh) * num_tiles;
  const int64_t head_elems = static_cast<int64_t>(num_tiles) * T * D;
  const uint16_t* kh = k + bh * head_elems;
  const uint16_t* vh = v + bh * head_elems;
  const int64_t row_g = (bh * num_tiles + tile_i) * T + qrow;  // this lane's query row
  // lists and lengths count tiles of T << sub_shift rows (see the forward)
  const int nt_list = num_tiles >> sub_shift;
  const int tile_l = tile_i >> sub_shift;
  const int64_t item_l = bh * nt_list + tile_l;
  const int vq = clampi(vbs[tile_l] - T * (tile_i & ((1 << sub_shift) - 1)), 0, T);
  const int count = max_sel > 0 ? clampi(q2k_num[item_l], 0, max_sel) : 0;
  const int32_t* list = q2k_idx + item_l * max_sel;

  bf16x8_t qop[C::kKSteps], dop[C::kKSteps];
#pragma unroll
  for (int kk = 0; kk < C::kKSteps; ++kk) {
    qop[kk] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(q + row_g * D + 16 * kk + 8 * half));
    dop[kk] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(dout + row_g * D + 16 * kk + 8 * half));
  }
  const float lse2 = lse[row_g] * kLog2e;
  const float dlt = delta[row_g];

  f32x16_t acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[db][r] = 0.0f;
  bool any_keys = false;
  const DmaLane<T, D, false> dl(wave, lane);
  const f32x16_t zero16 = {};

  for (int base = 0; base < count; base += C::kThreads) {
    int total;
    if constexpr (kPairs)
      total = compact_steps<T, C::kWaves>(list, base, count, vbs, nt_list, st, srt, wave_scratch, tid, wave,
                                          lane, sub_shift);
    else
      total = compact_list<T, C::kWaves, 2>(list, base, count, vbs, nt_list, st, wave_scratch, tid, wave, lane,
                                            sub_shift);
    if (total > 0) any_keys = true;
    // K and V are copied in 64-key halves, each as soon as its LDS half is
    // free: the next tile's half h once every wave is done with this tile's
    // half h, so that each half lands while the other half is computed.
    // Every copy issues all its instructions (padding rows cost no memory
    // traffic), which keeps the vmcnt waits exact.
    constexpr int NH = T / 64;                // 64-key halves
    constexpr int kHP = C::kDmaPerTile / NH;  // copy instructions per half and tensor
    // Step n = (j, vk): one tile (j >= 0), or a pair (j <= -2, the rest of the
    // step in st[2n + 1]) whose second tile's rows follow the first's; a
    // pair's copy may issue one instruction more per tensor (the block holding
    // the boundary row, split by lane), which only makes later waits for
    // earlier copies wait longer.
    auto copy_half = [&](auto hc, int n, int j, int vk) {
      constexpr int h = decltype(hc)::value;
      if (!kPairs || j >= 0) {
        dma_tile_part<T, D, h * kHP, (h + 1) * kHP>(kh + static_cast<int64_t>(j) * T * D, ks, wave, dl, vk);
        dma_tile_part<T, D, h * kHP, (h + 1) * kHP>(vh + static_cast<int64_t>(j) * T * D, vs, wave, dl, vk);
      } else {
        const int2 bv = st[2 * n + 1];
        const int jb = __builtin_amdgcn_readfirstlane(bv.x), va = __builtin_amdgcn_readfirstlane(bv.y);
        dma_pair<T, D, false, false, h * kHP, (h + 1) * kHP>(kh, -2 - j, va, jb, vk - va, ks, wave, lane, dl);
        dma_pair<T, D, false, false, h * kHP, (h + 1) * kHP>(vh, -2 - j, va, jb, vk - va, vs, wave, lane, dl);
      }
    };
    // Q, dO and the row statistics must be in registers before the first copy:
    // the copies are invisible to the compiler's wait-count bookkeeping, and a
    // drain here, on every path into the tile loop, keeps it from placing
    // waits for those loads inside the loop, where they would also wait for
    // the copies in flight.
    wait_vmcnt<0>();
    for (int t = 0; t < total; ++t) {
      const int2 e = st[2 * t];
      const int j = __builtin_amdgcn_readfirstlane(e.x);
      const int vk = __builtin_amdgcn_readfirstlane(e.y);
      int j2 = -1, vk2 = 0;
      if (t + 1 < total) {
        const int2 e2 = st[2 * (t + 1)];
        j2 = __builtin_amdgcn_readfirstlane(e2.x);
        vk2 = __builtin_amdgcn_readfirstlane(e2.y);
      }
      if (t == 0) static_for<NH>([&](auto hc) { copy_half(hc, 0, j, vk); });
      static_for<NH>([&](auto hc) {  // 64 keys: key blocks 2*hh, 2*hh + 1
        constexpr int hh = decltype(hc)::value;
        // half hh of this tile has landed; issued after it: its later halves
        // and, from hh = 2 on, the next tile's halves 0 .. hh - 2
        wait_vmcnt<2 * kHP * (NH - 1 - hh + (hh > 1 ? hh - 1 : 0))>();
        if (vk < T) {
          zero_padding_part<T, D, hh * kHP, (hh + 1) * kHP>(ks, vk, wave, lane);
          zero_padding_part<T, D, hh * kHP, (hh + 1) * kHP>(vs, vk, wave, lane);
        }
        lds_barrier();  // half hh visible; every wave is done with half hh - 1
        if constexpr (hh > 0)
          if (j2 != -1) copy_half(std::integral_constant<int, hh - 1>{}, t + 1, j2, vk2);
        if (wave * 32 < vq) {  // a wave whose rows are all padding computes nothing
        // Raised issue priority for the S/dP products: two workgroups share each
        // SIMD, and the wave in this phase winning issue pushes the pair towards
        // anti-phase, one wave's exponentials and dQ products under the other's
        // S/dP products.
        __builtin_amdgcn_s_setprio(1);
        f32x16_t s[2], dp[2];
#pragma unroll
        for (int kk = 0; kk < C::kKSteps; ++kk)
#pragma unroll
          for (int b2 = 0; b2 < 2; ++b2) {
            s[b2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                read_rows<D>(ks, 32 * (2 * hh + b2), kk, col, half), qop[kk], kk ? s[b2] : zero16, 0, 0, 0);
            dp[b2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                read_rows<D>(vs, 32 * (2 * hh + b2), kk, col, half), dop[kk], kk ? dp[b2] : zero16, 0, 0, 0);
          }
        __builtin_amdgcn_s_setprio(0);
        // P^T = exp2(S^T c - lse2) with keys at or past vk masked; dS^T = P^T (dP^T - D).
        // A masked logit is selected to -inf, so its p is exp2(-inf) = 0 (a row whose
        // lse is -inf or NaN is NaN through its valid keys in any case, or is padding),
        // and its dS is 0 * (0 - D) (V padding rows are zero in LDS): a zero, of
        // either sign, which leaves every dQ sum as the plain formula has it.
#pragma unroll
        for (int b2 = 0; b2 < 2; ++b2) {
          const int kb = 2 * hh + b2;
          if (32 * kb + 32 > vk) {  // only the blocks that reach vk take the mask (uniform)
            const int t0 = vk - 32 * kb - 4 * half;
#pragma unroll
            for (int r = 0; r < 16; ++r)
              if (8 * (r >> 2) + (r & 3) >= t0) s[b2][r] = -INFINITY;
          }
        }
#pragma unroll
        for (int b2 = 0; b2 < 2; ++b2)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[b2][r], c, -lse2));
            s[b2][r] = p * (dp[b2][r] - dlt);
          }
        // dQ^T += K^T dS^T over the four 16-key chunks of this half
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) {
          const bf16x8_t dsk = pack8(s[cc >> 1], 8 * (cc & 1));
#pragma unroll
          for (int db = 0; db < NDB; ++db)
            acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                read_rows_t<D>(ks, 4 * hh + cc, db, lane), dsk, acc[db], 0, 0, 0);
        }
        }
      });
      lds_barrier();  // every wave is done with the last half
      if (j2 != -1) copy_half(std::integral_constant<int, NH - 1>{}, t + 1, j2, vk2);
    }
  }
  wait_vmcnt<0>();
  const bool zero_row = !any_keys || qrow >= vq;
  store_t<D>(dq + row_g * D, acc, scale, zero_row, half);
}

// ---- dK, dV -------------------------------------------------------------------------------
// Issue schedule of the dK/dV products of one query tile.  Step qb*(NA+NB) + k
// is step k of 32-query block qb: S/dP steps (k < NA), then dV/dK steps, the
// first NB/2 on the block's first 16-query chunk.  A block's softmax runs in
// four groups of four queries; P and dS of its first chunk are packed after
// group 1, those of the second after group 3.  S/dP and the packed P/dS
// live in kSets register sets, block qb in set qb % kSets.
//   st[p]: the p-th step issued;
//   sm[p]: softmax groups run after step p: 16 * block + mask of groups, or -1.
// Two sets (one wave per SIMD at D = 128, registers to spare): block 0's S/dP
// steps, then block 1's with block 0's groups among them; then period b runs
// block b's dV/dK steps alternating with block b+2's S/dP steps, with block
// b+1's groups among them.  Nothing a period's softmax touches is touched by
// that period's products, so the exponentials run beside the matrix products.
// One set (two waves per SIMD at D = 64, where a second set would spill): a
// block's groups 0 and 1 after its last S/dP step, groups 2 and 3 after its
// first two dV/dK steps; the next block's S/dP steps then go between its
// remaining dV/dK steps, two of which come last, beside the next block's
// first groups.
template <int NQB, int NA, int NB, int kSets>
struct DkvPipe {
  static constexpr int NS = NA + NB, N = NQB * NS;
  int st[N];
  int sm[N];
  constexpr DkvPipe() : st{}, sm{} {
    for (int i = 0; i < N; ++i) sm[i] = -1;
    int p = 0;
    auto put = [&](int at, int b, int g) {
      sm[at] = (sm[at] < 0 ? 16 * b : sm[at]) | (1 << g);
    };
    if (kSets == 2) {
      // the four groups of block b spread over the `count` steps from `first`
      // (after steps 1, 5, 9, 13 of 16; 1, 3, 5, 7 of 8; 0, 1, 2, 3 of 4)
      auto groups = [&](int first, int count, int b) {
        for (int g = 0; g < 4; ++g) {
          const int x = count - 4 + g, y = 1 + g * count / 4;
          put(first + (x < y ? x : y), b, g);
        }
      };
      for (int a = 0; a < NA; ++a) st[p++] = a;
      {
        const int first = p;
        for (int a = 0; a < NA; ++a) st[p++] = NS + a;
        groups(first, NA, 0);
      }
      for (int b = 0; b < NQB; ++b) {
        const int first = p;
        const bool sdp = b + 2 < NQB;
        int x = 0, y = 0;
        while (x < NB || (sdp && y < NA)) {
          if (x < NB && (!sdp || y >= NA || x * NA <= y * NB)) st[p++] = b * NS + NA + x++;
          else st[p++] = (b + 2) * NS + y++;
        }
        if (b + 1 < NQB) groups(first, p - first, b + 1);
      }
    } else {
      const int tail = NB - 2 < 2 ? NB - 2 : 2;  // dV/dK steps after the next block's S/dP
      const int mid = NB - 2 - tail;             // dV/dK steps spread among them
      for (int a = 0; a < NA; ++a) st[p++] = a;
      put(p - 1, 0, 0);
      put(p - 1, 0, 1);
      for (int qb = 0; qb < NQB; ++qb) {
        const int base = qb * NS, next = base + NS;
        st[p++] = base + NA;
        put(p - 1, qb, 2);
        st[p++] = base + NA + 1;
        put(p - 1, qb, 3);
        int b = 2;
        if (qb + 1 < NQB) {
          int a = 0;
          for (int m = 0; m < mid; ++m) {
            st[p++] = base + NA + b++;
            for (int x = mid ? (m + 1) * NA / mid - m * NA / mid : 0; x > 0; --x) st[p++] = next + a++;
          }
          while (a < NA) st[p++] = next + a++;
        }
        while (b < NB) st[p++] = base + NA + b++;
        if (qb + 1 < NQB) {
          put(p - 1, qb + 1, 0);
          put(p - 1, qb + 1, 1);
        }
      }
    }
  }
};
template <int NQB, int NA, int NB, int kSets>
inline constexpr DkvPipe<NQB, NA, NB, kSets> kDkvPipe{};
// The data flow a schedule must respect (positions in issue order; a group at
// position q runs after step q): every step once, each block's steps in
// order; a block's groups in order, after its last S/dP step and before the
// S/dP step that reuses its register set (block + kSets); its dV/dK steps on
// chunk c after its packing group 2c + 1; the packing groups of block
// b + kSets after block b's last dV/dK step on that chunk.
template <int NQB, int NA, int NB, int kSets>
constexpr bool dkv_pipe_valid() {
  constexpr auto& s = kDkvPipe<NQB, NA, NB, kSets>;
  constexpr int NS = NA + NB, N = NQB * NS, C2 = NB / 2;
  int pos[N] = {}, gpos[NQB][4] = {};
  bool seen[N] = {}, gseen[NQB][4] = {};
  for (int p = 0; p < N; ++p) {
    const int st = s.st[p];
    if (st < 0 || st >= N || seen[st]) return false;
    seen[st] = true;
    pos[st] = p;
    if (s.sm[p] >= 0) {
      const int b = s.sm[p] / 16;
      if (b >= NQB) return false;
      for (int g = 0; g < 4; ++g)
        if (s.sm[p] >> g & 1) {
          if (gseen[b][g]) return false;
          gseen[b][g] = true;
          gpos[b][g] = p;
        }
    }
  }
  for (int b = 0; b < NQB; ++b) {
    const int base = b * NS;
    for (int g = 0; g < 4; ++g) {
      if (!gseen[b][g]) return false;
      if (g && gpos[b][g] < gpos[b][g - 1]) return false;
    }
    for (int k = 1; k < NS; ++k)
      if (pos[base + k] < pos[base + k - 1]) return false;
    if (gpos[b][0] < pos[base + NA - 1]) return false;
    for (int k = 0; k < NB; ++k)
      if (pos[base + NA + k] <= gpos[b][k < C2 ? 1 : 3]) return false;
    if (b + kSets < NQB) {
      if (pos[base + kSets * NS] <= gpos[b][3]) return false;
      if (gpos[b + kSets][1] < pos[base + NA + C2 - 1] ||
          gpos[b + kSets][3] < pos[base + NA + NB - 1])
        return false;
    }
  }
  return true;
}
static_assert(dkv_pipe_valid<4, 8, 8, 2>() && dkv_pipe_valid<2, 8, 8, 2>() &&
                  dkv_pipe_valid<4, 4, 4, 1>() && dkv_pipe_valid<2, 4, 4, 1>() &&
                  dkv_pipe_valid<4, 8, 8, 1>() && dkv_pipe_valid<4, 4, 4, 2>(),
              "dK/dV step schedule");

// At D = 128 a wave holds its K and V operands (64 registers) and two fp32
// accumulators (128) across the whole list: one wave per SIMD, up to 512
// registers, instead of spilling at two.
template <int T, int D>
__global__ __launch_bounds__(2 * T)
__attribute__((amdgpu_waves_per_eu(D == 128 ? 1 : 2, D == 128 ? 1 : (T == 128 ? 2 : 4))))
void dkv_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                const uint16_t* __restrict__ v, const uint16_t* __restrict__ dout,
                const float* __restrict__ lse, const float* __restrict__ delta,
                const int32_t* __restrict__ k2q_idx, const int32_t* __restrict__ k2q_num,
                const int32_t* __restrict__ vbs, uint16_t* __restrict__ dk, uint16_t* __restrict__ dv,
                int num_tiles, int max_k, int n_items, int n_padded, float c, float scale,
                int sub_shift) {
  using C = Cfg<T, D>;
  constexpr int NDB = C::kDBlocks;
  // Q and dO tiles and their row statistics, double-buffered: the copies of
  // the next query tile land while the current one is computed.
  __shared__ __attribute__((aligned(1024))) uint16_t qs_all[2][T * D];
  __shared__ __attribute__((aligned(1024))) uint16_t ds_all[2][T * D];  // dO tiles
  __shared__ __attribute__((aligned(16))) float lse_all[2][T];
  __shared__ __attribute__((aligned(16))) float dlt_all[2][T];
  // the steps of the current list chunk (compact_steps, as in the forward):
  // a query tile, or two that fit in T rows together
  __shared__ int2 st[2 * (T == 128 ? 2 : 1) * C::kThreads];
  __shared__ int2 srt[(T == 128 ? 2 : 1) * C::kThreads];
  __shared__ int wave_scratch[5 * C::kWaves];

  const int item = item_of(blockIdx.x, n_padded);  // (b*H + h) * NT + key tile j
  if (item >= n_items) return;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31;
  const int half = lane >> 5;
  const int krow = wave * 32 + col;
  const int64_t bh = item / num_tiles;
  const int tile_j = item - static_cast<int>(bh) * num_tiles;
  const int64_t head_elems = static_cast<int64_t>(num_tiles) * T * D;
  const uint16_t* qh = q + bh * head_elems;
  const uint16_t* oh = dout + bh * head_elems;
  const int64_t row_g = (bh * num_tiles + tile_j) * T + krow;  // this lane's key row
  const int nt_list = num_tiles >> sub_shift;
  const int tile_l = tile_j >> sub_shift;
  const int64_t item_l = bh * nt_list + tile_l;
  const int vk = clampi(vbs[tile_l] - T * (tile_j & ((1 << sub_shift) - 1)), 0, T);
  const int count = max_k > 0 ? clampi(k2q_num[item_l], 0, max_k) : 0;
  const int32_t* list = k2q_idx + item_l * max_k;

  bf16x8_t kop[C::kKSteps], vop[C::kKSteps];
#pragma unroll
  for (int kk = 0; kk < C::kKSteps; ++kk) {
    kop[kk] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(k + row_g * D + 16 * kk + 8 * half));
    vop[kk] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(v + row_g * D + 16 * kk + 8 * half));
  }
  f32x16_t acck[NDB], accv[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      acck[db][r] = 0.0f;
      accv[db][r] = 0.0f;
    }
  const DmaLane<T, D, false> dl(wave, lane);
  const f32x16_t zero16 = {};

  // Copies of step t of the chunk into buffer `buf`; its statistics go to
  // registers (threads below T), written to LDS once they have landed.  A step
  // is a query tile i with vq valid rows, or a pair (i = -2 - ia): rows
  // [0, va) of tile ia and, after them, the first vq - va rows of tile ib.
  float l_next = 0.0f, d_next = 0.0f;
  TileCopy<T, D, false> copy_q, copy_o;
  // Copy instruction n of a staged single tile: Q's for even n, dO's for odd n.
  // With kSkip, blocks wholly past the valid rows are not copied; without,
  // their lanes fail the range check (no memory traffic), and what they
  // leave in LDS is zeroed with the other padding rows once the copy lands.
  auto copy_one = [&](auto nc, auto skip) {
    constexpr int n = decltype(nc)::value;
    constexpr bool kSkip = decltype(skip)::value;
    if constexpr (n % 2 == 0) copy_q.template one<n / 2, kSkip>(dl, wave);
    else copy_o.template one<n / 2, kSkip>(dl, wave);
  };
  constexpr int kCopies = 2 * C::kDmaPerTile;
  // Stages step t: a single tile's copies are issued now, or, with `spread`,
  // left to copy_one (returns true); a pair's are always issued now.
  auto issue = [&](int t, int buf, bool spread) {
    const int2 e = st[2 * t];
    const int i = __builtin_amdgcn_readfirstlane(e.x);
    const int vq = __builtin_amdgcn_readfirstlane(e.y);
    int ia = i, va = vq, ib = 0;
    if (i >= 0) {
      const int64_t qtile = static_cast<int64_t>(i) * T;
      copy_q.set(qh + qtile * D, qs_all[buf], wave, vq);
      copy_o.set(oh + qtile * D, ds_all[buf], wave, vq);
      if (!spread) static_for<kCopies>([&](auto nc) { copy_one(nc, std::true_type{}); });
    } else {
      const int2 bv = st[2 * t + 1];
      ia = -2 - i;
      ib = __builtin_amdgcn_readfirstlane(bv.x);
      va = __builtin_amdgcn_readfirstlane(bv.y);
      dma_pair<T, D, false, true>(qh, ia, va, ib, vq - va, qs_all[buf], wave, lane, dl);
      dma_pair<T, D, false, true>(oh, ia, va, ib, vq - va, ds_all[buf], wave, lane, dl);
      spread = false;
    }
    if (tid < vq) {
      const int64_t r = (bh * num_tiles + (tid < va ? ia : ib)) * T + (tid < va ? tid : tid - va);
      l_next = lse[r];
      d_next = delta[r];
    }
    return spread;
  };

  for (int base = 0; base < count; base += C::kThreads) {
    const int total = compact_steps<T, C::kWaves>(list, base, count, vbs, nt_list, st, srt, wave_scratch,
                                                  tid, wave, lane, sub_shift);
    if (total == 0) continue;
    wait_vmcnt<0>();  // the register operands loaded above
    issue(0, 0, false);
    for (int t = 0; t < total; ++t) {
      const int buf = t & 1;
      const int vq = __builtin_amdgcn_readfirstlane(st[2 * t].y);
      uint16_t* qs = qs_all[buf];
      uint16_t* ds_ = ds_all[buf];
      float* lse_s = lse_all[buf];
      float* dlt_s = dlt_all[buf];
      wait_vmcnt<0>();  // tile t's copies and statistics have landed
      // padding query rows get lse = +inf, so P = 0 there
      if (tid < T) {
        lse_s[tid] = tid < vq ? l_next * kLog2e : INFINITY;
        dlt_s[tid] = tid < vq ? d_next : 0.0f;
      }
      if (vq < T) {
        zero_padding_rows<T, D>(qs, vq, wave, lane);
        zero_padding_rows<T, D>(ds_, vq, wave, lane);
      }
      lds_barrier();  // tile t visible; every wave is done with tile t - 1's buffer
      // Tile t + 1's copies.  At D = 128 the one wave per SIMD spreads them
      // over tile t's products: issued as one burst they would hold it for
      // as long as the L2 -> LDS path takes to accept them.  A wave without
      // products to hide them under issues them at once.
      constexpr bool kSpread = D == 128;
      bool spread_next = false;  // tile t + 1's copies are left to the steps below
      if (t + 1 < total) spread_next = issue(t + 1, buf ^ 1, kSpread && wave * 32 < vk);
    // Per 32-query block: S = Q K^T and dP = dO V^T (steps k < NA), P and dS,
    // then dV^T += dO^T P and dK^T += Q^T dS over its two 16-query chunks
    // (steps k >= NA), in the pipelined order kDkvPipe gives.  With one wave
    // per SIMD nothing hides LDS latency but the wave's own MFMAs, so the two
    // LDS operands of every step are read kAhead steps early, through a ring
    // of registers, across blocks and phases.  A wave whose key rows are all
    // padding skips the compute.
    if (wave * 32 < vk) {
      constexpr int NQB = T / 32, NA = C::kKSteps, NB = 2 * NDB, NS = NA + NB, kSteps = NQB * NS;
      constexpr int kSets = D == 128 ? 2 : 1;
      constexpr int kAhead = 3, kRing = kAhead + 1;
      bf16x8_t ra[kRing], rb[kRing];
      auto load = [&](int st, int sl) {
        const int qb = st / NS, k = st % NS;
        if (k < NA) {
          ra[sl] = read_rows<D>(qs, 32 * qb, k, col, half);
          rb[sl] = read_rows<D>(ds_, 32 * qb, k, col, half);
        } else {
          const int cc = (k - NA) / NDB, db = (k - NA) % NDB;
          ra[sl] = read_rows_t<D>(ds_, 2 * qb + cc, db, lane);
          rb[sl] = read_rows_t<D>(qs, 2 * qb + cc, db, lane);
        }
      };
      static_for<kAhead>([&](auto pc) {
        constexpr int p = decltype(pc)::value;
        load(kDkvPipe<NQB, NA, NB, kSets>.st[p], p % kRing);
      });
      f32x16_t s[kSets], dp[kSets];
      bf16x8_t pb[kSets][2], sb[kSets][2];
      // P and dS of block qb, four queries (one register group) at a time:
      // register r holds query 32*qb + 8*(r/4) + 4*half + r%4
      auto softmax_group = [&](int qb, int g, f32x16_t& sx, f32x16_t& dx) {
        const float4 l4 = *reinterpret_cast<const float4*>(lse_s + 32 * qb + 8 * g + 4 * half);
        const float4 d4 = *reinterpret_cast<const float4*>(dlt_s + 32 * qb + 8 * g + 4 * half);
        const float lv[4] = {l4.x, l4.y, l4.z, l4.w}, dv4[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * g + e;
          const float pr = __builtin_amdgcn_exp2f(__builtin_fmaf(sx[r], c, -lv[e]));
          sx[r] = pr;                     // P
          dx[r] = pr * (dx[r] - dv4[e]);  // dS
        }
      };
      static_for<kSteps>([&](auto pc) {
        constexpr int p = decltype(pc)::value;
        if constexpr (p + kAhead < kSteps)
          load(kDkvPipe<NQB, NA, NB, kSets>.st[p + kAhead], (p + kAhead) % kRing);
        constexpr int st = kDkvPipe<NQB, NA, NB, kSets>.st[p];
        constexpr int qb = st / NS, k = st % NS, sl = p % kRing, x = qb % kSets;
        if constexpr (k < NA) {
          s[x] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ra[sl], kop[k], k ? s[x] : zero16, 0, 0, 0);
          dp[x] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(rb[sl], vop[k], k ? dp[x] : zero16, 0, 0, 0);
        } else {
          constexpr int cc = (k - NA) / NDB, db = (k - NA) % NDB;
          accv[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ra[sl], pb[x][cc], accv[db], 0, 0, 0);
          acck[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(rb[sl], sb[x][cc], acck[db], 0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
        // copy n of tile t + 1 after step 2 + n * kCopyEvery: spread evenly
        // over the tile, every fourth step at most
        constexpr int kSpan = (kSteps - 3) / (kCopies - 1);
        constexpr int kCopyEvery = kSpan < 4 ? (kSpan > 0 ? kSpan : 1) : 4;
        static_assert(!kSpread || 2 + (kCopies - 1) * kCopyEvery < kSteps, "every copy is issued");
        if constexpr (kSpread && p >= 2 && (p - 2) % kCopyEvery == 0 && (p - 2) / kCopyEvery < kCopies) {
          if (spread_next) copy_one(std::integral_constant<int, (p - 2) / kCopyEvery>{}, std::false_type{});
        }
        constexpr int smg = kDkvPipe<NQB, NA, NB, kSets>.sm[p];
        if constexpr (smg >= 0) {
          constexpr int b = smg / 16, y = b % kSets;
          static_for<4>([&](auto gc) {
            constexpr int g = decltype(gc)::value;
            if constexpr ((smg >> g) & 1) {
              softmax_group(b, g, s[y], dp[y]);
              if constexpr (g == 1) {
                pb[y][0] = pack8(s[y], 0);
                sb[y][0] = pack8(dp[y], 0);
              } else if constexpr (g == 3) {
                pb[y][1] = pack8(s[y], 8);
                sb[y][1] = pack8(dp[y], 8);
              }
            }
          });
          __builtin_amdgcn_sched_barrier(0);
        }
      });
    }
  }
  }
  wait_vmcnt<0>();
  const bool zero_row = krow >= vk;
  store_t<D>(dk + row_g * D, acck, scale, zero_row, half);
  store_t<D>(dv + row_g * D, accv, 1.0f, zero_row, half);
}

template <int T, int D>
hipError_t launch_grads(const bsa::BwdProblem& p, hipStream_t stream) {
  const int64_t items = p.batch_heads * p.num_tiles;
  const int n_items = static_cast<int>(items);
  const int n_padded = (n_items + 7) / 8 * 8;
  const float scale = static_cast<float>(1.0 / __builtin_sqrt(static_cast<double>(D)));
  const float c = scale * kLog2e;
  dim3 block(Cfg<T, D>::kThreads);
  hipLaunchKernelGGL((dq_kernel<T, D>), dim3(n_padded), block, 0, stream, p.q, p.k, p.v, p.dout,
                     p.lse, p.delta, p.q2k_idx, p.q2k_num, p.block_sizes, p.dq, p.num_tiles,
                     p.max_sel, n_items, n_padded, c, scale, p.sub_shift);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL((dkv_kernel<T, D>), dim3(n_padded), block, 0, stream, p.q, p.k, p.v, p.dout,
                     p.lse, p.delta, p.k2q_idx, p.k2q_num, p.block_sizes, p.dk, p.dv, p.num_tiles,
                     p.max_k, n_items, n_padded, c, scale, p.sub_shift);
  return hipGetLastError();
}

}  // namespace

namespace bsa {

hipError_t launch_k2q(const K2qProblem& p, hipStream_t stream) {
  // Counting in LDS when the head's lengths fit and every workgroup's pass over the
  // head's lists stays short; the scan otherwise.
  if (p.num_tiles <= kCountMaxTiles && p.max_sel <= 65535) {
    int span = 2 * (kCountWords / p.num_tiles);
    if (span > kCountThreads) span = kCountThreads;
    if (span > p.num_tiles + (p.num_tiles & 1)) span = p.num_tiles + (p.num_tiles & 1);
    const int64_t groups = (p.num_tiles + span - 1) / span;
    if (groups * p.num_tiles * static_cast<int64_t>(p.max_sel) <= (int64_t{1} << 22)) {
      hipLaunchKernelGGL(k2q_count_kernel, dim3(static_cast<unsigned>(p.batch_heads * groups)),
                         dim3(kCountThreads), 0, stream, p.q2k_idx, p.q2k_num, p.num_tiles, p.max_sel, span,
                         static_cast<int>(groups), p.k2q_idx, p.k2q_num, p.max_k);
      return hipGetLastError();
    }
  }
  const int64_t lists = p.batch_heads * p.num_tiles;
  const int64_t blocks = (lists + 3) / 4;
  hipLaunchKernelGGL(k2q_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream,
                     p.q2k_idx, p.q2k_num, p.num_tiles, p.max_sel, lists, p.k2q_idx, p.k2q_num,
                     p.max_k);
  return hipGetLastError();
}

hipError_t launch_bwd(const BwdProblem& p, hipStream_t stream) {
  const int64_t rows = p.batch_heads * p.num_tiles * p.tile;
  const int lanes = p.head_dim / 8;
  const int64_t blocks = (rows * lanes + 255) / 256;
  if (p.head_dim == 128)
    hipLaunchKernelGGL(delta_kernel<128>, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream,
                       p.out, p.out_lo, p.dout, p.block_sizes, p.num_tiles, p.tile, rows, p.delta,
                       p.sub_shift);
  else
    hipLaunchKernelGGL(delta_kernel<64>, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream,
                       p.out, p.out_lo, p.dout, p.block_sizes, p.num_tiles, p.tile, rows, p.delta,
                       p.sub_shift);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (p.tile == 128) return p.head_dim == 128 ? launch_grads<128, 128>(p, stream)
                                               : launch_grads<128, 64>(p, stream);
  return p.head_dim == 128 ? launch_grads<64, 128>(p, stream) : launch_grads<64, 64>(p, stream);
}

}  // namespace bsa
