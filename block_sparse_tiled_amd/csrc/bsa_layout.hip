// Fused token-to-tile layout: token-major [B, S_tok, H, D] tensors (Q, K, V
// and the gate) gathered into the tile buffer [B, H, NT*T, D] in one pass.
//
// FastVideo fastvideo-kernel commit list, page 3, fused-layout commit: one
// kernel replaces the scatter into the tile buffer and the four transposed
// copies that followed it.  Here the map is given in gather form (the source
// token of every tile row, -1 for padding), which describes the same
// permutation and lets every output byte be written exactly once, so padding
// rows need no separate clearing pass.
//
// The inverse gather (tile buffer -> token-major, for the attention output)
// uses the token -> tile-row map and is written the same way.
//
// Pure HBM streaming: each thread moves one 16-byte chunk of a row for every
// tensor, reading the map entry once.  A workgroup covers whole rows, so the
// reads of one source row (D*2 contiguous bytes) and the writes of one tile
// row are each coalesced.
#include <hip/hip_runtime.h>

#include "bsa_launch.h"

namespace {

__device__ __forceinline__ int clampi_layout(int x, int lo, int hi) {
  return x < lo ? lo : (x > hi ? hi : x);
}

struct Ptrs {
  const uint4* src[4];
  uint4* dst[4];
};

// D8 = 16-byte chunks per row (8 for D = 64, 16 for D = 128).  Each thread
// moves one chunk per step, or, for small launches (U = 4), four chunks 256
// apart with all loads before the stores: fewer, fuller workgroups finish
// sooner there (measured: the 12-head, 8192-row ragged shape 33.4 -> 31.1
// us), while the larger shapes ran 1-2 % slower that way.
template <int D8, int U>
__global__ __launch_bounds__(256) void tile_layout_kernel(Ptrs p, int n_tensors,
                                                          const int32_t* __restrict__ map,
                                                          int64_t tokens, int64_t heads,
                                                          int64_t rows_per_head) {
  const int64_t bh = blockIdx.y;
  const int64_t b = bh / heads;
  const int64_t h = bh - b * heads;
  const int64_t chunks = rows_per_head * D8;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x * U;
  if constexpr (U == 1) {
    for (int64_t c = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; c < chunks;
         c += stride) {
      const int32_t s = map[c / D8];
      const int64_t out_off = bh * chunks + c;
      if (s >= 0 && s < tokens) {
        const int64_t in_off = ((b * tokens + s) * heads + h) * D8 + c % D8;
#pragma unroll
        for (int x = 0; x < 4; ++x)
          if (x < n_tensors) p.dst[x][out_off] = p.src[x][in_off];
      } else {
#pragma unroll
        for (int x = 0; x < 4; ++x)
          if (x < n_tensors) p.dst[x][out_off] = make_uint4(0u, 0u, 0u, 0u);
      }
    }
    return;
  }
  for (int64_t c0 = static_cast<int64_t>(blockIdx.x) * blockDim.x * U + threadIdx.x; c0 < chunks;
       c0 += stride) {
    uint4 val[U][4];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t c = c0 + u * 256;
      const int32_t s = c < chunks ? map[c / D8] : -1;
      const bool ok = s >= 0 && s < tokens;
      const int64_t in_off = ((b * tokens + (ok ? s : 0)) * heads + h) * D8 + c % D8;
#pragma unroll
      for (int x = 0; x < 4; ++x)
        val[u][x] = x < n_tensors && ok ? p.src[x][in_off] : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t c = c0 + u * 256;
      if (c >= chunks) break;
      const int64_t out_off = bh * chunks + c;
#pragma unroll
      for (int x = 0; x < 4; ++x)
        if (x < n_tensors) p.dst[x][out_off] = val[u][x];
    }
  }
}

// The layout with the coarse stage's pooling: one workgroup per (head, tile).
// For each tensor, the whole workgroup moves the tile's rows (every load
// issued before any store) and, for the first three (Q, K, V), keeps them in
// LDS; then thread d sums column d over the rows below block_sizes[t] in
// binary32, in row order, and divides by the count: the sums and quotients the
// coarse stage forms from the tile buffer, so the pooled rows are the same
// bits.  The tile's map entries are staged in LDS first.
constexpr int kPoolMaxTile = 256;
template <int D8>
__global__ __launch_bounds__(256) void tile_layout_pool_kernel(
    Ptrs p, int n_tensors, const int32_t* __restrict__ map, const int32_t* __restrict__ vbs,
    int64_t tokens, int64_t heads, int num_tiles, int tile, int64_t tiles_all,
    float* __restrict__ pooled) {
  constexpr int D = 8 * D8;
  __shared__ uint4 rows_s[kPoolMaxTile * D8];
  __shared__ int32_t smap[kPoolMaxTile];
  const int64_t bht = blockIdx.x;  // bh * num_tiles + t
  const int64_t bh = bht / num_tiles;
  const int t = static_cast<int>(bht - bh * num_tiles);
  const int64_t b = bh / heads, h = bh - b * heads;
  const int tid = threadIdx.x;
  for (int s = tid; s < tile; s += 256) smap[s] = map[static_cast<int64_t>(t) * tile + s];
  const int n = clampi_layout(vbs[t], 0, tile);
  __syncthreads();
  const int chunks = tile * D8;  // at most kPoolMaxTile * D8 = 16 per thread
  const int64_t out0 = bht * chunks;
  for (int x = 0; x < n_tensors; ++x) {
    constexpr int kMax = kPoolMaxTile * D8 / 256;
    uint4 val[kMax];
#pragma unroll
    for (int u = 0; u < kMax; ++u) {
      const int e = tid + 256 * u;
      val[u] = make_uint4(0u, 0u, 0u, 0u);
      if (e < chunks) {
        const int32_t tok = smap[e / D8];
        if (tok >= 0 && tok < tokens) val[u] = p.src[x][((b * tokens + tok) * heads + h) * D8 + e % D8];
      }
    }
#pragma unroll
    for (int u = 0; u < kMax; ++u) {
      const int e = tid + 256 * u;
      if (e < chunks) {
        p.dst[x][out0 + e] = val[u];
        if (x < 3) rows_s[e] = val[u];
      }
    }
    if (x < 3) {
      __syncthreads();
      if (tid < D) {
        const uint16_t* col = reinterpret_cast<const uint16_t*>(rows_s) + tid;
        float acc = 0.0f;
#pragma unroll 8
        for (int s = 0; s < n; ++s)
          acc = __fadd_rn(acc, __uint_as_float(static_cast<uint32_t>(col[s * D]) << 16));
        pooled[(x * tiles_all + bht) * D + tid] = n > 0 ? __fdiv_rn(acc, static_cast<float>(n)) : 0.0f;
      }
      __syncthreads();  // every column is summed before the next tensor's rows land
    }
  }
}

// The inverse: token-major rows gathered from the tile buffer through the
// token -> tile-row map.  One 16-byte chunk per thread, chunk index fastest,
// then head, then token, so the writes of consecutive threads are contiguous
// and each thread group of D8 threads reads one whole tile row.
template <int D8>
__global__ __launch_bounds__(256) void tile_unlayout_kernel(Ptrs p, int n_tensors,
                                                            const int32_t* __restrict__ token_row,
                                                            int64_t tokens, int64_t heads,
                                                            int64_t rows_per_head) {
  const int64_t b = blockIdx.y;
  const int64_t chunks = tokens * heads * D8;  // per batch
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t c = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; c < chunks;
       c += stride) {
    const int ch = static_cast<int>(c % D8);
    const int64_t th = c / D8;  // token * heads + head
    const int64_t n = th / heads;
    const int64_t h = th - n * heads;
    const int32_t r = token_row[n];
    const int64_t out_off = b * chunks + c;
    if (r >= 0 && r < rows_per_head) {
      const int64_t in_off = ((b * heads + h) * rows_per_head + r) * D8 + ch;
#pragma unroll
      for (int x = 0; x < 4; ++x)
        if (x < n_tensors) p.dst[x][out_off] = p.src[x][in_off];
    } else {
      const uint4 zero = make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
      for (int x = 0; x < 4; ++x)
        if (x < n_tensors) p.dst[x][out_off] = zero;
    }
  }
}

}  // namespace

namespace bsa {

hipError_t launch_tile_layout(const LayoutProblem& lp, hipStream_t stream) {
  Ptrs p;
  for (int x = 0; x < 4; ++x) {
    p.src[x] = static_cast<const uint4*>(lp.src[x]);
    p.dst[x] = static_cast<uint4*>(lp.dst[x]);
  }
  const int d8 = lp.head_dim / 8;
  const int64_t chunks = lp.rows_per_head * d8;
  const bool small = chunks * lp.batch * lp.heads < (int64_t{1} << 21);
  const int u = small ? 4 : 1;
  const int64_t want = (chunks + 256 * u - 1) / (256 * u);
  dim3 grid(static_cast<unsigned>(want < 65536 ? want : 65536),
            static_cast<unsigned>(lp.batch * lp.heads));
  dim3 block(256);
  int n = lp.n_tensors;
  const int32_t* map = lp.tile_src_token;
  int64_t tokens = lp.tokens, heads = lp.heads, rows = lp.rows_per_head;
  void* args[] = {&p, &n, &map, &tokens, &heads, &rows};
  const void* fn =
      d8 == 16 ? (small ? reinterpret_cast<const void*>(&tile_layout_kernel<16, 4>)
                        : reinterpret_cast<const void*>(&tile_layout_kernel<16, 1>))
               : (small ? reinterpret_cast<const void*>(&tile_layout_kernel<8, 4>)
                        : reinterpret_cast<const void*>(&tile_layout_kernel<8, 1>));
  return hipLaunchKernel(fn, grid, block, args, 0, stream);
}

hipError_t launch_tile_layout_pool(const LayoutProblem& lp, hipStream_t stream) {
  Ptrs p;
  for (int x = 0; x < 4; ++x) {
    p.src[x] = static_cast<const uint4*>(lp.src[x]);
    p.dst[x] = static_cast<uint4*>(lp.dst[x]);
  }
  const int d8 = lp.head_dim / 8;
  int num_tiles = static_cast<int>(lp.rows_per_head / lp.tile);
  int64_t tiles_all = lp.batch * lp.heads * num_tiles;
  int n = lp.n_tensors, tile = lp.tile;
  const int32_t* map = lp.tile_src_token;
  const int32_t* vbs = lp.block_sizes;
  int64_t tokens = lp.tokens, heads = lp.heads;
  float* pooled = lp.pooled;
  void* args[] = {&p, &n, &map, &vbs, &tokens, &heads, &num_tiles, &tile, &tiles_all, &pooled};
  const void* fn = d8 == 16 ? reinterpret_cast<const void*>(&tile_layout_pool_kernel<16>)
                            : reinterpret_cast<const void*>(&tile_layout_pool_kernel<8>);
  return hipLaunchKernel(fn, dim3(static_cast<unsigned>(tiles_all)), dim3(256), args, 0, stream);
}

hipError_t launch_tile_unlayout(const LayoutProblem& lp, hipStream_t stream) {
  Ptrs p;
  for (int x = 0; x < 4; ++x) {
    p.src[x] = static_cast<const uint4*>(lp.src[x]);
    p.dst[x] = static_cast<uint4*>(lp.dst[x]);
  }
  const int d8 = lp.head_dim / 8;
  const int64_t chunks = lp.tokens * lp.heads * d8;
  const int64_t want = (chunks + 255) / 256;
  dim3 grid(static_cast<unsigned>(want < 65536 ? want : 65536), static_cast<unsigned>(lp.batch));
  dim3 block(256);
  int n = lp.n_tensors;
  const int32_t* map = lp.tile_src_token;
  int64_t tokens = lp.tokens, heads = lp.heads, rows = lp.rows_per_head;
  void* args[] = {&p, &n, &map, &tokens, &heads, &rows};
  const void* fn = d8 == 16 ? reinterpret_cast<const void*>(&tile_unlayout_kernel<16>)
                            : reinterpret_cast<const void*>(&tile_unlayout_kernel<8>);
  return hipLaunchKernel(fn, grid, block, args, 0, stream);
}

}  // namespace bsa
