// Block-sparse tiled attention forward for gfx950 (AMD Instinct MI355X).
//
// FastVideo fastvideo-kernel commit list, page 3:
//  - 128-token sm_121a forward commit: the operation, (q, k, v, q2k_idx,
//    q2k_num, variable_block_sizes) -> out, inference only, no log-sum-exp;
//  - hardening commit: a NaN softmax sum yields a NaN row (test l != 0, not
//    l > 0), rows without keys stay zero, V padding rows are zeroed on
//    partial key chunks and key steps wholly past the valid keys are
//    skipped, so NaN/Inf padding never reaches the output;
//  - Attn-QAT commit: full key tiles run without bounds masks and only the
//    partial tail tile takes the masked step.
//
// Work mapping: one workgroup per (batch*head, query tile); T/32 waves, each
// owning 32 query rows.  For every listed key tile the workgroup stages K
// (row-major) and V (transposed, keys contiguous) in LDS, then each wave
// computes S^T = K Q^T with v_mfma_f32_32x32x16_bf16 so that every lane
// holds the logits of ONE query (16 keys per 32-key block, the other 16 in
// lane^32): the row max and row sum are in-lane reductions plus one exchange
// between the two half-waves.  The online softmax runs in the exp2 domain
// with scale*log2(e) folded into one FMA, and O^T += V^T P^T accumulates in
// fp32 MFMA accumulators.  P is rounded to bf16 for the second product.
//
// MFMA register layouts relied on (v_mfma_f32_32x32x16_bf16, wave64):
//   A (32 x 16): lane l holds A[l % 32][8*(l/32) + e], e = 0..7
//   B (16 x 32): lane l holds B[8*(l/32) + e][l % 32]
//   C (32 x 32): lane l, register r holds C[8*(r/4) + 4*(l/32) + r%4][l % 32]
// A and B share the k-mapping, so any permutation of the contraction index
// applied to both is harmless; the V^T tile in LDS is stored in exactly the
// key order in which the logits sit in the accumulator registers.
//
// Special values (exact, matching the plain definition):
//   - masked logits are SELECTED to -inf (never added), so NaN/Inf in padding
//     K rows cannot leak; padding V rows are written as zero in LDS;
//   - while the running max is -inf the exponent offset is 0, so -inf logits
//     give p = 0 and NaN logits give NaN; a NaN or +inf logit makes l NaN;
//   - the final row is 0 without keys, NaN when keys exist but l == 0 (all
//     logits -inf) or l is NaN, acc / l otherwise; padding query rows are 0.
#include <hip/hip_runtime.h>

#include "bsa_launch.h"

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr float kLog2e = 1.4426950408889634f;

template <int T, int D>
struct Cfg {
  static constexpr int kWaves = T / 32;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int kKStride = D + 8;  // bf16 per K row in LDS (+16 B: no bank conflicts)
  static constexpr int kVStride = T + 8;  // bf16 per V^T row in LDS
  static constexpr int kKBytes = T * kKStride * 2;
  static constexpr int kLdsBytes = kKBytes + D * kVStride * 2;
  static constexpr int kKeyBlocks = T / 32;  // 32-key blocks of S^T
  static constexpr int kKSteps = D / 16;     // k-steps of the QK^T product
  static constexpr int kDBlocks = D / 32;    // 32-row blocks of O^T
  static constexpr int kChunks = D / 8;      // 16-byte chunks per row
};

__device__ __forceinline__ int clampi(int x, int lo, int hi) {
  return x < lo ? lo : (x > hi ? hi : x);
}

// Position of key `key` (a multiple of 4) inside the V^T row: within every
// group of 16 keys the quads are stored in the order 0, 2, 1, 3, so that the
// 8 consecutive positions a half-wave reads hold keys {4h..4h+3, 8+4h..8+4h+3},
// the keys its accumulator registers 8g'..8g'+7 hold.
__device__ __forceinline__ int vt_pos(int key) {
  const int qd = (key >> 2) & 3;
  return (key & ~15) + 4 * (((qd & 1) << 1) | (qd >> 1));
}

__device__ __forceinline__ unsigned bf16_bits(float x) {
  __bf16 b = static_cast<__bf16>(x);  // round to nearest even
  return static_cast<unsigned>(__builtin_bit_cast(unsigned short, b));
}

template <int T, int D>
__global__ __launch_bounds__(2 * T) void bsa_fwd_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const int32_t* __restrict__ q2k_idx,
    const int32_t* __restrict__ q2k_num, const int32_t* __restrict__ vbs,
    uint16_t* __restrict__ out, int num_tiles, int max_sel, float c) {
  using C = Cfg<T, D>;
  __shared__ __attribute__((aligned(16))) uint16_t lds[C::kLdsBytes / 2];
  uint16_t* ks = lds;                      // [T][kKStride]
  uint16_t* vt = lds + C::kKBytes / 2;     // [D][kVStride], keys permuted per vt_pos

  const int tile_i = blockIdx.x;
  const int64_t bh = blockIdx.y;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int col = lane & 31;  // query within the wave's 32 rows; key/d row of A operands
  const int half = lane >> 5;

  const int64_t head_elems = static_cast<int64_t>(num_tiles) * T * D;
  const uint16_t* qh = q + bh * head_elems;
  const uint16_t* kh = k + bh * head_elems;
  const uint16_t* vh = v + bh * head_elems;
  uint16_t* oh = out + bh * head_elems;

  const int vq = clampi(vbs[tile_i], 0, T);
  const int64_t item = bh * num_tiles + tile_i;
  const int count = max_sel > 0 ? clampi(q2k_num[item], 0, max_sel) : 0;
  const int32_t* list = q2k_idx + item * max_sel;

  // Q^T operand (B of the first product): lane (query col, half) holds
  // Q[row][16*kk + 8*half + 0..7].
  const int qrow = wave * 32 + col;
  bf16x8_t qop[C::kKSteps];
  {
    const uint16_t* src = qh + (static_cast<int64_t>(tile_i) * T + qrow) * D + 8 * half;
#pragma unroll
    for (int kk = 0; kk < C::kKSteps; ++kk)
      qop[kk] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(src + 16 * kk));
  }

  f32x16_t acc[C::kDBlocks];
#pragma unroll
  for (int db = 0; db < C::kDBlocks; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[db][r] = 0.0f;
  float m_run = -INFINITY;  // running max of the raw logits of this lane's query
  float l_run = 0.0f;       // this half-wave's share of the softmax sum
  bool any_keys = false;

  for (int n = 0; n < count; ++n) {
    const int j = list[n];
    if (j < 0 || j >= num_tiles) continue;
    const int vk = clampi(vbs[j], 0, T);
    if (vk == 0) continue;
    any_keys = true;

    __syncthreads();  // the previous tile's LDS reads are done
    // ---- stage K_j (rows < vk) row-major --------------------------------------
    {
      const uint16_t* src = kh + static_cast<int64_t>(j) * T * D;
      for (int u = tid; u < T * C::kChunks; u += C::kThreads) {
        const int row = u / C::kChunks, ch = u % C::kChunks;
        if (row < vk)
          *reinterpret_cast<uint4*>(ks + row * C::kKStride + 8 * ch) =
              *reinterpret_cast<const uint4*>(src + row * D + 8 * ch);
      }
    }
    // ---- stage V_j transposed, rows >= vk as zeros ----------------------------
    {
      const uint16_t* src = vh + static_cast<int64_t>(j) * T * D;
      for (int u = tid; u < (T / 4) * C::kChunks; u += C::kThreads) {
        const int quad = u / C::kChunks, ch = u % C::kChunks;
        uint4 r4[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int row = 4 * quad + e;
          r4[e] = row < vk ? *reinterpret_cast<const uint4*>(src + row * D + 8 * ch)
                           : make_uint4(0u, 0u, 0u, 0u);
        }
        const int pos = vt_pos(4 * quad);
        const unsigned* w0 = reinterpret_cast<const unsigned*>(&r4[0]);
        const unsigned* w1 = reinterpret_cast<const unsigned*>(&r4[1]);
        const unsigned* w2 = reinterpret_cast<const unsigned*>(&r4[2]);
        const unsigned* w3 = reinterpret_cast<const unsigned*>(&r4[3]);
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const int d = 8 * ch + 2 * w;
          uint2 lo, hi;
          lo.x = (w0[w] & 0xFFFFu) | (w1[w] << 16);
          lo.y = (w2[w] & 0xFFFFu) | (w3[w] << 16);
          hi.x = (w0[w] >> 16) | (w1[w] & 0xFFFF0000u);
          hi.y = (w2[w] >> 16) | (w3[w] & 0xFFFF0000u);
          *reinterpret_cast<uint2*>(vt + d * C::kVStride + pos) = lo;
          *reinterpret_cast<uint2*>(vt + (d + 1) * C::kVStride + pos) = hi;
        }
      }
    }
    __syncthreads();

    // ---- S^T = K_j Q^T: 32-key blocks past vk are skipped ---------------------
    f32x16_t s[C::kKeyBlocks];
#pragma unroll
    for (int kb = 0; kb < C::kKeyBlocks; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kb][r] = 0.0f;
      if (32 * kb < vk) {
        const uint16_t* arow = ks + (32 * kb + col) * C::kKStride + 8 * half;
#pragma unroll
        for (int kk = 0; kk < C::kKSteps; ++kk) {
          const bf16x8_t a =
              __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(arow + 16 * kk));
          s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qop[kk], s[kb], 0, 0, 0);
        }
      }
    }
    // ---- mask (partial tiles only) and row max --------------------------------
    if (vk < T) {
#pragma unroll
      for (int kb = 0; kb < C::kKeyBlocks; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = 32 * kb + 8 * (r >> 2) + 4 * half + (r & 3);
          if (key >= vk) s[kb][r] = -INFINITY;
        }
    }
    float mt = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < C::kKeyBlocks; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mt = fmaxf(mt, s[kb][r]);
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    const float m_new = fmaxf(m_run, mt);
    const float mc = (m_new == -INFINITY ? 0.0f : m_new) * c;
    const float alpha = __builtin_amdgcn_exp2f(m_run * c - mc);
    float psum = 0.0f;
#pragma unroll
    for (int kb = 0; kb < C::kKeyBlocks; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][r], c, -mc));
        s[kb][r] = p;
        psum += p;
      }
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int db = 0; db < C::kDBlocks; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[db][r] *= alpha;

    // ---- O^T += V_j^T P^T over 16-key chunks below vk -------------------------
#pragma unroll
    for (int kc = 0; kc < T / 16; ++kc) {
      if (16 * kc < vk) {
        bf16x8_t pb;
#pragma unroll
        for (int e = 0; e < 8; ++e) pb[e] = static_cast<__bf16>(s[kc >> 1][8 * (kc & 1) + e]);
#pragma unroll
        for (int db = 0; db < C::kDBlocks; ++db) {
          const bf16x8_t a = __builtin_bit_cast(
              bf16x8_t, *reinterpret_cast<const uint4*>(vt + (32 * db + col) * C::kVStride +
                                                         16 * kc + 8 * half));
          acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb, acc[db], 0, 0, 0);
        }
      }
    }
  }

  // ---- epilogue ----------------------------------------------------------------
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const bool zero_row = !any_keys || qrow >= vq;
  const float inv = l_tot != 0.0f ? 1.0f / l_tot : __builtin_nanf("");
  uint16_t* dst = oh + (static_cast<int64_t>(tile_i) * T + qrow) * D + 4 * half;
#pragma unroll
  for (int db = 0; db < C::kDBlocks; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      uint2 pk;
      const float x0 = zero_row ? 0.0f : acc[db][4 * g + 0] * inv;
      const float x1 = zero_row ? 0.0f : acc[db][4 * g + 1] * inv;
      const float x2 = zero_row ? 0.0f : acc[db][4 * g + 2] * inv;
      const float x3 = zero_row ? 0.0f : acc[db][4 * g + 3] * inv;
      pk.x = bf16_bits(x0) | (bf16_bits(x1) << 16);
      pk.y = bf16_bits(x2) | (bf16_bits(x3) << 16);
      *reinterpret_cast<uint2*>(dst + 32 * db + 8 * g) = pk;
    }
}

template <int T, int D>
hipError_t launch(const bsa::FwdProblem& p, hipStream_t stream) {
  const void* fn = reinterpret_cast<const void*>(&bsa_fwd_kernel<T, D>);
  dim3 grid(static_cast<unsigned>(p.num_tiles), static_cast<unsigned>(p.batch_heads));
  dim3 block(Cfg<T, D>::kThreads);
  const float c = static_cast<float>(1.0 / __builtin_sqrt(static_cast<double>(D))) * kLog2e;
  const uint16_t* q = p.q;
  const uint16_t* k = p.k;
  const uint16_t* v = p.v;
  const int32_t* idx = p.q2k_idx;
  const int32_t* num = p.q2k_num;
  const int32_t* vbs = p.block_sizes;
  uint16_t* out = p.out;
  int nt = p.num_tiles, ms = p.max_sel;
  float cc = c;
  void* args[] = {&q, &k, &v, &idx, &num, &vbs, &out, &nt, &ms, &cc};
  return hipLaunchKernel(fn, grid, block, args, 0, stream);
}

}  // namespace

namespace bsa {

hipError_t launch_fwd(const FwdProblem& p, hipStream_t stream) {
  if (p.tile == 128) return p.head_dim == 128 ? launch<128, 128>(p, stream)
                                               : launch<128, 64>(p, stream);
  return p.head_dim == 128 ? launch<64, 128>(p, stream) : launch<64, 64>(p, stream);
}

}  // namespace bsa
