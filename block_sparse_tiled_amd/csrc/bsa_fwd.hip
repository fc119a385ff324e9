// Block-sparse tiled attention forward for gfx950 (AMD Instinct MI355X).
//
// FastVideo fastvideo-kernel commit list, page 3:
//  - 128-token sm_121a forward commit: the operation, (q, k, v, q2k_idx,
//    q2k_num, variable_block_sizes) -> out, inference only, no log-sum-exp;
//  - hardening commit: a NaN softmax sum yields a NaN row (test l != 0, not
//    l > 0), rows without keys stay zero, V padding rows are zeroed on
//    partial key chunks and key steps wholly past the valid keys are
//    skipped, so NaN/Inf padding never reaches the output; its QK/PV overlap
//    (one tile's loads in flight while another is computed) is realised
//    here with LDS DMA;
//  - Attn-QAT commit: full key tiles run without bounds masks and only the
//    partial tail tile takes the masked step.
//
// Work mapping.  One workgroup per (batch*head, query tile) with T/32 waves,
// each wave owning 32 query rows.  Workgroups are renumbered so that each of
// the 8 XCDs (dispatched round-robin by linear workgroup id) receives a
// contiguous run of work items, i.e. whole heads: the key tiles a head's
// lists share then stay in that XCD's L2.
//
// Data movement.  K and V tiles are copied HBM -> LDS with LDS DMA
// (global_load_lds_dwordx4, 16 bytes per lane, no registers).  Rows are dense
// in LDS with the 16-byte chunks of each row XOR-swizzled by the row index so
// that the MFMA operand reads are free of bank conflicts.  One K and one V
// buffer per workgroup: K(n+1) is requested as soon as every wave has
// finished reading K(n) and lands during the softmax and P.V of tile n;
// V(n+1) is requested after P.V(n) and lands during Q.K(n+1).
//
// Math.  Each wave computes S^T = K Q^T with v_mfma_f32_32x32x16_bf16, so
// every lane holds the logits of ONE query (16 keys per 32-key block, the
// other 16 in lane^32): the row max is an in-lane reduction plus one
// v_permlane32_swap, and the running sum stays split across the two halves
// until the end.  The online softmax runs in the exp2 domain with
// scale*log2(e) folded into one FMA; P is rounded to bf16 once and both the
// row sum (v_dot2 with ones) and O^T += V^T P^T use those rounded values.
// V^T operands come straight from the row-major V tile through the LDS
// transpose read ds_read_b64_tr_b16.
//
// The MFMA and LDS-transpose register layouts relied on are listed in
// bsa_fwd_common.h.
//
// Special values (exact, matching the plain definition):
//   - masked logits are SELECTED to -inf (never added), so NaN/Inf in padding
//     K rows cannot leak; padding V rows are overwritten with zeros in LDS;
//   - while the running max is -inf the exponent offset is 0, so -inf logits
//     give p = 0 and NaN logits give NaN; a NaN or +inf logit makes l NaN;
//   - the final row is 0 without keys, NaN when keys exist but l == 0 (all
//     logits -inf) or l is NaN, acc / l otherwise; padding query rows are 0.
#include <hip/hip_runtime.h>

#include "bsa_fwd_common.h"
#include "bsa_launch.h"

namespace {

using namespace bsa::detail;

template <int T, int D>
__global__ __launch_bounds__(2 * T) __attribute__((amdgpu_waves_per_eu(2, T == 128 ? 2 : 4)))
void bsa_fwd_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                    const uint16_t* __restrict__ v, const int32_t* __restrict__ q2k_idx,
                    const int32_t* __restrict__ q2k_num, const int32_t* __restrict__ vbs,
                    uint16_t* __restrict__ out, int num_tiles, int max_sel, int num_items,
                    float c) {
  using C = Cfg<T, D>;
  __shared__ __attribute__((aligned(1024))) uint16_t ks[T * D];
  __shared__ __attribute__((aligned(1024))) uint16_t vs[T * D];

  // XCD-aware renumbering: linear id L runs on XCD L % 8; give XCD x the
  // contiguous items [start(x), start(x) + count(x)).
  const int L = blockIdx.x + blockIdx.y * gridDim.x;
  const int xcd = L & 7, slot = L >> 3;
  const int per = num_items >> 3, rem = num_items & 7;
  const int item = xcd * per + (xcd < rem ? xcd : rem) + slot;
  const int64_t bh = item / num_tiles;
  const int tile_i = item - static_cast<int>(bh) * num_tiles;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wave
  const int col = lane & 31;
  const int half = lane >> 5;

  const int64_t head_elems = static_cast<int64_t>(num_tiles) * T * D;
  const uint16_t* qh = q + bh * head_elems;
  const uint16_t* kh = k + bh * head_elems;
  const uint16_t* vh = v + bh * head_elems;
  uint16_t* oh = out + bh * head_elems;

  const int vq = clampi(vbs[tile_i], 0, T);
  const int64_t item64 = bh * num_tiles + tile_i;
  const int count = max_sel > 0 ? clampi(q2k_num[item64], 0, max_sel) : 0;
  const int32_t* list = q2k_idx + item64 * max_sel;

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
  // Q must be in registers before the first tile DMA is issued: the DMAs are
  // invisible to the compiler's wait-count bookkeeping, and an explicit drain
  // here keeps it from placing waits for Q inside the tile loop.
  wait_vmcnt<0>();

  f32x16_t acc[C::kDBlocks];
#pragma unroll
  for (int db = 0; db < C::kDBlocks; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[db][r] = 0.0f;
  float m_run = -INFINITY;  // running max of the raw logits of this lane's query
  float l_run = 0.0f;       // this half-wave's share of the softmax sum
  bool any_keys = false;

  int n = 0, vk = 0;
  int j = next_tile(list, count, vbs, num_tiles, T, n, vk);
  if (j >= 0) {
    dma_tile<T, D, false>(kh + static_cast<int64_t>(j) * T * D, ks, wave, lane);
    dma_tile<T, D, true>(vh + static_cast<int64_t>(j) * T * D, vs, wave, lane);
  }

  // Loop-invariant parts of the LDS operand addresses.
  const int k_swz = swz_k<D>(col);  // rows 32*kb + col share it
  const int tr_i = lane & 15, tr_g = (lane >> 4) & 1;
  const int v_row = 4 * half + (tr_i >> 2);  // + 16*kc (+ 8 for the high half)
  const int v_swz = swz_v<D>(v_row);
  const bf16x2_t ones = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};
  const f32x16_t zero16 = {};

  while (j >= 0) {
    any_keys = true;
    int n2 = n + 1, vk2 = 0;
    const int j2 = next_tile(list, count, vbs, num_tiles, T, n2, vk2);
    const int nkb = (vk + 31) >> 5;  // 32-key blocks holding valid keys

    wait_vmcnt<C::kDmaPerTile>();  // K(j) has landed (V(j) may be in flight)
    lds_barrier();

    // ---- S^T = K_j Q^T over the blocks below vk ----------------------------------
    f32x16_t s[C::kKeyBlocks];
#pragma unroll
    for (int kb = 0; kb < C::kKeyBlocks; ++kb) {
      if (kb < nkb) {
        const uint16_t* base = ks + (32 * kb + col) * D;
#pragma unroll
        for (int kk = 0; kk < C::kKSteps; ++kk) {
          const int chunk = (2 * kk + half) ^ k_swz;
          const bf16x8_t a =
              __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(base + 8 * chunk));
          s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qop[kk], kk ? s[kb] : zero16,
                                                          0, 0, 0);
        }
      }
    }
    lds_barrier();  // every wave is done with K(j)
    if (j2 >= 0) dma_tile<T, D, false>(kh + static_cast<int64_t>(j2) * T * D, ks, wave, lane);

    // ---- mask the partial block, running max ---------------------------------------
    if (vk & 31) {
      const int kbp = vk >> 5;
      const int lim = (vk & 31) - 4 * half;  // register r holds key 8*(r/4) + r%4 (+4*half)
#pragma unroll
      for (int kb = 0; kb < C::kKeyBlocks; ++kb)
        if (kb == kbp) {
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (8 * (r >> 2) + (r & 3) >= lim) s[kb][r] = -INFINITY;
        }
    }
    float mt = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < C::kKeyBlocks; ++kb)
      if (kb < nkb) {
        mt = max3<true>(mt, s[kb][0], s[kb][1]);
#pragma unroll
        for (int r = 2; r < 16; r += 2) mt = max3<false>(mt, s[kb][r], s[kb][r + 1]);
      }
    {
      float a, b;
      swap_halves(mt, a, b);
      mt = fmaxf(a, b);
    }
    const float m_new = fmaxf(m_run, mt);
    const float mc = (m_new == -INFINITY ? 0.0f : m_new) * c;
    const float alpha = __builtin_amdgcn_exp2f(m_run * c - mc);
    m_run = m_new;
    l_run *= alpha;
    if (__any(alpha != 1.0f)) {
#pragma unroll
      for (int db = 0; db < C::kDBlocks; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[db][r] *= alpha;
    }

    // ---- V(j) in LDS: wait, blank its padding rows -----------------------------------
    if (j2 >= 0) {
      wait_vmcnt<C::kDmaPerTile>();
    } else {
      wait_vmcnt<0>();
    }
    if (vk < T) zero_padding_rows<T, D>(vs, vk, wave, lane);
    lds_barrier();

    // ---- per 16-key chunk: P = exp2(S*c - m*c) in bf16, row sum, O^T += V^T P^T ------
#pragma unroll
    for (int kc = 0; kc < C::kKeyChunks; ++kc) {
      if (16 * kc < vk) {
        const f32x16_t& sb = s[kc >> 1];
        const int e0 = 8 * (kc & 1);
        bf16x2_t pp[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          pp[e] = to_bf16x2(
              __builtin_amdgcn_exp2f(__builtin_fmaf(sb[e0 + 2 * e], c, -mc)),
              __builtin_amdgcn_exp2f(__builtin_fmaf(sb[e0 + 2 * e + 1], c, -mc)));
          l_run = __builtin_amdgcn_fdot2_f32_bf16(pp[e], ones, l_run, false);
        }
        const bf16x8_t pk = __builtin_shufflevector(
            __builtin_shufflevector(pp[0], pp[1], 0, 1, 2, 3),
            __builtin_shufflevector(pp[2], pp[3], 0, 1, 2, 3), 0, 1, 2, 3, 4, 5, 6, 7);
        const uint16_t* vrow = vs + (16 * kc + v_row) * D;
#pragma unroll
        for (int db = 0; db < C::kDBlocks; ++db) {
          const int colv = 32 * db + 16 * tr_g + 4 * (tr_i & 3);
          const int off = ((colv >> 3) ^ v_swz) * 8 + (colv & 7);
          const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(vrow + off));
          const i16x4_t hi =
              __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(vrow + 8 * D + off));
          const bf16x8_t a = __builtin_bit_cast(
              bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
          acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pk, acc[db], 0, 0, 0);
        }
      }
    }
    lds_barrier();  // every wave is done with V(j)
    if (j2 >= 0) dma_tile<T, D, true>(vh + static_cast<int64_t>(j2) * T * D, vs, wave, lane);

    j = j2;
    vk = vk2;
    n = n2;
  }

  // ---- epilogue ------------------------------------------------------------------
  float l_tot;
  {
    float a, b;
    swap_halves(l_run, a, b);
    l_tot = a + b;
  }
  const bool zero_row = !any_keys || qrow >= vq;
  const float inv = l_tot != 0.0f ? 1.0f / l_tot : __builtin_nanf("");
  uint16_t* dst = oh + (static_cast<int64_t>(tile_i) * T + qrow) * D + 4 * half;
#pragma unroll
  for (int db = 0; db < C::kDBlocks; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      float x[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] = zero_row ? 0.0f : acc[db][4 * g + e] * inv;
      const bf16x2_t lo = to_bf16x2(x[0], x[1]);
      const bf16x2_t hi = to_bf16x2(x[2], x[3]);
      uint2 pkd;
      pkd.x = __builtin_bit_cast(unsigned, lo);
      pkd.y = __builtin_bit_cast(unsigned, hi);
      *reinterpret_cast<uint2*>(dst + 32 * db + 8 * g) = pkd;
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
  int items = static_cast<int>(p.batch_heads * p.num_tiles);
  float cc = c;
  void* args[] = {&q, &k, &v, &idx, &num, &vbs, &out, &nt, &ms, &items, &cc};
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
