// Block-sparse tiled attention forward for gfx950 (AMD Instinct MI355X).
//
// FastVideo fastvideo-kernel commit list, page 3:
//  - 128-token sm_121a forward commit: the operation, (q, k, v, q2k_idx,
//    q2k_num, variable_block_sizes) -> out, a forward without log-sum-exp;
//  - hardening commit: a NaN softmax sum yields a NaN row (test l != 0, not
//    l > 0), rows without keys stay zero, and NaN/Inf in padding rows never
//    reach the output; its QK/PV overlap (one tile's loads in flight while
//    another is computed) is realised here with LDS DMA;
//  - Attn-QAT commit: full key tiles run without bounds masks; here only
//    tiles shorter than T take the mask, and only on the 32-key blocks that
//    reach the valid length.
// That commit also drops key steps entirely beyond the valid keys; this kernel
// instead runs every tile at full size (masked logits give p = 0 against
// zeroed V rows, adding exact zeros), which keeps one register assignment
// for the accumulators across the tile loop.
//
// Work mapping.  A work unit is one (batch*head, query tile) item, or one
// list segment of an item: items that fill whole rounds of resident
// workgroups run whole, and the items left over for a last, mostly empty
// round are cut into list segments (see plan()).  One workgroup of T/32
// waves per unit, each wave owning 32 query rows.  Units are renumbered so
// that each of the 8 XCDs (dispatched round-robin by linear workgroup id)
// receives a contiguous run, i.e. whole heads: the workgroups of one XCD
// start together on consecutive query tiles of one head and sweep its key
// tiles together, so the tiles stay in that XCD's L2.
//
// Data movement.  Each list chunk is first compacted into LDS (usable tile
// indices with their valid lengths).  K and V tiles are copied HBM -> LDS
// with LDS DMA (global_load_lds_dwordx4, 16 bytes per lane, no registers).
// Rows are dense in LDS with the 16-byte chunks of each row XOR-swizzled by
// the row index so that the MFMA operand reads are free of bank conflicts.
// One K and one V buffer per workgroup (two workgroups share a CU): K(n+1) is
// requested as soon as every wave has finished reading K(n) and lands during
// the softmax and P.V of tile n; V(n+1) is requested after P.V(n) and lands
// during Q.K(n+1).  Two workgroup barriers per tile: after Q.K(n) (K(n) free,
// V(n) landed and visible) and after P.V(n) (V(n) free, K(n+1) visible).
//
// Math.  Each wave computes S^T = K Q^T with v_mfma_f32_32x32x16_bf16, k-step
// outer over independent accumulators, so every lane holds the logits of ONE
// query (16 keys per 32-key block, the other 16 in lane^32): the row max is
// an in-lane reduction plus one v_permlane32_swap, and the running sum stays
// split across the two halves until the end.  The online softmax runs in the
// exp2 domain with scale*log2(e) folded into one FMA, and the exponent offset
// follows the running max lazily (only rises of more than 8 in exp2 units);
// P is rounded to bf16 for O^T += V^T P^T and the row sum adds the fp32 p.
// V^T operands come straight from the row-major V tile through the LDS
// transpose read ds_read_b64_tr_b16.  Operand reads run one step ahead of the
// MFMAs that use them, and in P.V the exponentials of the next 16-key chunk
// are interleaved with the MFMAs of the current one.
//
// Split items.  A segment stores its (m, l, unnormalised O) partial in a
// slot of the caller's workspace; a second, small launch on the same stream
// merges each split item's partials in segment order (the same guarded
// rescaling as the online update) and stores its rows.  The kernel boundary
// orders the partial stores before their reads on every XCD, so the
// workspace is ordinary device memory and needs no counters, atomics or
// clearing.
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

#include <atomic>

#include "bsa_fwd_common.h"
#include "bsa_launch.h"

namespace {

using namespace bsa::detail;

// Partial results of a split item, one slot per segment: the unnormalised
// accumulator in register order (float index (((wave*kDBlocks + db)*4 + r/4)
// *64 + lane)*4 + r%4), then per lane the running max and this half-wave's
// share of the sum, then the any-keys flag.
template <int T, int D>
struct Slot {
  using C = Cfg<T, D>;
  static constexpr int kAcc = C::kWaves * C::kDBlocks * 16 * 64;  // floats
  static constexpr int kM = kAcc;
  static constexpr int kL = kAcc + C::kWaves * 64;
  static constexpr int kAny = kAcc + 2 * C::kWaves * 64;
  static constexpr int kFloats = kAny + 64;  // keeps slots 256-byte aligned
};

// Normalise and store the 32 x D rows of one wave of query tile `itile` of
// head `ibh` (0 for padding query rows and rows without keys; NaN when l == 0
// or l is NaN).  acc, m_run and l_run are the wave's accumulators in the
// kernel's register layout (l_run: this half-wave's share of the sum).  With
// lse, also each row's log-sum-exp and, in out_lo, the bf16 rounding residual
// of every stored value (out_lo = bf16(o - out) for the fp32 result o), from
// which the backward forms dO . o to about 2^-17 of its size.
template <int T, int D>
__device__ __forceinline__ void store_tile_rows(const f32x16_t* acc, float m_run, float l_run,
                                                bool any_keys, int64_t ibh, int itile,
                                                int num_tiles, const int32_t* __restrict__ vbs,
                                                int sub_shift, int wave, int lane, float c,
                                                uint16_t* __restrict__ out, float* __restrict__ lse,
                                                uint16_t* __restrict__ out_lo) {
  using C = Cfg<T, D>;
  const int vq = clampi(vbs[itile >> sub_shift] - T * (itile & ((1 << sub_shift) - 1)), 0, T);
  const int ln = launder(lane);  // per-lane addresses computed here, not hoisted
  const int row = wave * 32 + (ln & 31);
  float l_tot;
  {
    float lo_half, hi_half;
    swap_halves(l_run, lo_half, hi_half);
    l_tot = lo_half + hi_half;
  }
  const bool zero_row = !any_keys || row >= vq;
  const float inv = l_tot != 0.0f ? 1.0f / l_tot : __builtin_nanf("");
  const int64_t row_id = (ibh * num_tiles + itile) * T + row;
  if (lse != nullptr && ln < 32) {
    // natural-log log-sum-exp of the scaled logits: (m*c + log2 l) * ln 2,
    // with the exponent offset m*c taken as 0 while m is -inf (then l is 0
    // and the result -inf); -inf for padding rows and rows without keys
    const float mc = (m_run == -INFINITY ? 0.0f : m_run) * c;
    lse[row_id] = zero_row ? -INFINITY : (mc + __builtin_amdgcn_logf(l_tot)) * 0.69314718055994531f;
  }
  const int64_t off = row_id * D + 4 * (ln >> 5);
#pragma unroll
  for (int db = 0; db < C::kDBlocks; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      float x[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] = zero_row ? 0.0f : acc[db][4 * g + e] * inv;
      const unsigned w0 = __builtin_bit_cast(unsigned, to_bf16x2(x[0], x[1]));
      const unsigned w1 = __builtin_bit_cast(unsigned, to_bf16x2(x[2], x[3]));
      *reinterpret_cast<uint2*>(out + off + 32 * db + 8 * g) = make_uint2(w0, w1);
      if (lse != nullptr) {
        // element 0 of a bf16 pair is its low half
        const float r0 = x[0] - __uint_as_float(w0 << 16);
        const float r1 = x[1] - __uint_as_float(w0 & 0xffff0000u);
        const float r2 = x[2] - __uint_as_float(w1 << 16);
        const float r3 = x[3] - __uint_as_float(w1 & 0xffff0000u);
        *reinterpret_cast<uint2*>(out_lo + off + 32 * db + 8 * g) =
            make_uint2(__builtin_bit_cast(unsigned, to_bf16x2(r0, r1)),
                       __builtin_bit_cast(unsigned, to_bf16x2(r2, r3)));
      }
    }
}

// Persistent launch (kPersistent): one round of workgroups, each taking work
// units from queues instead of one unit per dispatched workgroup.  With many
// short units of uneven cost (one round of workgroups per 4 or more rounds of
// units), dispatch in linear order leaves slots idle: a slot freed on one XCD
// waits until the workgroups ahead of its next one have found free slots on
// the other XCDs.  next_unit() returns the linear id that a one-unit launch
// would have given the unit (so the XCD renumbering applies unchanged), or -1
// once every queue is empty.  Queue x holds the ids x, x + 8, x + 16, ... below
// `units` in order, behind an atomic counter; a workgroup draws from the queue
// of its own XCD (its linear id mod 8, the dispatch order) and, once that is
// empty, from the others in turn.  Units are independent, so which workgroup
// runs one does not change a bit of the result.
__device__ __forceinline__ int next_unit(uint32_t* __restrict__ queue, int units, int& xq,
                                         int* s_unit) {
  __syncthreads();  // every thread has read the previous unit
  if (threadIdx.x == 0) {
    int L = -1;
    for (int tries = 0; tries < 8; ++tries) {
      const int x = (xq + tries) & 7;
      const uint32_t kq = atomicAdd(queue + 16 * x, 1u);  // counters 64 bytes apart
      const int64_t Lc = 8 * static_cast<int64_t>(kq) + x;
      if (Lc < units) {
        L = static_cast<int>(Lc);
        xq = x;
        break;
      }
    }
    *s_unit = L;
  }
  __syncthreads();
  return *s_unit;
}

// Zeroes the queue counters (kFwdQueueBytes) before a persistent launch: a
// kernel, so that the pair can be captured into a graph.
__global__ void clear_queue_kernel(uint32_t* __restrict__ queue) {
  if (threadIdx.x < bsa::kFwdQueueBytes / 4) queue[threadIdx.x] = 0u;
}

// kTrain: the forward of the training path (bsa_fwd_lse).  It writes the
// log-sum-exp and the output's rounding residual, and its exponent offset
// follows the running max eagerly, so that a row's largest logit gets
// p = exp2(0) = 1, which bf16 holds exactly: on a sharply peaked row the bf16
// rounding of that one p would otherwise enter o at 2^-9 of |o| and, through
// D = dO . o, dominate the backward's dS = P (dP - D).
template <int T, int D, bool kTrain, bool kPersistent>
__global__ __launch_bounds__(2 * T) __attribute__((amdgpu_waves_per_eu(2, T == 128 ? 2 : 4)))
void bsa_fwd_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                    const uint16_t* __restrict__ v, const int32_t* __restrict__ q2k_idx,
                    const int32_t* __restrict__ q2k_num, const int32_t* __restrict__ vbs,
                    uint16_t* __restrict__ out, int num_tiles, int max_sel, int n_whole,
                    int n_whole_padded, int n_split_units, int splits, float* __restrict__ ws,
                    float c, float* __restrict__ lse, uint16_t* __restrict__ out_lo,
                    int sub_shift, uint32_t* __restrict__ queue, int total_units) {
  using C = Cfg<T, D>;
  using S = Slot<T, D>;
  __shared__ __attribute__((aligned(1024))) uint16_t ks[T * D];
  __shared__ __attribute__((aligned(1024))) uint16_t vs[T * D];
  // the steps of the current chunk (compact_steps): two int2 per step, at
  // most one step per T-row part of a list entry (two parts per entry when
  // the lists name tiles of 2T rows)
  // Two key tiles share a step at T = 128 only: at T = 64 the step is bound by
  // the tile copies, which pairing does not reduce, and the pairing's order
  // and bookkeeping cost more than the steps it saves.
  constexpr bool kPairs = T == 128;
  __shared__ int2 st[2 * (T == 128 ? 2 : 1) * C::kThreads];
  __shared__ int2 srt[kPairs ? 2 * C::kThreads : 1];  // the parts by length (compact_steps)
  __shared__ int wave_scratch[5 * C::kWaves];

  // One work unit (linear id L); `return` ends the unit.
  auto unit = [&](const int L) {
  // Work units: items [0, n_whole) whole, one workgroup each, dispatched
  // first; then each of the remaining items cut into `splits` list segments
  // (segment s covers list positions [s*n/splits, (s+1)*n/splits) of the
  // item's n = max(max_sel, 1)), whose partial results are merged.
  // XCD-aware renumbering: linear id L runs on XCD L % 8.  Within each set,
  // XCD x receives a contiguous run of units, i.e. whole heads, so the key
  // tiles a head's lists share stay in that XCD's L2, and the workgroups of
  // one XCD, started together on consecutive query tiles, sweep the same key
  // tiles at the same time.  The first set is padded to a multiple of 8
  // units so that the second starts on XCD 0.
  const int xcd = L & 7;
  int item, seg = 0, nseg = 1, unit2 = 0;
  if (L < n_whole_padded) {
    item = xcd * (n_whole_padded >> 3) + (L >> 3);
    if (item >= n_whole) return;  // padding unit
  } else {
    const int l2 = L - n_whole_padded;
    const int per = n_split_units >> 3, rem = n_split_units & 7;
    unit2 = xcd * per + (xcd < rem ? xcd : rem) + (l2 >> 3);
    item = n_whole + unit2 / splits;
    seg = unit2 - (unit2 / splits) * splits;
    nseg = splits;
  }
  const int positions = max_sel > 0 ? max_sel : 1;
  const int a = static_cast<int>(static_cast<int64_t>(seg) * positions / nseg);
  const int b = static_cast<int>(static_cast<int64_t>(seg + 1) * positions / nseg);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wave
  const int col = lane & 31;
  const int half = lane >> 5;
  const int qrow = wave * 32 + col;

  const int64_t bh = item / num_tiles;
  const int tile_i = item - static_cast<int>(bh) * num_tiles;
  const int64_t head_elems = static_cast<int64_t>(num_tiles) * T * D;
  const uint16_t* qh = q + bh * head_elems;
  const uint16_t* kh = k + bh * head_elems;
  const uint16_t* vh = v + bh * head_elems;
  // Lists and lengths count tiles of T << sub_shift rows ("list tiles"); the
  // kernel works on T-row tiles, sub_shift + 1 of them per list tile (the
  // row layout is the same).
  const int nt_list = num_tiles >> sub_shift;
  const int tile_l = tile_i >> sub_shift;
  const int64_t item_l = bh * nt_list + tile_l;
  const int count = max_sel > 0 ? clampi(q2k_num[item_l], 0, max_sel) : 0;
  // A wave whose 32 query rows are all padding only copies and synchronises:
  // its rows are written +0 whatever it computes (the other wave on its SIMD
  // gets the issue slots).
  const bool active = wave * 32 < clampi(vbs[tile_l] - T * (tile_i & ((1 << sub_shift) - 1)), 0, T);
  const int32_t* list = q2k_idx + item_l * max_sel;
  const int end = b < count ? b : count;

  // Q^T operand (B of the first product): lane (query col, half) holds
  // Q[row][16*kk + 8*half + 0..7].
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
    for (int rr = 0; rr < 16; ++rr) acc[db][rr] = 0.0f;
  float m_run = -INFINITY;  // running max of the raw logits of this lane's query
  float l_run = 0.0f;       // this half-wave's share of the softmax sum
  bool any_keys = false;

  const DmaLane<T, D, false> k_dma(wave, lane);
  const DmaLane<T, D, true> v_dma(wave, lane);
  // Loop-invariant parts of the LDS operand addresses.
  const int k_swz = swz_k<D>(col);  // rows 32*kb + col share it
  const int tr_i = lane & 15, tr_g = (lane >> 4) & 1;
  const int v_row = 4 * half + (tr_i >> 2);  // + 16*kc (+ 8 for the high half)
  const int v_swz = swz_v<D>(v_row);
  const f32x16_t zero16 = {};
  const float neg_inf = launder_f(-INFINITY);

  // K operands of k-step kk for every 32-key block.
  // (the per-lane swizzle is laundered so that the addresses of all k-steps
  // are recomputed per step rather than held in registers across the loop)
  auto read_k = [&](int kk, bf16x8_t* dst) {
    constexpr int NKB = C::kKeyBlocks;
    const int chunk = (2 * kk + half) ^ launder(k_swz);
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
      dst[kb] = __builtin_bit_cast(
          bf16x8_t, *reinterpret_cast<const uint4*>(ks + (32 * kb + col) * D + 8 * chunk));
  };
  // V^T operands of 16-key chunk kc for every 32-row block of O^T.
  auto read_v = [&](int kc, bf16x8_t* dst) {
    const uint16_t* vrow = vs + (16 * kc + v_row) * D;
#pragma unroll
    for (int db = 0; db < C::kDBlocks; ++db) {
      const int colv = 32 * db + 16 * tr_g + 4 * (tr_i & 3);
      const int off = ((colv >> 3) ^ v_swz) * 8 + (colv & 7);
      const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(vrow + off));
      const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(vrow + 8 * D + off));
      dst[db] = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }
  };

  // The copy of step n = (j, vk) into the K or V buffer: one tile (j >= 0) or
  // a pair of tiles that fit in T rows together (j <= -2, the rest of the step
  // in st[2n + 1]); j = -1: no step.  The pair's test sits behind the single
  // tile's, so a list of whole tiles runs the same instructions as without
  // pairs.
  auto copy_step = [&](auto is_v, auto skip, int n, int j, int vk) {
    constexpr bool kV = decltype(is_v)::value, kSkip = decltype(skip)::value;
    const uint16_t* head = kV ? vh : kh;
    uint16_t* buf = kV ? vs : ks;
    const auto& dl = [&]() -> const auto& {
      if constexpr (kV)
        return v_dma;
      else
        return k_dma;
    }();
    if (j >= 0) {
      dma_tile<T, D, kV, kSkip>(head + static_cast<int64_t>(j) * T * D, buf, wave, dl, vk);
    } else if (kPairs && j <= -2) {
      const int2 bv = st[2 * n + 1];
      const int jb = __builtin_amdgcn_readfirstlane(bv.x), va = __builtin_amdgcn_readfirstlane(bv.y);
      dma_pair<T, D, kV, kSkip>(head, -2 - j, va, jb, vk - va, buf, wave, lane, dl);
    }
  };

  // One step of vk valid keys (1 <= vk <= T): a tile, or two tiles packed
  // into the first vk rows of the buffers.  On entry its K is in LDS
  // and visible, its V may be in flight; on exit the K of step n2 = (j2, vk2)
  // is in LDS and visible and its V is requested.  Every step is full-size
  // (all T/32 key blocks): keys at or past vk are masked, and a single step
  // keeps the accumulators in one register assignment across the loop (a
  // second, half-size step made the compiler move all of them every tile).
  auto tile_step = [&](int vk, int n2, int j2, int vk2) {
    constexpr int NKB = C::kKeyBlocks;

    // ---- S^T = K_j Q^T, k-step outer: NKB independent accumulators, the
    //      operands of step kk + 1 requested before the MFMAs of step kk ----------
    f32x16_t s[NKB];
    bf16x8_t kop[2][NKB];  // operands of steps kk (kop[kk & 1]) and kk + 1, no copies
    if (active) {
      read_k(0, kop[0]);
#pragma unroll
      for (int kk = 0; kk < C::kKSteps; ++kk) {
        if (kk + 1 < C::kKSteps) read_k(kk + 1, kop[(kk + 1) & 1]);
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
          s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop[kk & 1][kb], qop[kk],
                                                          kk ? s[kb] : zero16, 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);  // keeps the reads one step ahead, no further
      }
    }
    wait_vmcnt<0>();  // V(j) (the only copy in flight)
    if (vk < T) zero_padding_rows<T, D>(vs, vk, wave, lane);
    lds_barrier();  // every wave is done with K(j); V(j) is visible
    copy_step(Flag<false>{}, Flag<true>{}, n2, j2, vk2);

    // ---- mask keys at or past vk (whole blocks included), running max ------------
    if (active) {
    if (vk < 32 * NKB) {
      // register r of block kb holds key 32*kb + 8*(r/4) + r%4 (+ 4 in the high
      // half-wave): masked when 8*(r/4) + r%4 >= t = vk - 32*kb - 4*half, a
      // compare against a small inline constant per register
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
        if (32 * kb + 32 > vk) {  // only the blocks that reach vk (uniform branch)
          const int t = launder(vk - 32 * kb - 4 * half);
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (8 * (r >> 2) + (r & 3) >= t) s[kb][r] = -INFINITY;
        }
    }
    float mx[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
      mx[kb] = kb == 0 ? max3<true>(neg_inf, s[0][0], s[0][1])
                       : max3<false>(neg_inf, s[kb][0], s[kb][1]);
#pragma unroll
    for (int r = 2; r < 16; r += 2)
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) mx[kb] = max3<false>(mx[kb], s[kb][r], s[kb][r + 1]);
    float mt = mx[0];
#pragma unroll
    for (int kb = 1; kb < NKB; kb += 2)
      mt = max3<false>(mt, mx[kb], kb + 1 < NKB ? mx[kb + 1] : mx[kb]);
    {
      float a, b;
      swap_halves(mt, a, b);
      mt = fmaxf(a, b);
    }
    // The exponent offset m_run follows the running max only when the max
    // rises by more than kRescaleSlack in exp2 units (or leaves -inf); below
    // that, p = exp2(s*c - m_run*c) stays under 2^kRescaleSlack, which bf16 P
    // and the fp32 sums hold, and the accumulators are not rescaled.  The
    // result is the same quotient.  NaN differences (-inf to -inf, +inf to
    // +inf) compare false and keep the offset.  The training variant takes
    // every rise (slack 0).
    constexpr float kSlack = kTrain ? 0.0f : kRescaleSlack;
    const float m_new = fmaxf(m_run, mt);
    const bool raise = (m_new - m_run) * c > kSlack;
    const float m_use = raise ? m_new : m_run;
    const float mc = (m_use == -INFINITY ? 0.0f : m_use) * c;
    const float alpha = raise ? __builtin_amdgcn_exp2f(m_run * c - mc) : 1.0f;
    m_run = m_use;
    l_run *= alpha;
    if (__any(alpha != 1.0f)) {
#pragma unroll
      for (int db = 0; db < C::kDBlocks; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[db][r] *= alpha;
    }


    // ---- per 16-key chunk: P = exp2(S*c - m*c) in bf16, row sum, O^T += V^T P^T.
    //      Every chunk up to the one holding key vk - 1 is processed, and the
    //      whole second half unless vk <= T/2: keys at or past vk have p = 0
    //      and zeroed V rows, so they add exact zeros.  Software-pipelined: the
    //      exponentials of chunk kc + 1 and the V operand reads of chunk kc + 1
    //      are interleaved with the four MFMAs of chunk kc (one MFMA, then two
    //      LDS reads and up to seven VALU instructions), so that the wave's
    //      VALU work runs under its own MFMAs.  The row sum adds the fp32 p
    //      (v_dot2 on the packed bf16 P would occupy the matrix pipe and stall
    //      behind the MFMAs). -----
    bf16x8_t vop[2][C::kDBlocks];  // operands of chunks kc (vop[kc & 1]) and kc + 1
    // The P.V phase (MFMAs and the exponentials) takes issue priority on the
    // SIMD: two workgroups share each SIMD, and the wave in this phase winning
    // issue pushes the pair towards anti-phase, one wave's softmax and Q.K
    // under the other's P.V.  (Priority for Q.K as well measured slower.)
    __builtin_amdgcn_s_setprio(1);
    read_v(0, vop[0]);
    auto make_p = [&](int kc) {
      const int e0 = 8 * (kc & 1);
      bf16x2_t pp[4];
      float ps[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kc >> 1][e0 + 2 * e], c, -mc));
        const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kc >> 1][e0 + 2 * e + 1], c, -mc));
        pp[e] = to_bf16x2(p0, p1);
        ps[e] = p0 + p1;
      }
      l_run += (ps[0] + ps[1]) + (ps[2] + ps[3]);
      asm volatile("" : "+v"(l_run));  // this chunk's sum is formed here, not in a chain after the tile
      return __builtin_shufflevector(
          __builtin_shufflevector(pp[0], pp[1], 0, 1, 2, 3),
          __builtin_shufflevector(pp[2], pp[3], 0, 1, 2, 3), 0, 1, 2, 3, 4, 5, 6, 7);
    };
    bf16x8_t pk = make_p(0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int kc = 0; kc < 2 * NKB; ++kc) {
      if (kc + 1 < 2 * NKB) read_v(kc + 1, vop[(kc + 1) & 1]);
      bf16x8_t pk_next = pk;
      if (kc + 1 < 2 * NKB) pk_next = make_p(kc + 1);
#pragma unroll
      for (int db = 0; db < C::kDBlocks; ++db)
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop[kc & 1][db], pk, acc[db], 0, 0, 0);
      if (kc + 1 < 2 * NKB) {
#pragma unroll
        for (int g = 0; g < C::kDBlocks; ++g) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // two LDS reads
          __builtin_amdgcn_sched_group_barrier(0x002, 7, 0);  // seven VALU
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      pk = pk_next;
      // A tile whose valid keys all lie in its first half stops here.  (One exit
      // point only: an exit after every chunk made the compiler drain the LDS
      // reads in flight at each one, 2-6 % slower on full tiles.)
      if (kc == NKB - 1 && 16 * (kc + 1) >= vk) break;
    }

    __builtin_amdgcn_s_setprio(0);
    }  // active

    // ---- K of step n2 landed (the only copy in flight); every wave is done with V ----
    if (j2 != -1) wait_vmcnt<0>();
    lds_barrier();
    copy_step(Flag<true>{}, Flag<true>{}, n2, j2, vk2);
  };

  // The segment in chunks of kThreads list entries; within a chunk the steps
  // are pipelined (the copies of the next step overlap the current one).
  for (int base = a; base < end; base += C::kThreads) {
    int total;
    if constexpr (kPairs)
      total = compact_steps<T, C::kWaves>(list, base, end, vbs, nt_list, st, srt, wave_scratch, tid, wave,
                                          lane, sub_shift);
    else
      total = compact_list<T, C::kWaves, 2>(list, base, end, vbs, nt_list, st, wave_scratch, tid, wave, lane,
                                            sub_shift);
    if (total == 0) continue;
    any_keys = true;
    int2 e = st[0];
    const int j0 = __builtin_amdgcn_readfirstlane(e.x);
    int vk = __builtin_amdgcn_readfirstlane(e.y);
    // Q must be in registers before the first tile DMA is issued: the DMAs
    // are invisible to the compiler's wait-count bookkeeping, and an explicit
    // drain here keeps it from placing waits for Q inside the tile loop.
    wait_vmcnt<0>();
    copy_step(Flag<false>{}, Flag<false>{}, 0, j0, vk);
    copy_step(Flag<true>{}, Flag<false>{}, 0, j0, vk);
    // the first step's K has landed (its V may be in flight: at least
    // kDmaPerTile copies, one more when a pair's split block is copied twice)
    wait_vmcnt<C::kDmaPerTile>();
    lds_barrier();
    for (int t = 0; t < total; ++t) {
      int j2 = -1, vk2 = 0;
      if (t + 1 < total) {
        e = st[2 * (t + 1)];
        j2 = __builtin_amdgcn_readfirstlane(e.x);
        vk2 = __builtin_amdgcn_readfirstlane(e.y);
      }
      tile_step(vk, t + 1, j2, vk2);
      vk = vk2;
    }
  }
  wait_vmcnt<0>();  // Q, when no tile was processed

  if (nseg == 1) {  // the whole item: store
    const int64_t ibh = item / num_tiles;
    store_tile_rows<T, D>(acc, m_run, l_run, any_keys, ibh, item - static_cast<int>(ibh) * num_tiles,
                          num_tiles, vbs, sub_shift, wave, lane, c, out, lse, out_lo);
    return;
  }

  // ---- a split item: store this segment's partial (merged by the next launch) ---------
  const int ln = launder(lane);
  float* slot = ws + static_cast<int64_t>(unit2) * S::kFloats;
#pragma unroll
  for (int db = 0; db < C::kDBlocks; ++db)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4)
      *reinterpret_cast<float4*>(slot + (((wave * C::kDBlocks + db) * 4 + r4) * 64 + ln) * 4) =
          make_float4(acc[db][4 * r4], acc[db][4 * r4 + 1], acc[db][4 * r4 + 2],
                      acc[db][4 * r4 + 3]);
  slot[S::kM + wave * 64 + ln] = m_run;
  slot[S::kL + wave * 64 + ln] = l_run;
  if (tid == 0) slot[S::kAny] = any_keys ? 1.0f : 0.0f;
  };

  if constexpr (kPersistent) {
    __shared__ int s_unit;
    int xq = static_cast<int>(blockIdx.x & 7);
    for (;;) {
      const int L = next_unit(queue, total_units, xq, &s_unit);
      if (L < 0) break;
      unit(L);
    }
  } else {
    unit(static_cast<int>(blockIdx.x));
  }
}

// Merge of the split items: one workgroup per (item, 32-column block of the
// output), the same T/32 waves and lane layout as the segments that wrote the
// item's `splits` slots (at most 4).  Every slot's values for the block are
// loaded first; then the partials are combined in segment order with the
// guarded rescaling of the online update (an exponent offset of 0 while the
// running max is -inf), so the result is a fixed function of the slots, and
// the block's rows are stored as for a whole item (the first block's
// workgroup also writes the log-sum-exp).
template <int T, int D>
__global__ __launch_bounds__(2 * T) void bsa_fwd_merge_kernel(
    const float* __restrict__ ws, const int32_t* __restrict__ vbs, uint16_t* __restrict__ out,
    int num_tiles, int n_whole, int splits, float c, float* __restrict__ lse,
    uint16_t* __restrict__ out_lo, int sub_shift) {
  using C = Cfg<T, D>;
  using S = Slot<T, D>;
  constexpr int kMaxSplits = 4;
  const int m = blockIdx.x;
  const int db = blockIdx.y;
  const int item = n_whole + m;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ln = launder(lane);
  float4 xv[kMaxSplits][4];
  float ms[kMaxSplits], ls[kMaxSplits], as[kMaxSplits];
#pragma unroll
  for (int sg = 0; sg < kMaxSplits; ++sg) {
    if (sg >= splits) break;
    const float* slot = ws + (static_cast<int64_t>(m) * splits + sg) * S::kFloats;
    ms[sg] = slot[S::kM + wave * 64 + ln];
    ls[sg] = slot[S::kL + wave * 64 + ln];
    as[sg] = slot[S::kAny];
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4)
      xv[sg][r4] = *reinterpret_cast<const float4*>(
          slot + (((wave * C::kDBlocks + db) * 4 + r4) * 64 + ln) * 4);
  }
  float acc[16];
#pragma unroll
  for (int rr = 0; rr < 16; ++rr) acc[rr] = 0.0f;
  float mm = -INFINITY, l_run = 0.0f;
  bool any_all = false;
#pragma unroll
  for (int sg = 0; sg < kMaxSplits; ++sg) {
    if (sg >= splits) break;
    const float mn = fmaxf(mm, ms[sg]);
    const float mnc = (mn == -INFINITY ? 0.0f : mn) * c;
    const float sa = __builtin_amdgcn_exp2f(mm * c - mnc);
    const float sb = __builtin_amdgcn_exp2f(ms[sg] * c - mnc);
    mm = mn;
    l_run = l_run * sa + ls[sg] * sb;
    any_all = any_all || as[sg] != 0.0f;
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      acc[4 * r4 + 0] = acc[4 * r4 + 0] * sa + xv[sg][r4].x * sb;
      acc[4 * r4 + 1] = acc[4 * r4 + 1] * sa + xv[sg][r4].y * sb;
      acc[4 * r4 + 2] = acc[4 * r4 + 2] * sa + xv[sg][r4].z * sb;
      acc[4 * r4 + 3] = acc[4 * r4 + 3] * sa + xv[sg][r4].w * sb;
    }
  }
  // normalise and store this block's columns of the wave's 32 rows (as store_tile_rows)
  const int64_t ibh = item / num_tiles;
  const int itile = item - static_cast<int>(ibh) * num_tiles;
  const int vq = clampi(vbs[itile >> sub_shift] - T * (itile & ((1 << sub_shift) - 1)), 0, T);
  const int row = wave * 32 + (ln & 31);
  float l_tot;
  {
    float lo_half, hi_half;
    swap_halves(l_run, lo_half, hi_half);
    l_tot = lo_half + hi_half;
  }
  const bool zero_row = !any_all || row >= vq;
  const float inv = l_tot != 0.0f ? 1.0f / l_tot : __builtin_nanf("");
  const int64_t row_id = (ibh * num_tiles + itile) * T + row;
  if (lse != nullptr && db == 0 && ln < 32) {
    const float mc = (mm == -INFINITY ? 0.0f : mm) * c;
    lse[row_id] = zero_row ? -INFINITY : (mc + __builtin_amdgcn_logf(l_tot)) * 0.69314718055994531f;
  }
  const int64_t off = row_id * D + 32 * db + 4 * (ln >> 5);
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    float x[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) x[e] = zero_row ? 0.0f : acc[4 * g + e] * inv;
    const unsigned w0 = __builtin_bit_cast(unsigned, to_bf16x2(x[0], x[1]));
    const unsigned w1 = __builtin_bit_cast(unsigned, to_bf16x2(x[2], x[3]));
    *reinterpret_cast<uint2*>(out + off + 8 * g) = make_uint2(w0, w1);
    if (lse != nullptr) {
      const float r0 = x[0] - __uint_as_float(w0 << 16);
      const float r1 = x[1] - __uint_as_float(w0 & 0xffff0000u);
      const float r2 = x[2] - __uint_as_float(w1 << 16);
      const float r3 = x[3] - __uint_as_float(w1 & 0xffff0000u);
      *reinterpret_cast<uint2*>(out_lo + off + 8 * g) =
          make_uint2(__builtin_bit_cast(unsigned, to_bf16x2(r0, r1)),
                     __builtin_bit_cast(unsigned, to_bf16x2(r2, r3)));
    }
  }
}

template <int T, int D, bool kPersistent>
const void* kernel_of(bool train) {
  return train ? reinterpret_cast<const void*>(&bsa_fwd_kernel<T, D, true, kPersistent>)
               : reinterpret_cast<const void*>(&bsa_fwd_kernel<T, D, false, kPersistent>);
}

template <int T, int D>
hipError_t launch(const bsa::FwdProblem& p, hipStream_t stream) {
  const bool persistent = p.queue != nullptr;
  const void* fn = persistent ? kernel_of<T, D, true>(p.lse != nullptr)
                              : kernel_of<T, D, false>(p.lse != nullptr);
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
  int n_whole = p.n_whole, n_whole_padded = (p.n_whole + 7) / 8 * 8;
  int n_split_units = p.n_split_units, splits = p.splits;
  float* ws = p.ws;
  float cc = c;
  float* lse = p.lse;
  uint16_t* out_lo = p.out_lo;
  int sub_shift = p.sub_shift;
  uint32_t* queue = p.queue;
  int units = n_whole_padded + n_split_units;
  void* args[] = {&q, &k, &v, &idx, &num, &vbs, &out, &nt, &ms, &n_whole, &n_whole_padded,
                  &n_split_units, &splits, &ws, &cc, &lse, &out_lo, &sub_shift, &queue, &units};
  unsigned grid = static_cast<unsigned>(units);
  if (persistent) {
    hipLaunchKernelGGL(clear_queue_kernel, dim3(1), dim3(bsa::kFwdQueueBytes / 4), 0, stream, queue);
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    if (p.grid < units) grid = static_cast<unsigned>(p.grid);
  }
  hipError_t err = hipLaunchKernel(fn, dim3(grid), block, args, 0, stream);
  if (err != hipSuccess || splits <= 1 || n_split_units == 0) return err;
  const void* merge = reinterpret_cast<const void*>(&bsa_fwd_merge_kernel<T, D>);
  const float* wsc = ws;
  void* margs[] = {&wsc, &vbs, &out, &nt, &n_whole, &splits, &cc, &lse, &out_lo, &sub_shift};
  return hipLaunchKernel(merge, dim3(static_cast<unsigned>(n_split_units / splits), Cfg<T, D>::kDBlocks),
                         block, margs, 0, stream);
}

// Work split.  Workgroups run in rounds of `resident` (occupancy x CUs); the
// items that fill whole rounds run whole, and when the leftover items would
// leave the last round less than half full (e.g. 768 items on 512 resident
// workgroups: 256 left over), each leftover item's list is cut into
// s = min(4, resident / leftover) segments, so that the last round is full
// (256 x 2), as long as every segment keeps at least 4 list positions.
// Resident workgroups per CU of bsa_fwd_kernel<T, D, *>: a property of the
// code objects, the same on every gfx950, queried once and kept in an atomic
// (so that later plans, also those made while a stream is being captured into
// a graph, make no runtime call).  The smaller of the two variants' counts, so
// that bsa_fwd and bsa_fwd_lse make the same plan and need the same workspace;
// kPersistent: of the persistent kernels, whose count sizes their grid.
template <int T, int D, bool kPersistent>
hipError_t blocks_per_cu(int* per_cu) {
  static std::atomic<int> cached{0};
  int n = cached.load(std::memory_order_acquire);
  if (n == 0) {
    int a = 0, b = 0;
    hipError_t err = hipOccupancyMaxActiveBlocksPerMultiprocessor(
        &a, kernel_of<T, D, kPersistent>(false), Cfg<T, D>::kThreads, 0);
    if (err != hipSuccess) return err;
    err = hipOccupancyMaxActiveBlocksPerMultiprocessor(
        &b, kernel_of<T, D, kPersistent>(true), Cfg<T, D>::kThreads, 0);
    if (err != hipSuccess) return err;
    n = a < b ? a : b;
    if (n < 1) n = 1;
    cached.store(n, std::memory_order_release);
  }
  *per_cu = n;
  return hipSuccess;
}

template <int T, int D>
hipError_t plan(const bsa::FwdProblem& p, bsa::FwdPlan* plan) {
  int per_cu = 0;
  hipError_t err = blocks_per_cu<T, D, false>(&per_cu);
  if (err != hipSuccess) return err;
  const int64_t resident = static_cast<int64_t>(per_cu) * p.num_cus;
  const int64_t items = p.batch_heads * p.num_tiles;
  const int positions = p.max_sel > 0 ? p.max_sel : 1;
  const int64_t left = items % resident;
  int64_t s = left > 0 && 2 * left <= resident ? resident / left : 1;
  if (s > 4) s = 4;
  while (s > 1 && positions / s < 4) --s;
  plan->splits = static_cast<int32_t>(s);
  plan->n_whole = static_cast<int32_t>(s > 1 ? items - left : items);
  plan->n_split_units = static_cast<int32_t>(s > 1 ? left * s : 0);
  // Persistent launch from four rounds of units on (one round of workgroups
  // taking units from per-XCD queues): measured faster with many rounds of
  // short units of uneven cost (24 rounds: 8-10 %, 6 rounds: 5 %), slower with
  // two or three rounds of long ones (1-2 %).
  const int64_t units = (plan->n_whole + 7) / 8 * 8 + plan->n_split_units;
  plan->persistent = units > 4 * resident ? 1 : 0;
  plan->grid = 0;
  if (plan->persistent) {
    int per_cu_p = 0;
    err = blocks_per_cu<T, D, true>(&per_cu_p);
    if (err != hipSuccess) return err;
    plan->grid = static_cast<int32_t>(static_cast<int64_t>(per_cu_p) * p.num_cus);
  }
  plan->ws_bytes = (plan->persistent ? bsa::kFwdQueueBytes : 0) +
                   static_cast<size_t>(plan->n_split_units) * Slot<T, D>::kFloats * sizeof(float);
  return hipSuccess;
}

}  // namespace

namespace bsa {

hipError_t plan_fwd(const FwdProblem& p, FwdPlan* out) {
  if (p.tile == 128) return p.head_dim == 128 ? plan<128, 128>(p, out) : plan<128, 64>(p, out);
  return p.head_dim == 128 ? plan<64, 128>(p, out) : plan<64, 64>(p, out);
}

hipError_t launch_fwd(const FwdProblem& p, hipStream_t stream) {
  if (p.tile == 128) return p.head_dim == 128 ? launch<128, 128>(p, stream)
                                               : launch<128, 64>(p, stream);
  return p.head_dim == 128 ? launch<64, 128>(p, stream) : launch<64, 64>(p, stream);
}

}  // namespace bsa
