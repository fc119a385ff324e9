// Device helpers shared by the block-sparse attention forward kernels
// (bsa_fwd.hip): vector types, the LDS tile layout and its
// swizzles, LDS DMA, explicit waits and barriers, scalar list reads, and the
// small asm pieces whose compiler-generated forms are wrong or slow.
//
// MFMA register layouts relied on (v_mfma_f32_32x32x16_bf16, wave64):
//   A (32 x 16): lane l holds A[l % 32][8*(l/32) + e], e = 0..7
//   B (16 x 32): lane l holds B[8*(l/32) + e][l % 32]
//   C (32 x 32): lane l, register r holds C[8*(r/4) + 4*(l/32) + r%4][l % 32]
// A and B share the k-mapping, so a permutation of the contraction index
// applied to both is harmless: element e of half h of a 16-key chunk stands
// for key 8*(e/4) + 4*h + e%4, the order in which S^T leaves the keys.
// ds_read_b64_tr_b16: within each 16-lane group, lane i receives element e
// from the 8 bytes addressed by lane 4*e + i/4, at position i%4.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bsa {
namespace detail {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;

constexpr float kLog2e = 1.4426950408889634f;
// Largest rise of the running max, in exp2 units, absorbed without moving the
// exponent offset (p stays below 2^8 = 256).
constexpr float kRescaleSlack = 8.0f;

template <int T, int D>
struct Cfg {
  static constexpr int kWaves = T / 32;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int kChunks = D / 8;                            // 16-byte chunks per row
  static constexpr int kDmaPerTile = T * D * 2 / (kThreads * 16);  // per thread, per tensor
  static constexpr int kKeyBlocks = T / 32;                        // 32-key blocks of S^T
  static constexpr int kKSteps = D / 16;                           // k-steps of Q.K^T
  static constexpr int kDBlocks = D / 32;                          // 32-row blocks of O^T
  static constexpr int kKeyChunks = T / 16;                        // 16-key steps of P.V
};

__device__ __forceinline__ int clampi(int x, int lo, int hi) {
  return x < lo ? lo : (x > hi ? hi : x);
}

// Chunk swizzles (16-byte chunks within a row), for an LDS of 64 banks x 4
// bytes serving 256 bytes per clock.
//  K: a ds_read_b128 serves 16 lanes per clock; they read 16 consecutive rows
//     at one logical chunk, so the 16 rows must land on 16 distinct 16-byte
//     bank groups.  D = 128: a row spans all 64 banks, XOR with row % 16.
//     D = 64: a row spans 32 banks and row parity picks the half, so XOR the
//     8 chunks with (row / 2) % 8.
//  V: a ds_read_b64_tr_b16 serves 32 lanes per clock: two 16-lane groups
//     reading 4 consecutive rows x 4 adjacent logical chunks (32 bytes each
//     group).  XOR with 4 * (row % 4) (D = 128) gives every row its own
//     4-chunk group; for D = 64, rows r and r + 2 share a bank half, so XOR
//     with 4 * ((row / 2) % 2).
template <int D>
__device__ __forceinline__ int swz_k(int row) {
  return D == 128 ? (row & 15) : ((row >> 1) & 7);
}
template <int D>
__device__ __forceinline__ int swz_v(int row) {
  return D == 128 ? 4 * (row & 3) : 4 * ((row >> 1) & 1);
}

// s_waitcnt vmcnt(n) with the other counters left alone (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// Workgroup barrier ordering LDS only (global loads in flight stay in flight).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Byte offset, inside a T x D tile, of the global chunk that lane `lane`
// copies for 1 KiB LDS block `blk`: lane p of the block fills LDS slot p, so
// it fetches the chunk that the swizzle stores there.
template <int D, bool kIsV>
__device__ __forceinline__ uint32_t dma_offset(int blk, int lane) {
  constexpr int kChunks = D / 8;
  const int row = blk * (64 / kChunks) + lane / kChunks;
  const int chunk = (lane % kChunks) ^ (kIsV ? swz_v<D>(row) : swz_k<D>(row));
  return static_cast<uint32_t>((row * D + chunk * 8) * 2);
}

// One LDS DMA instruction: buffer_load_dwordx4 ... lds copies 64 lanes x 16
// bytes from the buffer `srd` at byte offset voff + soff into LDS at
// m0 + 16 * lane.  The buffer descriptor covers one tile, so an offset
// outside it reads zeros instead of faulting.  Issued as asm so that the
// compiler's wait-count pass, which cannot tell this workgroup's K and V
// buffers apart, does not add full drains before unrelated LDS reads; the
// kernel waits explicitly.  M0 is an input operand, so the compiler writes it
// (one s_add per copy) and knows its value; the s_nop is the wait state that
// a write of M0 needs before an LDS DMA.  No memory clobber: the statement is
// volatile, so it keeps its place between the barriers and fences that order
// it, and the index lists stay scalar loads.
__device__ __forceinline__ void dma16(i32x4_t srd, uint32_t voff, uint32_t soff, uint32_t lds_addr) {
  asm volatile(
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %0, %1, %3 offen lds"
      :
      : "v"(voff), "s"(srd), "{m0}"(lds_addr), "s"(soff));
}

__device__ __forceinline__ uint32_t lds_address(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void_t*)p));
}

// Opaque copy of a uniform value: keeps the compiler from precomputing and
// holding every per-block address of every DMA in scalar registers.
__device__ __forceinline__ uint32_t launder_s(uint32_t x) {
  asm volatile("" : "+s"(x));
  return x;
}

// An opaque copy of x: keeps the compiler from hoisting per-iteration
// expressions of x out of the tile loop (which costs registers it does not have).
__device__ __forceinline__ int launder(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

__device__ __forceinline__ float launder_f(float x) {
  asm volatile("" : "+v"(x));
  return x;
}

// A compile-time flag for generic lambdas.
template <bool B>
struct Flag {
  static constexpr bool value = B;
};

// Per-lane byte offsets of a wave's tile copies.  Instruction it of wave w
// fills 1 KiB block blk = it*kWaves + w, whose global offset is the lane
// offset of swizzle phase blk % kPeriod plus (blk - blk % kPeriod) KiB.  Of
// that block term, it*kWaves KiB is the copy's scalar offset; the remainder,
// w - phase KiB, depends only on the phase, and the phases a wave meets repeat
// every kN instructions, so kN (1 or 2) registers hold whole lane offsets.
// Computed once per workgroup.
template <int T, int D, bool kIsV>
struct DmaLane {
  static constexpr int kWaves = Cfg<T, D>::kWaves;
  static constexpr int kPeriod = kIsV ? 1 : (D == 128 ? 4 : 2);
  static constexpr int kGcd = kWaves % kPeriod == 0 ? kPeriod : (kPeriod % kWaves == 0 ? kWaves : 1);
  static constexpr int kN = kPeriod / kGcd;
  uint32_t off[kN];
  __device__ __forceinline__ DmaLane(int wave, int lane) {
#pragma unroll
    for (int i = 0; i < kN; ++i) {
      const int phase = (wave + i * kWaves) % kPeriod;
      off[i] = dma_offset<D, kIsV>(phase, lane) + static_cast<uint32_t>((wave - phase) * 1024);
    }
  }
};

// Copy the first `rows` rows (1 <= rows <= T) of a T x D bf16 tile (rows at
// stride D from `src`) into `lds`, one 1 KiB block per wave instruction
// (kDmaPerTile instructions per wave).  Instruction it of every wave moves
// both its global offset and its LDS offset on by it * kWaves KiB, which is
// the scalar offset of the copy (and added to M0); the rest of each address
// is a lane register of dl.
// Buffer descriptor: base address, stride 0, size of the `rows` rows in
// bytes, and the gfx9 word 3 for raw 32-bit data (data format 4 at bit 15).
// Lanes whose 16 bytes lie past that size fail the range check: they read
// nothing from memory and never fault, so the padding rows of a short tile
// cost no memory traffic.  What such a lane leaves in LDS is not relied on:
// K padding keys are masked by select and V padding rows are zeroed after
// the copy lands.
//
// With kSkipPadding, a wave also skips the instructions whose whole block lies
// past `rows` (a uniform test), so it issues fewer than kDmaPerTile copies:
// only for copies that are waited for with vmcnt(0).
template <int T, int D, bool kIsV, bool kSkipPadding = false>
__device__ __forceinline__ void dma_tile(const uint16_t* __restrict__ src, uint16_t* lds,
                                         int wave, const DmaLane<T, D, kIsV>& dl, int rows = T) {
  using C = Cfg<T, D>;
  using DL = DmaLane<T, D, kIsV>;
  const uint32_t base = launder_s(__builtin_amdgcn_readfirstlane(lds_address(lds)) + wave * 1024);
  const uint64_t g = reinterpret_cast<uintptr_t>(src);
  const i32x4_t srd = {static_cast<int>(static_cast<uint32_t>(g)),
                       static_cast<int>(static_cast<uint32_t>(g >> 32)), rows * D * 2, 0x00020000};
  if (!kSkipPadding || rows >= T) {
#pragma unroll
    for (int it = 0; it < C::kDmaPerTile; ++it) {
      const uint32_t soff = it * C::kWaves * 1024;
      dma16(srd, dl.off[it % DL::kN], soff, base + soff);
    }
  } else {
    constexpr int kRowsPerBlock = 512 / D;  // rows in one 1 KiB block
#pragma unroll
    for (int it = 0; it < C::kDmaPerTile; ++it) {
      if ((it * C::kWaves + wave) * kRowsPerBlock >= rows) break;
      const uint32_t soff = it * C::kWaves * 1024;
      dma16(srd, dl.off[it % DL::kN], soff, base + soff);
    }
  }
}

// The copy of a step that packs two key tiles of va + vb <= T valid rows
// (otherwise as dma_tile): rows [0, va) of the buffer from tile ja and rows
// [va, va + vb) from rows [0, vb) of tile jb, so that the step's valid keys
// are its first va + vb rows and every row after them is padding, as for one
// short tile.
// Two descriptors: tile ja's covering va rows, and one based va rows before
// tile jb covering va + vb rows, so that the usual offsets of buffer rows
// [va, va + vb) land on tile jb's rows [0, vb).  A block wholly before row va
// copies through the first, a block wholly after it through the second; the
// block that holds row va is copied twice, every lane active (EXEC) in exactly
// one of the two instructions, so each writes only its own lanes' LDS slots.
// Every address stays inside tile ja or tile jb.
// Only instructions [kLo, kHi) when given, for a caller that copies a tile in
// parts (as dma_tile_part).
template <int T, int D, bool kIsV, bool kSkipPadding = false, int kLo = 0, int kHi = Cfg<T, D>::kDmaPerTile>
__device__ __forceinline__ void dma_pair(const uint16_t* __restrict__ head, int ja, int va, int jb,
                                         int vb, uint16_t* lds, int wave, int lane,
                                         const DmaLane<T, D, kIsV>& dl) {
  using C = Cfg<T, D>;
  using DL = DmaLane<T, D, kIsV>;
  constexpr int kRowsPerBlock = 512 / D;  // rows in one 1 KiB block
  const uint32_t base = launder_s(__builtin_amdgcn_readfirstlane(lds_address(lds)) + wave * 1024);
  const uint64_t ga = reinterpret_cast<uintptr_t>(head + static_cast<int64_t>(ja) * T * D);
  const uint64_t gb = reinterpret_cast<uintptr_t>(head + static_cast<int64_t>(jb) * T * D) -
                      static_cast<uint64_t>(va) * D * 2;
  const i32x4_t srd_a = {static_cast<int>(static_cast<uint32_t>(ga)),
                         static_cast<int>(static_cast<uint32_t>(ga >> 32)), va * D * 2, 0x00020000};
  const i32x4_t srd_b = {static_cast<int>(static_cast<uint32_t>(gb)),
                         static_cast<int>(static_cast<uint32_t>(gb >> 32)), (va + vb) * D * 2, 0x00020000};
  const int lane_row = launder(lane) / C::kChunks;
#pragma unroll
  for (int it = kLo; it < kHi; ++it) {
    const int row0 = (it * C::kWaves + wave) * kRowsPerBlock;
    if (kSkipPadding && row0 >= va + vb) break;
    const uint32_t soff = it * C::kWaves * 1024;
    const uint32_t off = dl.off[it % DL::kN];
    if (row0 + kRowsPerBlock <= va) {
      dma16(srd_a, off, soff, base + soff);
    } else if (row0 >= va) {
      dma16(srd_b, off, soff, base + soff);
    } else {  // the block holding row va (a uniform test), then split by lane
      if (lane_row < va - row0) dma16(srd_a, off, soff, base + soff);
      if (lane_row >= va - row0) dma16(srd_b, off, soff, base + soff);
    }
  }
}

// Zero the slots of padding rows (row >= vk) that this lane's own DMA wrote.
// Slot p = 64*blk + lane holds row (64*blk + lane) / kChunks: a per-lane row
// plus a uniform one, and a per-lane address plus an immediate offset.
template <int T, int D>
__device__ __forceinline__ void zero_padding_rows(uint16_t* lds, int vk, int wave, int lane) {
  using C = Cfg<T, D>;
  constexpr int kRowsPerBlock = 64 / C::kChunks;
  const int lane_row = launder(lane) / C::kChunks;
  uint4* slot = reinterpret_cast<uint4*>(lds) + lane;
#pragma unroll
  for (int it = 0; it < C::kDmaPerTile; ++it) {
    const int blk = it * C::kWaves + wave;
    if (vk < (blk + 1) * kRowsPerBlock && lane_row >= vk - blk * kRowsPerBlock)  // uniform test first
      slot[blk * 64] = make_uint4(0u, 0u, 0u, 0u);
  }
}

// Copies the usable entries of list[base, min(base + 64*NW, count)) -- in
// range and with at least one valid key -- into tl[] in list order, with
// their valid lengths (clamped); returns how many there are (uniform).
// With sub_shift = 1 the list names tiles of 2T rows (lengths up to 2T), and
// each entry becomes its non-empty T-row halves (tile 2j + t, t = 0, 1), in
// order: tl[] then holds up to 2 * 64 * NW entries.  One list entry per thread
// of an NW-wave workgroup; the order is kept by wave-level prefix counts
// (mbcnt) plus per-wave offsets.  Entry n is written to tl[kStride * n].
// Three barriers.
template <int T, int NW, int kStride = 1>
__device__ __forceinline__ int compact_list(const int32_t* __restrict__ list, int base, int count,
                                            const int32_t* __restrict__ vbs, int num_tiles,
                                            int2* tl, int* wave_count, int tid, int wave,
                                            int lane, int sub_shift = 0) {
  const int e = base + tid;
  int jj = -1, len = 0;
  if (e < count) {
    jj = list[e];
    if (jj >= 0 && jj < num_tiles) len = clampi(vbs[jj], 0, T << sub_shift);
  }
  const int parts = (len + T - 1) / T;  // non-empty T-row parts, a prefix of the tile
  const uint64_t m1 = __ballot(parts >= 1);
  const uint64_t m2 = __ballot(parts >= 2);
  lds_barrier();  // the previous chunk's readers of tl[] and wave_count[] are done
  if (lane == 0) wave_count[wave] = __popcll(m1) + __popcll(m2);
  lds_barrier();
  int off = 0, total = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const int cw = wave_count[w];
    off += w < wave ? cw : 0;
    total += cw;
  }
  auto below = [&](uint64_t m) {
    return __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(m >> 32),
                                     __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m), 0));
  };
  const int pos = below(m1) + below(m2);
  for (int t = 0; t < parts; ++t)
    tl[kStride * (off + pos + t)] = make_int2((jj << sub_shift) + t, len - T * t < T ? len - T * t : T);
  lds_barrier();
  return __builtin_amdgcn_readfirstlane(total);
}

// The steps of a tile loop (the forward's; the dQ and dK/dV kernels' too) for
// list[base, min(base + 64*NW, count)): the usable entries (index in range, at
// least one valid key) cut into T-row parts as compact_list does.  Step n is
// the int2 st[2n] = (j, vk): one part, tile j >= 0 with vk valid rows, or a
// pair, j = -2 - ja and vk = va + vb, with st[2n + 1] = (jb, va).  When no two
// parts fit in T rows together, every part is a step of its own, in list order.
// Otherwise the steps hold as many pairs as possible: with the parts sorted by
// length (ties in list order), k pairs exist exactly when the 2k shortest,
// paired first with 2k-th, second with (2k-1)-th and so on, all fit, so k is
// the largest such count (a binary search, one ballot and one barrier per
// probe); pair i is parts i and 2k-1-i of that order and the other parts follow
// one per step.  srt holds the sorted parts; scratch holds 5 * NW ints.
// Returns the number of steps (uniform).
template <int T, int NW>
__device__ __forceinline__ int compact_steps(const int32_t* __restrict__ list, int base, int count,
                                             const int32_t* __restrict__ vbs, int num_tiles,
                                             int2* st, int2* srt, int* scratch, int tid, int wave,
                                             int lane, int sub_shift) {
  constexpr int kBig = 1 << 20;
  const int e = base + tid;
  int jj = -1, len = 0;
  if (e < count) {
    jj = list[e];
    if (jj >= 0 && jj < num_tiles) len = clampi(vbs[jj], 0, T << sub_shift);
  }
  const int parts = (len + T - 1) / T;  // non-empty T-row parts, a prefix of the tile
  const int len0 = len < T ? len : T, len1 = len - T;
  const uint64_t m1 = __ballot(parts >= 1);
  const uint64_t m2 = __ballot(parts >= 2);
  // the two shortest parts of the wave (len1 <= len0 when both exist)
  int lo = parts >= 2 ? len1 : (parts >= 1 ? len0 : kBig);
  int hi = parts >= 2 ? len0 : kBig;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const int lo2 = __shfl_xor(lo, o), hi2 = __shfl_xor(hi, o);
    const int a = lo < lo2 ? lo2 : lo, b = hi < hi2 ? hi : hi2;
    hi = a < b ? a : b;
    lo = lo < lo2 ? lo : lo2;
  }
  int* const wave_count = scratch;  // [NW] parts, [NW, 3NW) shortest two, [3NW, 5NW) flags
  lds_barrier();  // the previous chunk's readers of st[], srt[] and scratch[] are done
  if (lane == 0) {
    wave_count[wave] = __popcll(m1) + __popcll(m2);
    scratch[NW + 2 * wave] = lo;
    scratch[NW + 2 * wave + 1] = hi;
  }
  lds_barrier();
  int off = 0, total = 0, glo = kBig, ghi = kBig;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const int cw = wave_count[w];
    off += w < wave ? cw : 0;
    total += cw;
    const int lo2 = scratch[NW + 2 * w], hi2 = scratch[NW + 2 * w + 1];
    const int a = glo < lo2 ? lo2 : glo, b = ghi < hi2 ? ghi : hi2;
    ghi = a < b ? a : b;
    glo = glo < lo2 ? glo : lo2;
  }
  auto below = [&](uint64_t m) {
    return __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(m >> 32),
                                     __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m), 0));
  };
  const int pos = off + below(m1) + below(m2);
  const int tile0 = jj << sub_shift;
  total = __builtin_amdgcn_readfirstlane(total);
  if (__builtin_amdgcn_readfirstlane(glo + ghi) > T) {  // no pair fits: list order
    if (parts >= 1) st[2 * pos] = make_int2(tile0, len0);
    if (parts >= 2) st[2 * pos + 2] = make_int2(tile0 + 1, len1);
    lds_barrier();
    return total;
  }
  // the parts in list order, then each part's rank by (length, list position)
  if (parts >= 1) st[pos] = make_int2(tile0, len0);
  if (parts >= 2) st[pos + 1] = make_int2(tile0 + 1, len1);
  lds_barrier();
  int r0 = 0, r1 = 0;
  if (parts >= 1) {
    for (int q = 0; q < total; ++q) {
      const int lq = st[q].y;
      r0 += lq < len0 || (lq == len0 && q < pos);
      r1 += lq < len1 || (lq == len1 && q < pos + 1);
    }
    srt[r0] = make_int2(tile0, len0);
    if (parts >= 2) srt[r1] = make_int2(tile0 + 1, len1);
  }
  lds_barrier();
  // k: the most nested pairs of the 2k shortest that fit (at least one does)
  int klo = 1, khi = total >> 1, it = 0;
  while (klo < khi) {  // uniform
    const int mid = (klo + khi + 1) >> 1;
    const bool bad = tid < mid && srt[tid].y + srt[2 * mid - 1 - tid].y > T;
    const uint64_t mb = __ballot(bad);
    int* const flags = scratch + 3 * NW + (it & 1) * NW;
    if (lane == 0) flags[wave] = mb != 0;
    lds_barrier();
    int any = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) any |= flags[w];
    if (__builtin_amdgcn_readfirstlane(any))
      khi = mid - 1;
    else
      klo = mid;
    ++it;
  }
  const int k = klo;
  // pair r (r < k) is written by its shorter part, which reads its partner
  auto place = [&](int r, int tile, int l) {
    if (r < k) {
      const int2 big = srt[2 * k - 1 - r];
      st[2 * r] = make_int2(-2 - big.x, big.y + l);
      st[2 * r + 1] = make_int2(tile, big.y);
    } else if (r >= 2 * k) {
      st[2 * (r - k)] = make_int2(tile, l);
    }
  };
  if (parts >= 1) place(r0, tile0, len0);
  if (parts >= 2) place(r1, tile0 + 1, len1);
  lds_barrier();
  return total - k;
}

// max(m, a, b), ignoring quiet NaNs.  Written as asm because the compiler
// wraps fmaxf on values it cannot prove canonical (such as MFMA results) in
// extra canonicalising moves.  The compiler does not insert the wait states an
// MFMA result needs before a VALU read when that read is inline asm, so the
// first read of each MFMA output block (kFirst) carries them itself: 21 wait
// states, more than the 32x32x16 MFMA requires.  The statements are volatile,
// so they stay in program order and the later reads of a block follow it.
template <bool kFirst>
__device__ __forceinline__ float max3(float m, float a, float b) {
  float r;
  if (kFirst)
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 4\n\tv_max3_f32 %0, %1, %2, %3"
                 : "=v"(r) : "v"(m), "v"(a), "v"(b));
  else
    asm volatile("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(m), "v"(a), "v"(b));
  return r;
}

// Exchange a value between the two half-waves: afterwards (a, b) hold the
// values of lanes (l & 31, (l & 31) + 32) in every lane l.  Written as asm:
// the v_permlane32_swap builtin called with the same value in both operands
// is folded as if its two results were equal.
__device__ __forceinline__ void swap_halves(float x, float& a, float& b) {
  a = x;
  b = x;
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
}

__device__ __forceinline__ bf16x2_t to_bf16x2(float a, float b) {
  return __builtin_convertvector((f32x2_t){a, b}, bf16x2_t);  // round to nearest even
}

}  // namespace detail
}  // namespace bsa
