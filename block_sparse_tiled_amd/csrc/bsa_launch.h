// Internal interface between the C-ABI entry points (bsa_api.hip) and the
// kernel translation units.  Arguments have been validated by the caller;
// every launcher returns the hipError_t of its launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bsa {

struct FwdProblem {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const int32_t* q2k_idx;  // may be null when max_sel == 0
  const int32_t* q2k_num;
  const int32_t* block_sizes;
  uint16_t* out;
  int64_t batch_heads;
  int32_t num_tiles;
  int32_t max_sel;
  int32_t tile;
  int32_t head_dim;
  int32_t num_cus;  // compute units of the device, for the work mapping
  // set from FwdPlan by the caller before launch_fwd:
  int32_t n_whole;        // items [0, n_whole) run whole
  int32_t n_split_units;  // the other items, `splits` list segments each
  int32_t splits;
  float* ws;              // n_split_units partial slots (when splits > 1)
  uint32_t* queue;        // per-XCD work-queue counters: persistent launch; null: one unit per workgroup
  int32_t grid;           // workgroups of a persistent launch
  float* lse;             // [B, H, NT*T] log-sum-exp per row, or null
  uint16_t* out_lo;       // [B, H, NT*T, D] bf16 rounding residual of out (with lse)
  int32_t sub_shift;      // 1: the lists and lengths count tiles of 2*tile rows
};

// How the items are cut into work units, and the workspace that needs (none
// when no item is split).
// Bytes of per-XCD work-queue counters at the front of a persistent launch's
// workspace (8 counters, 64 bytes apart).
constexpr size_t kFwdQueueBytes = 512;

struct FwdPlan {
  int32_t n_whole;
  int32_t n_split_units;
  int32_t splits;
  int32_t persistent;  // one round of workgroups taking units from per-XCD queues
  int32_t grid;        // its workgroups
  size_t ws_bytes;     // queue counters (persistent), then the split partials
};

hipError_t plan_fwd(const FwdProblem& p, FwdPlan* plan);
// One launch, or two when items are split (the segments, then their merge).
hipError_t launch_fwd(const FwdProblem& p, hipStream_t stream);

struct LayoutProblem {
  const void* src[4];
  void* dst[4];
  int32_t n_tensors;
  const int32_t* tile_src_token;
  int64_t batch;
  int64_t tokens;
  int64_t heads;
  int64_t rows_per_head;  // num_tiles * tile
  int32_t head_dim;
  // the layout with pooling only (launch_tile_layout_pool)
  int32_t tile = 0;
  const int32_t* block_sizes = nullptr;  // [num_tiles]
  float* pooled = nullptr;               // [3, B*H*num_tiles, head_dim]
};

hipError_t launch_tile_layout(const LayoutProblem& p, hipStream_t stream);
hipError_t launch_tile_layout_pool(const LayoutProblem& p, hipStream_t stream);

// Transposed lists for the backward: for each key tile, the query tiles whose
// lists name it (ascending; a tile listed twice appears twice).
struct K2qProblem {
  const int32_t* q2k_idx;  // may be null when max_sel == 0
  const int32_t* q2k_num;
  int32_t* k2q_idx;        // [B, H, NT, max_k]
  int32_t* k2q_num;        // [B, H, NT], the true counts
  int64_t batch_heads;
  int32_t num_tiles;
  int32_t max_sel;
  int32_t max_k;
};

hipError_t launch_k2q(const K2qProblem& p, hipStream_t stream);

struct BwdProblem {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* out;
  const uint16_t* out_lo;  // bf16 rounding residual of out
  const uint16_t* dout;
  const float* lse;
  const int32_t* q2k_idx;
  const int32_t* q2k_num;
  const int32_t* k2q_idx;
  const int32_t* k2q_num;
  const int32_t* block_sizes;
  uint16_t* dq;
  uint16_t* dk;
  uint16_t* dv;
  float* delta;  // [B, H, NT*T] workspace
  int64_t batch_heads;
  int32_t num_tiles;
  int32_t max_sel;
  int32_t max_k;
  int32_t tile;
  int32_t head_dim;
  int32_t sub_shift;  // 1: the lists and lengths count tiles of 2*tile rows
};

hipError_t launch_bwd(const BwdProblem& p, hipStream_t stream);

// The coarse stage: tile selection and the coarse output.
struct CoarseProblem {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const int32_t* block_sizes;
  int32_t* q2k_idx;   // [B, H, NT, max_sel]
  int32_t* q2k_num;   // [B, H, NT]
  float* coarse_out;  // [B, H, NT, D], or null
  float* ws;          // coarse_workspace_bytes(), or the logits only when pooled is given
  const float* pooled = nullptr;  // [3, B*H*NT, D] pooled Q, K, V already formed, or null
  int64_t batch_heads;
  int32_t num_tiles;
  int32_t tile;
  int32_t head_dim;
  int32_t topk;
  int32_t max_sel;
};

size_t coarse_workspace_bytes(int64_t batch_heads, int64_t num_tiles, int32_t head_dim);
hipError_t launch_coarse(const CoarseProblem& p, hipStream_t stream);

// The combine and the inverse gather in one pass (bsa_tile_unlayout_combine).
struct UnlayoutCombineProblem {
  const uint16_t* out;          // [B, H, NT*T, D] fine output (read only)
  const uint16_t* gate;         // [B, H, NT*T, D]
  const float* coarse_out;      // [B, H, NT, D]
  const int32_t* block_sizes;   // [NT]
  const int32_t* token_row;     // [tokens]
  uint16_t* dst;                // [B, tokens, H, D]
  int64_t batch;
  int64_t tokens;
  int64_t heads;
  int32_t num_tiles;
  int32_t tile;
  int32_t head_dim;
};

hipError_t launch_unlayout_combine(const UnlayoutCombineProblem& p, hipStream_t stream);

struct CombineProblem {
  uint16_t* out;           // [B, H, NT*T, D], updated in place
  const uint16_t* gate;    // [B, H, NT*T, D]
  const float* coarse_out; // [B, H, NT, D]
  const int32_t* block_sizes;
  int32_t num_tiles;
  int32_t tile;
  int32_t head_dim;
  int64_t rows;  // B*H*NT*T
};

hipError_t launch_coarse_combine(const CombineProblem& p, hipStream_t stream);

// The inverse gather: p.src are tile buffers, p.dst token-major outputs, and
// p.tile_src_token holds the tile row of every token (token_row).
hipError_t launch_tile_unlayout(const LayoutProblem& p, hipStream_t stream);

}  // namespace bsa
