// Internal launch interface between the C ABI (dsa_api.cpp) and the kernels.
// Arguments here are already validated; the launchers only pick a launch shape.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dsa {

struct IndexArgs {
  const uint8_t* q_idx;  // [B, Lq, HI, dI] e4m3fn
  const uint8_t* k_idx;  // [B, Lk, dI]     e4m3fn
  const float* w;        // [B, Lq, HI]
  float* scores;         // [B, Lq, out_ld] (unless filtering, below)
  int B, Lq, Lk, q_start, HI, dI;
  int n_qtiles, n_splits;  // filled by the launcher
  // Key sampling: the kernel scores the keys s = key_stride * s' (s' = 0,
  // 1, ...) and writes score s' of a row at scores[row * out_ld + s'].
  // Plain scoring: key_stride 1, out_ld Lk.
  int key_stride, out_ld;
  // Filtering (thresh non-null): no scores are written.  The keys of row r
  // whose order key is >= thresh[r] are written, in ascending index order, as
  // (max(key, 1), index) to the cap_s slots of (row r, split) in
  // cand_key / cand_idx ([B*Lq, n_splits, cap_s]); unused slots get (0, -1)
  // and row_count[r * n_splits + split] the number found (possibly > cap_s).
  // The prefill shape only (q_len >= 8).
  const uint32_t* thresh;
  uint32_t* cand_key;
  int32_t* cand_idx;
  int32_t* row_count;
  int cap_s;
  // Row subset (non-null): only query tiles holding a row r with
  // only_rows[r] != 0 are scored.
  const int32_t* only_rows;
};

struct TopkArgs {
  const float* scores;  // [B, Lq, Lk]
  int32_t* indices;     // [B, Lq, k]
  void* workspace;      // topk_workspace_bytes() bytes, or null when that is 0
  int B, Lq, Lk, q_start, k;
  // filled by the launcher for the two-stage path
  int nseg;
  uint32_t* cand_key;   // [B*Lq, nseg, seg_cap]
  int32_t* cand_idx;    // [B*Lq, nseg, seg_cap]
  int seg_cap;          // candidate slots per segment (k for the two-stage path)
  // Row subset (non-null): rows r with only_rows[r] == 0 are left untouched.
  const int32_t* only_rows;
};

// Selection fused with the indexer for long rows (topk.hip + indexer.hip):
// sizes of its buffers, decided from the problem alone.
struct FusedPlan {
  bool use;          // the fused path applies
  int stride;        // key sampling stride S
  int ls;            // sampled keys per row: ceil(longest row / S), <= 32768
  int n_splits;      // key-range splits of the filtering indexer
  int cap_s;         // candidate slots per (row, split)
};

struct AttnArgs {
  const uint16_t* q;        // [B, Lq, H, Dqk] bf16
  const uint16_t* kv;       // [B, Lk, Dqk]    bf16
  const int32_t* indices;   // [B, Lq, k]
  float* out;               // [B, Lq, H, Dv]
  float* lse;               // [B, Lq, H] or null
  int B, Lq, Lk, H, Dv, Dr, k;
  int q_start;              // position of query row 0 (masked mode)
  float scale_log2;         // softmax_scale * log2(e)
  // split over the selected chunks (nsplit > 1): block (row, part) writes the
  // attention over its share of the chunks, normalised, with its lse, to
  // part_out [B*Lq, nsplit, H, Dv] and part_lse [B*Lq, nsplit, H]
  int nsplit;
  float* part_out;
  float* part_lse;
};

// Backward of the sparse attention over fixed indices.
struct AttnBwdArgs {
  const uint16_t* q;        // [B, Lq, H, Dqk] bf16
  const uint16_t* kv;       // [B, Lk, Dqk]    bf16
  const int32_t* indices;   // [B, Lq, k]
  const float* out;         // [B, Lq, H, Dv]  forward output
  const float* lse;         // [B, Lq, H]      forward log-sum-exp (natural log)
  const float* dout;        // [B, Lq, H, Dv]  upstream gradient
  float* dq;                // [B, Lq, H, Dqk] written
  float* dkv;               // [B, Lk, Dqk]    accumulated into
  // workspace parts, set by launch_sparse_mla_attn_bwd from one buffer:
  // dZ in operand order, P and scale * dZ key-major ([B*Lq, kpad, 128] bf16),
  // partial dkv rows per (row, slot) ([B*Lq, kpad, Dqk] bf16), the (row, slot)
  // lists of every key with their counts and offsets, scan block sums
  uint16_t* ws_pk;
  uint16_t* ws_dzk;
  uint16_t* ws_part;
  int32_t* ws_list;
  int32_t* ws_cnt;
  int32_t* ws_off;
  int32_t* ws_cur;
  int32_t* ws_bsum;
  int B, Lq, Lk, H, Dv, Dr, k;
  float scale;              // softmax_scale
  float scale_log2;         // softmax_scale * log2(e)
};

// Dense warm-up objective of the indexer.
struct WarmupArgs {
  const uint16_t* q;       // [B, Lq, H, Dqk] bf16
  const uint16_t* kv;      // [B, Lk, Dqk]    bf16
  float* target;           // [B, Lq, Lk]     written for s <= pos(t)
  const float* scores;     // [B, Lq, Lk]     indexer scores (KL kernel)
  float* loss;             // [B, Lq]
  float* dscores;          // [B, Lq, Lk]     written for s <= pos(t); may be `scores`
  const float* lse_in;     // [B, Lq, H]      natural-log lse given by the caller, or null
  float* lse_out;          // [B, Lq, H]      the computed lse (when lse_in is null), or null
  int B, Lq, Lk, q_start, H, Dv, Dr;
  float scale_log2;        // softmax_scale * log2(e)
  float inv_heads;         // 1 / H
};

// Gradients of the indexer scores with respect to q_I, w and k_I.
struct IndexBwdArgs {
  const uint8_t* q_idx;    // [B, Lq, H_I, d_I] e4m3fn
  const uint8_t* k_idx;    // [B, Lk, d_I]      e4m3fn
  const float* w;          // [B, Lq, H_I]
  const float* dscores;    // [B, Lq, Lk]       read for s <= pos(t)
  float* dq_idx;           // [B, Lq, H_I, d_I] written
  float* dw;               // [B, Lq, H_I]      written
  float* dk_idx;           // [B, Lk, d_I]      accumulated into
  int B, Lq, Lk, q_start, H, DI;
};

// Launch `kernel(args...)` and return the launch's own status (not the
// thread's sticky last-error state, which other libraries in the process also
// write).  The argument types must match the kernel's parameters exactly.
template <typename... Args>
inline hipError_t launch_kernel(const void* kernel, dim3 grid, dim3 block, size_t smem,
                                hipStream_t stream, const Args&... args) {
  void* ptrs[] = {const_cast<Args*>(&args)...};
  return hipLaunchKernel(kernel, grid, block, ptrs, smem, stream);
}

hipError_t launch_index_scores(const IndexArgs& a, hipStream_t stream);
// Key-range splits launch_index_scores would use for `a` (any key_stride).
int index_splits(const IndexArgs& a);
FusedPlan fused_plan(int B, int Lq, int Lk, int q_start, int HI, int dI, int k);
// Per-row thresholds of the fused selection from the sampled scores
// [B*Lq, ls]: an order key t such that, judging from the sample, a little
// more than k of the row's keys are >= t.
hipError_t launch_fused_threshold(const float* sample, uint32_t* thresh, int B, int Lq, int Lk, int q_start,
                                  int k, int stride, int ls, hipStream_t stream);
// Exact top-k of each row from the filtering indexer's candidate slots;
// rows whose candidates cannot be trusted (a split overflowed its slots, or
// fewer than k were found) get flags[r] = 1 and are left for the plain path.
hipError_t launch_fused_select(const TopkArgs& a, const int32_t* row_count, int32_t* flags, hipStream_t stream);
hipError_t launch_topk(const TopkArgs& a, hipStream_t stream);
size_t topk_workspace_bytes(int B, int Lq, int q_start, int Lk, int k);
hipError_t launch_sparse_mla_attn(const AttnArgs& a, hipStream_t stream);
// Masked mode for short prefill: dense over the causal range, masked to the
// selection (no split: nsplit must be 1).
hipError_t launch_masked_mha_attn(const AttnArgs& a, hipStream_t stream);
// Parts per row when few rows would leave most CUs idle (1: no split), and the
// workspace the split needs.
int attn_splits(int rows, int k);
// `workspace` holds attn_bwd_workspace_bytes(B, Lq, Lk, k, Dv + Dr) bytes,
// 256-byte aligned; the ws_* members of `a` are ignored and set from it.
hipError_t launch_sparse_mla_attn_bwd(const AttnBwdArgs& a, void* workspace, hipStream_t stream);
size_t attn_bwd_workspace_bytes(int B, int Lq, int Lk, int k, int dqk);
size_t attn_workspace_bytes(int rows, int k, int H, int Dv);
hipError_t launch_warmup_target(const WarmupArgs& a, hipStream_t stream);
hipError_t launch_warmup_kl(const WarmupArgs& a, hipStream_t stream);
hipError_t launch_index_scores_bwd(const IndexBwdArgs& a, hipStream_t stream);

}  // namespace dsa
