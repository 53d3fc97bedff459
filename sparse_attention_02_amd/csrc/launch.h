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
  float* scores;         // [B, Lq, Lk]
  int B, Lq, Lk, q_start, HI, dI;
  int n_qtiles, n_splits;  // filled by the launcher
};

struct TopkArgs {
  const float* scores;  // [B, Lq, Lk]
  int32_t* indices;     // [B, Lq, k]
  void* workspace;      // topk_workspace_bytes() bytes, or null when that is 0
  int B, Lq, Lk, q_start, k;
  // filled by the launcher for the two-stage path
  int nseg;
  uint32_t* cand_key;   // [B*Lq, nseg, k]
  int32_t* cand_idx;    // [B*Lq, nseg, k]
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
  // workspace: dZ in operand order, P and dZ key-major ([B*Lq, kpad, 128] bf16)
  uint16_t* ws_dzf;
  uint16_t* ws_pk;
  uint16_t* ws_dzk;
  int B, Lq, Lk, H, Dv, Dr, k;
  float scale;              // softmax_scale
  float scale_log2;         // softmax_scale * log2(e)
};

// Launch `kernel(arg)` and return the launch's own status (not the thread's
// sticky last-error state, which other libraries in the process also write).
template <typename Arg>
inline hipError_t launch_kernel(const void* kernel, dim3 grid, dim3 block, size_t smem,
                                hipStream_t stream, const Arg& arg) {
  void* args[] = {const_cast<Arg*>(&arg)};
  return hipLaunchKernel(kernel, grid, block, args, smem, stream);
}

hipError_t launch_index_scores(const IndexArgs& a, hipStream_t stream);
hipError_t launch_topk(const TopkArgs& a, hipStream_t stream);
size_t topk_workspace_bytes(int B, int Lq, int q_start, int Lk, int k);
hipError_t launch_sparse_mla_attn(const AttnArgs& a, hipStream_t stream);
// Masked mode for short prefill: dense over the causal range, masked to the
// selection (no split: nsplit must be 1).
hipError_t launch_masked_mha_attn(const AttnArgs& a, hipStream_t stream);
// Parts per row when few rows would leave most CUs idle (1: no split), and the
// workspace the split needs.
int attn_splits(int rows, int k);
hipError_t launch_sparse_mla_attn_bwd(const AttnBwdArgs& a, hipStream_t stream);
size_t attn_bwd_workspace_bytes(int rows, int k);
size_t attn_workspace_bytes(int rows, int k, int H, int Dv);

}  // namespace dsa
