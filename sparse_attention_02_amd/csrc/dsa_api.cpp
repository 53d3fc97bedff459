// C ABI of libdsa.so: argument checks, workspace layout and kernel launches.
// The entry points and their contracts are declared in include/dsa.h.
#include "dsa.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <climits>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "launch.h"

namespace {

thread_local char g_last_error[512] = "";

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
  va_end(ap);
  return status;
}

constexpr size_t kAlign = 256;
constexpr int kMaskedMaxKv = 65536;  // masked attention: longest causal range (LDS bitmap)
size_t round_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned(const void* ptr, size_t a) { return ((uintptr_t)ptr % a) == 0; }

int check_common(const dsa_problem* p) {
  if (!p) return fail(DSA_ERR_NULL, "problem is NULL");
  if (p->batch < 1 || p->q_len < 1 || p->kv_len < 1 || p->q_start < 0)
    return fail(DSA_ERR_SHAPE, "batch, q_len, kv_len must be >= 1 and q_start >= 0 (got %d, %d, %d, %d)",
                p->batch, p->q_len, p->kv_len, p->q_start);
  if ((long long)p->q_start + p->q_len > p->kv_len)
    return fail(DSA_ERR_SHAPE, "q_start + q_len (%lld) exceeds kv_len (%d)",
                (long long)p->q_start + p->q_len, p->kv_len);
  if ((long long)p->batch * p->q_len > 0x7FFFFFFFLL)
    return fail(DSA_ERR_UNSUPPORTED, "batch * q_len exceeds 2^31 - 1");
  return DSA_OK;
}

int check_index(const dsa_problem* p) {
  if (p->idx_heads < 1 || p->idx_dim < 1)
    return fail(DSA_ERR_SHAPE, "idx_heads and idx_dim must be >= 1");
  if (p->idx_heads > 64) return fail(DSA_ERR_UNSUPPORTED, "idx_heads %d > 64", p->idx_heads);
  if (p->idx_dim % 32 != 0 || p->idx_dim > 128)
    return fail(DSA_ERR_UNSUPPORTED, "idx_dim %d: supported 32, 64, 96, 128", p->idx_dim);
  return DSA_OK;
}

int check_topk(const dsa_problem* p) {
  if (p->topk < 1) return fail(DSA_ERR_SHAPE, "topk must be >= 1");
  if (p->topk > 2048) return fail(DSA_ERR_UNSUPPORTED, "topk %d > 2048", p->topk);
  return DSA_OK;
}

// heads, latent shape and scale of the main attention (no top-k)
int check_latent(const dsa_problem* p) {
  if (p->heads < 1 || p->d_latent < 1 || p->d_rope < 0)
    return fail(DSA_ERR_SHAPE, "heads, d_latent must be >= 1 and d_rope >= 0");
  if (!(std::isfinite(p->softmax_scale) && p->softmax_scale > 0.0f))
    return fail(DSA_ERR_SHAPE, "softmax_scale must be finite and > 0");
  if (p->heads > 128) return fail(DSA_ERR_UNSUPPORTED, "heads %d > 128", p->heads);
  const bool mla = p->d_latent == 512 && p->d_rope == 64;
  const bool tiny = p->d_latent == 64 && p->d_rope == 16;
  if (!mla && !tiny)
    return fail(DSA_ERR_UNSUPPORTED, "latent shape %d + %d: supported 512 + 64 and 64 + 16",
                p->d_latent, p->d_rope);
  // the latent gather addresses one sequence's cache with 32-bit byte offsets
  // (plus a few KiB of bias) and multiplies row indices in 24 bits
  if ((long long)p->kv_len * (p->d_latent + p->d_rope) * 2 > (1LL << 32) - 8192 ||
      p->kv_len > (1 << 24))
    return fail(DSA_ERR_UNSUPPORTED,
                "kv_len %d: the latent gather needs kv_len <= 2^24 and one sequence's cache "
                "below 4 GiB - 8 KiB", p->kv_len);
  return DSA_OK;
}

int check_attn(const dsa_problem* p) {
  if (int s = check_topk(p)) return s;
  return check_latent(p);
}

// The backward's key lists name a (row, slot) pair as row * kpad + slot and
// count entries per key in 32-bit integers.
int check_bwd_size(const dsa_problem* p) {
  const long long kpad = (p->topk + 31) / 32 * 32;
  if ((long long)p->batch * p->q_len * kpad > INT32_MAX || (long long)p->batch * p->kv_len > INT32_MAX)
    return fail(DSA_ERR_UNSUPPORTED,
                "sparse_mla_attn_bwd: batch*q_len*topk (topk rounded up to 32) and batch*kv_len must "
                "stay below 2^31");
  return DSA_OK;
}

size_t bwd_ws_bytes(const dsa_problem* p) {
  return dsa::attn_bwd_workspace_bytes(p->batch, p->q_len, p->kv_len, p->topk, p->d_latent + p->d_rope);
}

int check_ptr(const void* ptr, const char* name, size_t align) {
  if (!ptr) return fail(DSA_ERR_NULL, "%s is NULL", name);
  if (!aligned(ptr, align)) return fail(DSA_ERR_ALIGN, "%s is not %zu-byte aligned", name, align);
  return DSA_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return DSA_OK;
  return fail(DSA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

size_t scores_bytes(const dsa_problem* p) {
  return (size_t)p->batch * p->q_len * p->kv_len * sizeof(float);
}
size_t indices_bytes(const dsa_problem* p) {
  return (size_t)p->batch * p->q_len * p->topk * sizeof(int32_t);
}

dsa::IndexArgs index_args(const dsa_problem* p, const uint8_t* q_idx, const uint8_t* k_idx,
                          const float* w, float* scores) {
  dsa::IndexArgs a{};
  a.q_idx = q_idx; a.k_idx = k_idx; a.w = w; a.scores = scores;
  a.B = p->batch; a.Lq = p->q_len; a.Lk = p->kv_len; a.q_start = p->q_start;
  a.HI = p->idx_heads; a.dI = p->idx_dim;
  a.key_stride = 1;
  a.out_ld = p->kv_len;
  return a;
}

dsa::TopkArgs topk_args(const dsa_problem* p, const float* scores, int32_t* indices, void* ws) {
  dsa::TopkArgs a{};
  a.scores = scores; a.indices = indices; a.workspace = ws;
  a.B = p->batch; a.Lq = p->q_len; a.Lk = p->kv_len; a.q_start = p->q_start; a.k = p->topk;
  a.seg_cap = p->topk;
  return a;
}

// Workspace of dsa_index_topk: the plain path's score matrix and top-k
// scratch (also the fused path's fallback), and for the fused path the
// sampled scores, the thresholds, the candidate slots, their counts and the
// fallback flags.  Offsets are 256-byte aligned.
struct IndexTopkLayout {
  dsa::FusedPlan f;
  size_t scores, topk_ws, sample, thresh, cand_key, cand_idx, count, flags, total;
};

IndexTopkLayout index_topk_layout(const dsa_problem* p) {
  IndexTopkLayout L{};
  L.f = dsa::fused_plan(p->batch, p->q_len, p->kv_len, p->q_start, p->idx_heads, p->idx_dim, p->topk);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += round_up(bytes);
    return o;
  };
  const size_t rows = (size_t)p->batch * p->q_len;
  L.scores = take(scores_bytes(p));
  L.topk_ws = take(dsa::topk_workspace_bytes(p->batch, p->q_len, p->q_start, p->kv_len, p->topk));
  if (L.f.use) {
    const size_t slots = rows * L.f.n_splits * L.f.cap_s;
    L.sample = take(rows * L.f.ls * sizeof(float));
    L.thresh = take(rows * sizeof(uint32_t));
    L.cand_key = take(slots * sizeof(uint32_t));
    L.cand_idx = take(slots * sizeof(int32_t));
    L.count = take(rows * L.f.n_splits * sizeof(int32_t));
    L.flags = take(rows * sizeof(int32_t));
  }
  L.total = off;
  return L;
}

// Indexer scores and top-k into `indices`.  Plain: the scores go to the
// workspace and the top-k reads them.  Fused (long rows, prefill shape): the
// indexer scores a key sample, a threshold per row is taken from it, the
// indexer writes only the (key, index) pairs at or above the threshold, and
// the top-k selects among those; rows whose candidates cannot be trusted are
// redone by the plain path, restricted to them.
int run_index_topk(const dsa_problem* p, const uint8_t* q_idx, const uint8_t* k_idx, const float* w,
                   int32_t* indices, uint8_t* ws, hipStream_t st) {
  const IndexTopkLayout L = index_topk_layout(p);
  float* scores = (float*)(ws + L.scores);
  void* topk_ws = ws + L.topk_ws;
  if (!L.f.use) {
    if (int s = hip_status(dsa::launch_index_scores(index_args(p, q_idx, k_idx, w, scores), st),
                           "index_scores launch"))
      return s;
    return hip_status(dsa::launch_topk(topk_args(p, scores, indices, topk_ws), st), "topk launch");
  }
  float* sample = (float*)(ws + L.sample);
  uint32_t* thresh = (uint32_t*)(ws + L.thresh);
  uint32_t* cand_key = (uint32_t*)(ws + L.cand_key);
  int32_t* cand_idx = (int32_t*)(ws + L.cand_idx);
  int32_t* count = (int32_t*)(ws + L.count);
  int32_t* flags = (int32_t*)(ws + L.flags);
  dsa::IndexArgs sa = index_args(p, q_idx, k_idx, w, sample);
  sa.key_stride = L.f.stride;
  sa.out_ld = L.f.ls;
  if (int s = hip_status(dsa::launch_index_scores(sa, st), "sampled index_scores launch")) return s;
  if (int s = hip_status(dsa::launch_fused_threshold(sample, thresh, p->batch, p->q_len, p->kv_len, p->q_start,
                                                     p->topk, L.f.stride, L.f.ls, st),
                         "threshold launch"))
    return s;
  dsa::IndexArgs fa = index_args(p, q_idx, k_idx, w, nullptr);
  fa.thresh = thresh;
  fa.cand_key = cand_key;
  fa.cand_idx = cand_idx;
  fa.row_count = count;
  fa.cap_s = L.f.cap_s;
  fa.n_splits = L.f.n_splits;
  if (int s = hip_status(dsa::launch_index_scores(fa, st), "filtering index_scores launch")) return s;
  dsa::TopkArgs ta = topk_args(p, nullptr, indices, nullptr);
  ta.nseg = L.f.n_splits;
  ta.seg_cap = L.f.cap_s;
  ta.cand_key = cand_key;
  ta.cand_idx = cand_idx;
  if (int s = hip_status(dsa::launch_fused_select(ta, count, flags, st), "fused select launch")) return s;
  dsa::IndexArgs pa = index_args(p, q_idx, k_idx, w, scores);
  pa.only_rows = flags;
  if (int s = hip_status(dsa::launch_index_scores(pa, st), "fallback index_scores launch")) return s;
  dsa::TopkArgs tb = topk_args(p, scores, indices, topk_ws);
  tb.only_rows = flags;
  return hip_status(dsa::launch_topk(tb, st), "fallback topk launch");
}

size_t attn_ws_bytes(const dsa_problem* p) {
  return dsa::attn_workspace_bytes(p->batch * p->q_len, p->topk, p->heads, p->d_latent);
}

// The chunk split is used when the workspace can hold its partial results.
dsa::AttnArgs attn_args(const dsa_problem* p, const uint16_t* q, const uint16_t* kv,
                        const int32_t* indices, float* out, float* lse, void* ws, size_t ws_bytes) {
  dsa::AttnArgs a{};
  a.q = q; a.kv = kv; a.indices = indices; a.out = out; a.lse = lse;
  a.B = p->batch; a.Lq = p->q_len; a.Lk = p->kv_len; a.H = p->heads;
  a.Dv = p->d_latent; a.Dr = p->d_rope; a.k = p->topk; a.q_start = p->q_start;
  a.scale_log2 = p->softmax_scale * 1.44269504088896340736f;
  a.nsplit = 1;
  const size_t need = attn_ws_bytes(p);
  if (need > 0 && ws && ws_bytes >= need) {
    const size_t rows = (size_t)p->batch * p->q_len;
    a.nsplit = dsa::attn_splits((int)rows, p->topk);
    a.part_out = (float*)ws;
    a.part_lse = a.part_out + rows * a.nsplit * p->heads * p->d_latent;
  }
  return a;
}

int check_forward(const dsa_problem* p, const uint8_t* q_idx, const uint8_t* k_idx, const float* w,
                  const uint16_t* q, const uint16_t* kv, const float* out, const float* lse,
                  const int32_t* indices) {
  if (int s = check_common(p)) return s;
  if (int s = check_index(p)) return s;
  if (int s = check_attn(p)) return s;
  if (int s = check_ptr(q_idx, "q_idx", 16)) return s;
  if (int s = check_ptr(k_idx, "k_idx", 16)) return s;
  if (int s = check_ptr(w, "w", 4)) return s;
  if (int s = check_ptr(q, "q", 16)) return s;
  if (int s = check_ptr(kv, "kv", 16)) return s;
  if (int s = check_ptr(out, "out", 16)) return s;
  if (lse && !aligned(lse, 4)) return fail(DSA_ERR_ALIGN, "lse is not 4-byte aligned");
  if (indices && !aligned(indices, 16)) return fail(DSA_ERR_ALIGN, "indices is not 16-byte aligned");
  return DSA_OK;
}

// Indexer -> top-k -> attention on `st`, with the scores, the selection (when
// the caller does not take it) and the top-k and attention scratch carved from
// `ws` (dsa_workspace_size(p, DSA_OP_FORWARD) bytes, 256-byte aligned).
int run_forward(const dsa_problem* p, const uint8_t* q_idx, const uint8_t* k_idx, const float* w,
                const uint16_t* q, const uint16_t* kv, float* out, float* lse, int32_t* indices,
                uint8_t* ws, hipStream_t st) {
  const size_t it_bytes = index_topk_layout(p).total;
  int32_t* sel = indices ? indices : (int32_t*)(ws + it_bytes);
  void* attn_ws = ws + it_bytes + round_up(indices_bytes(p));
  if (int s = run_index_topk(p, q_idx, k_idx, w, sel, ws, st)) return s;
  return hip_status(
      dsa::launch_sparse_mla_attn(attn_args(p, q, kv, sel, out, lse, attn_ws, attn_ws_bytes(p)), st),
      "sparse_mla_attn launch");
}

// Static scratch of dsa_forward_noalloc, for callers that cannot allocate.
// Each device holds its own copy for the life of the process.  Host code uses
// the device address hipGetSymbolAddress returns for the current device, never
// the array's name.  No part of the forward's workspace needs to start at
// zero, so the contents a previous call left are harmless; calls that overlap
// on one device race for it.
constexpr size_t kScratchBytes = size_t(128) << 20;
constexpr int kMaxDevices = 64;
__device__ __align__(256) uint8_t scratch[kScratchBytes];
std::atomic<uint8_t*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

int scratch_for_current_device(uint8_t** out) {
  int dev = -1;
  if (int s = hip_status(hipGetDevice(&dev), "hipGetDevice")) return s;
  if (dev < 0 || dev >= kMaxDevices) return fail(DSA_ERR_UNSUPPORTED, "device %d >= %d", dev, kMaxDevices);
  uint8_t* ptr = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!ptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    ptr = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (!ptr) {
      void* addr = nullptr;
      if (int s = hip_status(hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)"))
        return s;
      if (!addr || !aligned(addr, kAlign)) return fail(DSA_ERR_HIP, "scratch address %p not usable", addr);
      ptr = (uint8_t*)addr;
      g_scratch_ptr[dev].store(ptr, std::memory_order_release);
    }
  }
  *out = ptr;
  return DSA_OK;
}

}  // namespace

extern "C" {

const char* dsa_status_string(int status) {
  switch (status) {
    case DSA_OK: return "ok";
    case DSA_ERR_NULL: return "null pointer";
    case DSA_ERR_SHAPE: return "invalid shape or scale";
    case DSA_ERR_UNSUPPORTED: return "unsupported size";
    case DSA_ERR_WORKSPACE: return "workspace too small";
    case DSA_ERR_ALIGN: return "misaligned pointer";
    case DSA_ERR_HIP: return "HIP launch error";
    default: return "unknown status";
  }
}

const char* dsa_last_error(void) { return g_last_error; }

size_t dsa_workspace_size(const dsa_problem* p, int op) {
  const size_t bad = (size_t)-1;
  if (check_common(p)) return bad;
  switch (op) {
    case DSA_OP_INDEX_SCORES:
      return check_index(p) ? bad : 0;
    case DSA_OP_TOPK:
      if (check_topk(p)) return bad;
      return dsa::topk_workspace_bytes(p->batch, p->q_len, p->q_start, p->kv_len, p->topk);
    case DSA_OP_SPARSE_MLA_ATTN:
      return check_attn(p) ? bad : attn_ws_bytes(p);
    case DSA_OP_SPARSE_MLA_ATTN_BWD:
      return check_attn(p) || check_bwd_size(p) ? bad : bwd_ws_bytes(p);
    case DSA_OP_INDEX_TOPK:
      if (check_index(p) || check_topk(p)) return bad;
      return index_topk_layout(p).total;
    case DSA_OP_FORWARD:
      if (check_index(p) || check_attn(p)) return bad;
      return index_topk_layout(p).total + round_up(indices_bytes(p)) + round_up(attn_ws_bytes(p));
    default:
      fail(DSA_ERR_SHAPE, "unknown op %d", op);
      return bad;
  }
}

int dsa_index_scores(const dsa_problem* p, const uint8_t* q_idx, const uint8_t* k_idx,
                     const float* w, float* scores, void* stream) {
  if (int s = check_common(p)) return s;
  if (int s = check_index(p)) return s;
  if (int s = check_ptr(q_idx, "q_idx", 16)) return s;
  if (int s = check_ptr(k_idx, "k_idx", 16)) return s;
  if (int s = check_ptr(w, "w", 4)) return s;
  if (int s = check_ptr(scores, "scores", 4)) return s;
  return hip_status(dsa::launch_index_scores(index_args(p, q_idx, k_idx, w, scores),
                                             (hipStream_t)stream),
                    "index_scores launch");
}

int dsa_topk(const dsa_problem* p, const float* scores, int32_t* indices, void* workspace,
             size_t workspace_bytes, void* stream) {
  if (int s = check_common(p)) return s;
  if (int s = check_topk(p)) return s;
  if (int s = check_ptr(scores, "scores", 4)) return s;
  if (int s = check_ptr(indices, "indices", 4)) return s;
  const size_t need = dsa::topk_workspace_bytes(p->batch, p->q_len, p->q_start, p->kv_len, p->topk);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(DSA_ERR_WORKSPACE, "topk needs %zu workspace bytes, got %zu", need, workspace_bytes);
  if (need > 0 && !aligned(workspace, 16))
    return fail(DSA_ERR_ALIGN, "workspace is not 16-byte aligned");
  return hip_status(dsa::launch_topk(topk_args(p, scores, indices, need > 0 ? workspace : nullptr),
                                     (hipStream_t)stream),
                    "topk launch");
}

int dsa_index_topk(const dsa_problem* p, const uint8_t* q_idx, const uint8_t* k_idx, const float* w,
                   int32_t* indices, void* workspace, size_t workspace_bytes, void* stream) {
  if (int s = check_common(p)) return s;
  if (int s = check_index(p)) return s;
  if (int s = check_topk(p)) return s;
  if (int s = check_ptr(q_idx, "q_idx", 16)) return s;
  if (int s = check_ptr(k_idx, "k_idx", 16)) return s;
  if (int s = check_ptr(w, "w", 4)) return s;
  if (int s = check_ptr(indices, "indices", 4)) return s;
  const size_t need = index_topk_layout(p).total;
  if (!workspace || workspace_bytes < need)
    return fail(DSA_ERR_WORKSPACE, "index_topk needs %zu workspace bytes, got %zu", need, workspace_bytes);
  if (!aligned(workspace, kAlign)) return fail(DSA_ERR_ALIGN, "workspace is not 256-byte aligned");
  return run_index_topk(p, q_idx, k_idx, w, indices, (uint8_t*)workspace, (hipStream_t)stream);
}

int dsa_sparse_mla_attn_ws(const dsa_problem* p, const uint16_t* q, const uint16_t* kv,
                           const int32_t* indices, float* out, float* lse, void* workspace,
                           size_t workspace_bytes, void* stream) {
  if (int s = check_common(p)) return s;
  if (int s = check_attn(p)) return s;
  if (int s = check_ptr(q, "q", 16)) return s;
  if (int s = check_ptr(kv, "kv", 16)) return s;
  if (int s = check_ptr(indices, "indices", 16)) return s;
  if (int s = check_ptr(out, "out", 16)) return s;
  if (lse && !aligned(lse, 4)) return fail(DSA_ERR_ALIGN, "lse is not 4-byte aligned");
  if (workspace && !aligned(workspace, 16)) return fail(DSA_ERR_ALIGN, "workspace is not 16-byte aligned");
  return hip_status(dsa::launch_sparse_mla_attn(
                        attn_args(p, q, kv, indices, out, lse, workspace, workspace_bytes),
                        (hipStream_t)stream),
                    "sparse_mla_attn launch");
}

int dsa_sparse_mla_attn(const dsa_problem* p, const uint16_t* q, const uint16_t* kv,
                        const int32_t* indices, float* out, float* lse, void* stream) {
  return dsa_sparse_mla_attn_ws(p, q, kv, indices, out, lse, nullptr, 0, stream);
}

int dsa_sparse_mla_attn_bwd(const dsa_problem* p, const uint16_t* q, const uint16_t* kv,
                            const int32_t* indices, const float* out, const float* lse,
                            const float* dout, float* dq, float* dkv, void* workspace,
                            size_t workspace_bytes, void* stream) {
  if (int s = check_common(p)) return s;
  if (int s = check_attn(p)) return s;
  if (int s = check_ptr(q, "q", 16)) return s;
  if (int s = check_ptr(kv, "kv", 16)) return s;
  if (int s = check_ptr(indices, "indices", 16)) return s;
  if (int s = check_ptr(out, "out", 16)) return s;
  if (int s = check_ptr(lse, "lse", 4)) return s;
  if (int s = check_ptr(dout, "dout", 16)) return s;
  if (int s = check_ptr(dq, "dq", 16)) return s;
  if (int s = check_ptr(dkv, "dkv", 16)) return s;
  if (int s = check_bwd_size(p)) return s;
  const size_t need = bwd_ws_bytes(p);
  if (!workspace || workspace_bytes < need)
    return fail(DSA_ERR_WORKSPACE, "sparse_mla_attn_bwd needs %zu workspace bytes, got %zu", need,
                workspace_bytes);
  if (!aligned(workspace, 256)) return fail(DSA_ERR_ALIGN, "workspace is not 256-byte aligned");
  dsa::AttnBwdArgs a{};
  a.q = q; a.kv = kv; a.indices = indices; a.out = out; a.lse = lse; a.dout = dout;
  a.dq = dq; a.dkv = dkv;
  a.B = p->batch; a.Lq = p->q_len; a.Lk = p->kv_len; a.H = p->heads;
  a.Dv = p->d_latent; a.Dr = p->d_rope; a.k = p->topk;
  a.scale = p->softmax_scale;
  a.scale_log2 = p->softmax_scale * 1.44269504088896340736f;
  return hip_status(dsa::launch_sparse_mla_attn_bwd(a, workspace, (hipStream_t)stream),
                    "sparse_mla_attn_bwd launch");
}

int dsa_warmup_target(const dsa_problem* p, const uint16_t* q, const uint16_t* kv, const float* lse_in,
                      float* lse_out, float* target, void* stream) {
  if (int s = check_common(p)) return s;
  if (int s = check_latent(p)) return s;
  if (int s = check_ptr(q, "q", 16)) return s;
  if (int s = check_ptr(kv, "kv", 16)) return s;
  if (int s = check_ptr(target, "target", 4)) return s;
  if (lse_in && !aligned(lse_in, 4)) return fail(DSA_ERR_ALIGN, "lse_in is not 4-byte aligned");
  if (lse_out && !aligned(lse_out, 4)) return fail(DSA_ERR_ALIGN, "lse_out is not 4-byte aligned");
  if (lse_in && lse_out) return fail(DSA_ERR_SHAPE, "warmup_target: give lse_in or lse_out, not both");
  dsa::WarmupArgs a{};
  a.q = q; a.kv = kv; a.target = target; a.lse_in = lse_in; a.lse_out = lse_out;
  a.B = p->batch; a.Lq = p->q_len; a.Lk = p->kv_len; a.q_start = p->q_start; a.H = p->heads;
  a.Dv = p->d_latent; a.Dr = p->d_rope;
  a.scale_log2 = p->softmax_scale * 1.44269504088896340736f;
  a.inv_heads = 1.0f / (float)p->heads;
  return hip_status(dsa::launch_warmup_target(a, (hipStream_t)stream), "warmup_target launch");
}

int dsa_warmup_kl(const dsa_problem* p, const float* scores, const float* target, float* loss,
                  float* dscores, void* stream) {
  if (int s = check_common(p)) return s;
  if (int s = check_ptr(scores, "scores", 4)) return s;
  if (int s = check_ptr(target, "target", 4)) return s;
  if (int s = check_ptr(loss, "loss", 4)) return s;
  if (int s = check_ptr(dscores, "dscores", 4)) return s;
  if ((const void*)dscores == (const void*)target || (const void*)loss == (const void*)target ||
      (const void*)loss == (const void*)scores || (const void*)loss == (const void*)dscores)
    return fail(DSA_ERR_SHAPE, "warmup_kl: only dscores may share its buffer (with scores)");
  dsa::WarmupArgs a{};
  a.scores = scores; a.target = const_cast<float*>(target); a.loss = loss; a.dscores = dscores;
  a.B = p->batch; a.Lq = p->q_len; a.Lk = p->kv_len; a.q_start = p->q_start;
  return hip_status(dsa::launch_warmup_kl(a, (hipStream_t)stream), "warmup_kl launch");
}

int dsa_index_scores_bwd(const dsa_problem* p, const uint8_t* q_idx, const uint8_t* k_idx, const float* w,
                         const float* dscores, float* dq_idx, float* dw, float* dk_idx, void* stream) {
  if (int s = check_common(p)) return s;
  if (int s = check_index(p)) return s;
  if (int s = check_ptr(q_idx, "q_idx", 16)) return s;
  if (int s = check_ptr(k_idx, "k_idx", 16)) return s;
  if (int s = check_ptr(w, "w", 4)) return s;
  if (int s = check_ptr(dscores, "dscores", 4)) return s;
  if (int s = check_ptr(dq_idx, "dq_idx", 16)) return s;
  if (int s = check_ptr(dw, "dw", 4)) return s;
  if (int s = check_ptr(dk_idx, "dk_idx", 16)) return s;
  dsa::IndexBwdArgs a{};
  a.q_idx = q_idx; a.k_idx = k_idx; a.w = w; a.dscores = dscores;
  a.dq_idx = dq_idx; a.dw = dw; a.dk_idx = dk_idx;
  a.B = p->batch; a.Lq = p->q_len; a.Lk = p->kv_len; a.q_start = p->q_start;
  a.H = p->idx_heads; a.DI = p->idx_dim;
  return hip_status(dsa::launch_index_scores_bwd(a, (hipStream_t)stream), "index_scores_bwd launch");
}

int dsa_masked_mha_attn(const dsa_problem* p, const uint16_t* q, const uint16_t* kv,
                        const int32_t* indices, float* out, float* lse, void* stream) {
  if (int s = check_common(p)) return s;
  if (int s = check_attn(p)) return s;
  // the selection bitmap of a row (one bit per key) sits in LDS
  if (p->kv_len > kMaskedMaxKv)
    return fail(DSA_ERR_UNSUPPORTED, "masked mode: kv_len %d > %d", p->kv_len, kMaskedMaxKv);
  if (int s = check_ptr(q, "q", 16)) return s;
  if (int s = check_ptr(kv, "kv", 16)) return s;
  if (int s = check_ptr(indices, "indices", 16)) return s;
  if (int s = check_ptr(out, "out", 16)) return s;
  if (lse && !aligned(lse, 4)) return fail(DSA_ERR_ALIGN, "lse is not 4-byte aligned");
  return hip_status(dsa::launch_masked_mha_attn(attn_args(p, q, kv, indices, out, lse, nullptr, 0),
                                                (hipStream_t)stream),
                    "masked_mha_attn launch");
}

int dsa_forward(const dsa_problem* p, const uint8_t* q_idx, const uint8_t* k_idx, const float* w,
                const uint16_t* q, const uint16_t* kv, float* out, float* lse, int32_t* indices,
                void* workspace, size_t workspace_bytes, void* stream) {
  if (int s = check_forward(p, q_idx, k_idx, w, q, kv, out, lse, indices)) return s;
  const size_t need = dsa_workspace_size(p, DSA_OP_FORWARD);
  if (!workspace || workspace_bytes < need)
    return fail(DSA_ERR_WORKSPACE, "forward needs %zu workspace bytes, got %zu", need, workspace_bytes);
  if (!aligned(workspace, kAlign)) return fail(DSA_ERR_ALIGN, "workspace is not 256-byte aligned");
  return run_forward(p, q_idx, k_idx, w, q, kv, out, lse, indices, (uint8_t*)workspace, (hipStream_t)stream);
}

int dsa_forward_noalloc(const dsa_problem* p, const uint8_t* q_idx, const uint8_t* k_idx, const float* w,
                        const uint16_t* q, const uint16_t* kv, float* out, float* lse, int32_t* indices,
                        void* stream) {
  if (int s = check_forward(p, q_idx, k_idx, w, q, kv, out, lse, indices)) return s;
  const size_t need = dsa_workspace_size(p, DSA_OP_FORWARD);
  if (need > kScratchBytes)
    return fail(DSA_ERR_UNSUPPORTED,
                "forward_noalloc: this problem needs %zu bytes of scratch; the library's static scratch "
                "holds %zu (use dsa_forward with a workspace)", need, kScratchBytes);
  uint8_t* ws = nullptr;
  if (int s = scratch_for_current_device(&ws)) return s;
  return run_forward(p, q_idx, k_idx, w, q, kv, out, lse, indices, ws, (hipStream_t)stream);
}

}  // extern "C"
