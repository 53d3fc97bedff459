/*
 * dsa.h — C ABI of libdsa.so, the DeepSeek Sparse Attention (DSA) hot path on
 * one AMD Instinct MI355X (gfx950).
 *
 * The path has three stages, each its own entry point, plus a fused forward:
 *
 *   dsa_index_scores     lightning indexer: a few indexer heads score every
 *                        (query, preceding token) pair as a weighted sum of
 *                        ReLU'd FP8 dot products.
 *                        ("DeepSeek V3.2 and the lightning indexer", section
 *                        "How the lightning indexer works"; DeepSeek-V3.2 spec
 *                        sheet, design overview / section 2.1.)
 *   dsa_topk             fine-grained token selection: each query keeps the k
 *                        best-scoring preceding tokens (same sections; k = 2048
 *                        in the sparse training stage).
 *   dsa_sparse_mla_attn  MLA in its MQA mode over the selected latents only:
 *                        one latent vector per token, shared by every query
 *                        head, one selection per query position (lightning
 *                        indexer post, same section; spec sheet, "Inference
 *                        efficiency" table, KV-cache design).
 *   dsa_sparse_mla_attn_ws  the same with a workspace that lets few rows
 *                        (decode) spread over the whole chip.
 *   dsa_sparse_mla_attn_bwd  gradients of the sparse attention (dq, dkv) over
 *                        fixed indices, for the sparse training stage.
 *   dsa_warmup_target    the main attention's distribution summed over the
 *                        heads, dense over each query's causal range: the
 *                        target of the indexer's warm-up objective.
 *   dsa_warmup_kl        KL(target || softmax(indexer scores)) per query and
 *                        its gradient with respect to the scores.
 *   dsa_index_scores_bwd gradients of the indexer scores with respect to the
 *                        indexer's q_I, w and k_I.
 *   dsa_masked_mha_attn  the same attention computed densely over each
 *                        query's causal range with the non-selected tokens
 *                        masked: the masked mode for short prefill.
 *   dsa_index_topk       the indexer and the top-k together, without
 *                        materialising every score of long rows.
 *   dsa_forward          the three stages in order on one stream.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every tensor pointer is a DEVICE pointer to a dense row-major buffer that
 *    the caller allocates and owns.  The library never allocates, frees or
 *    retains device memory and keeps no state between calls.  Buffers must
 *    stay alive until the stream work completes.  Outputs must not alias
 *    inputs.
 *  - `stream` is a hipStream_t (NULL = the legacy default stream).  Calls only
 *    enqueue work and return; kernel faults surface at the caller's next
 *    synchronisation.
 *  - Shapes: B = batch, Lq = new query tokens per sequence, Lk = cached tokens
 *    per sequence, H_I = indexer heads, d_I = indexer dim, H = query heads,
 *    D_v = latent (= value) width, D_r = rope width, D_qk = D_v + D_r.
 *    Query row t of sequence b sits at absolute position pos(t) = q_start + t
 *    and may look at tokens s = 0 .. pos(t) (its own token included).
 *  - Return value: DSA_OK (0) or a negative status.  Every argument check runs
 *    before any launch, so a call that fails leaves every buffer untouched.
 *    dsa_last_error() gives a thread-local description of the last failure.
 *  - There is no CPU fallback: shapes the kernels do not cover return
 *    DSA_ERR_UNSUPPORTED.
 */
#ifndef DSA_H_
#define DSA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum dsa_status {
  DSA_OK = 0,
  DSA_ERR_NULL = -1,        /* a required pointer is NULL                         */
  DSA_ERR_SHAPE = -2,       /* non-positive size, q_start+q_len > kv_len, bad scale */
  DSA_ERR_UNSUPPORTED = -3, /* a size the kernels do not cover                    */
  DSA_ERR_WORKSPACE = -4,   /* workspace missing or smaller than required         */
  DSA_ERR_ALIGN = -5,       /* a pointer is not 16-byte aligned                    */
  DSA_ERR_HIP = -6          /* the HIP runtime rejected a launch                   */
};

/* Problem description.  All fields are read by every entry point that needs
 * them; unused fields are ignored (e.g. heads/d_latent by dsa_index_scores). */
typedef struct dsa_problem {
  int32_t batch;       /* B  >= 1                                              */
  int32_t q_len;       /* Lq >= 1                                              */
  int32_t kv_len;      /* Lk >= 1, q_start + q_len <= kv_len; for the attention
                          also Lk <= 2^24 and Lk * D_qk * 2 <= 4 GiB - 8 KiB  */
  int32_t q_start;     /* absolute position of query row 0 (>= 0)              */
  int32_t idx_heads;   /* H_I, 1..64                                           */
  int32_t idx_dim;     /* d_I: 32, 64, 96 or 128                                */
  int32_t topk;        /* k, 1..2048                                           */
  int32_t heads;       /* H, 1..128                                            */
  int32_t d_latent;    /* D_v: 512, or 64 (with D_r = 16)                       */
  int32_t d_rope;      /* D_r: 64 (with D_v = 512), or 16 (with D_v = 64)       */
  float softmax_scale; /* finite, > 0; e.g. 1/sqrt(D_qk)                       */
} dsa_problem;

/* Operation selector for dsa_workspace_size(). */
enum dsa_op {
  DSA_OP_INDEX_SCORES = 0,
  DSA_OP_TOPK = 1,
  DSA_OP_SPARSE_MLA_ATTN = 2,
  DSA_OP_FORWARD = 3,
  DSA_OP_SPARSE_MLA_ATTN_BWD = 4,
  DSA_OP_INDEX_TOPK = 5
};

/*
 * Lightning indexer scores.
 *   I[b,t,s] = sum_{j<H_I} w[b,t,j] * ReLU( sum_{d<d_I} q_idx[b,t,j,d] * k_idx[b,s,d] )
 * for s = 0 .. pos(t); entries with s > pos(t) are NOT written.
 *
 *   q_idx  [B, Lq, H_I, d_I] uint8, OCP FP8 e4m3fn (scale 1)
 *   k_idx  [B, Lk, d_I]      uint8, OCP FP8 e4m3fn, one key per token shared by
 *                             every indexer head
 *   w      [B, Lq, H_I]      float32 head weights
 *   scores [B, Lq, Lk]       float32 output, row stride Lk
 * The dot products run on FP8 matrix cores with fp32 accumulation; the ReLU
 * and the weighted head sum in fp32.  Zero results are +0.  When every partial
 * sum is exactly representable in fp32 (true for the 0.25-step value grids of
 * [-4,4] for q/k and [-1,1] for w) the result equals the exact value; for
 * other finite inputs it is the exact value within fp32 accumulation error.
 * Every finite e4m3fn code (subnormals and +-448 included) is read as its OCP
 * value; the NaN codes 0x7F and 0xFF give unspecified scores.
 */
int dsa_index_scores(const dsa_problem* p, const uint8_t* q_idx, const uint8_t* k_idx,
                     const float* w, float* scores, void* stream);

/*
 * Top-k selection per query row.
 * Row (b,t) keeps the min(k, pos(t)+1) candidates s in 0..pos(t) that come
 * first under the order (score descending, index ascending) — ties go to the
 * lower index, and -0 equals +0.  Indices are written in ascending order; the
 * remaining slots hold -1.  Scores at s > pos(t) are never read.  NaN scores
 * give an unspecified (but in-range) selection.
 *
 *   scores  [B, Lq, Lk] float32 (as written by dsa_index_scores)
 *   indices [B, Lq, k]  int32 output
 *   workspace: device scratch of at least dsa_workspace_size(p, DSA_OP_TOPK)
 *              bytes, 16-byte aligned (may be NULL when that size is 0).  It
 *              is non-zero when rows can exceed 32768 candidates: such rows are
 *              selected in two stages (top k of each segment, then of their
 *              union), with B*Lq*nseg*k*8 bytes of candidates in between.
 *              Segments hold 32768 keys while nseg*k <= 65536 (rows of up to
 *              1,048,576 candidates at k = 2048); 8192 keys instead when
 *              nseg*k <= 32768 for them and B*Lq times the 32768-key segment
 *              count is below 2048.  At most 256 such rows (k % 4 == 0, as
 *              in decode) are selected instead from a cut taken on a 1/16
 *              sample of each row: the keys at or above it are kept in
 *              4096-key splits of a few hundred slots each, then selected
 *              exactly (a row the cut does not settle is selected from its
 *              scores by passes over the row); the workspace then holds a
 *              cut per row, a count per split and the splits' slots (about
 *              4 MB for 64 rows of 131072 keys).  Longer rows need no
 *              workspace: they are selected by passes that re-read the
 *              row.  Contents on return are unspecified.
 */
int dsa_topk(const dsa_problem* p, const float* scores, int32_t* indices, void* workspace,
             size_t workspace_bytes, void* stream);

/*
 * dsa_index_scores followed by dsa_topk, without necessarily materialising
 * the scores: the selection of the lightning indexer ("DeepSeek V3.2 and the
 * lightning indexer", "How the lightning indexer works": score every
 * preceding token, keep the k best per query).  The result is bit-identical
 * to the two calls.
 *
 *   q_idx, k_idx, w  as for dsa_index_scores
 *   indices  [B, Lq, k] int32 output, as for dsa_topk
 *   workspace: at least dsa_workspace_size(p, DSA_OP_INDEX_TOPK) bytes,
 *              256-byte aligned; contents on return are unspecified.
 * When rows exceed 32768 keys in a problem of at least 8 queries per
 * sequence, the scores of one key in 16 (32, 64, ... for rows past 512K keys)
 * give each row a threshold, the indexer then writes only the keys at or
 * above it (a little more than k per row instead of the whole row) and the
 * top-k selects among those; a row whose sample misled the threshold (fewer
 * than k keys above it, or more than its candidate slots hold, e.g. heavy
 * ties) is recomputed through its full score row, so every row's result is
 * exact.  Otherwise (decode, rows up to 32768 keys) it runs the two stages as
 * they are.  The workspace holds the full score matrix either way
 * (4 * B * Lq * Lk bytes, for the recomputed rows).
 */
int dsa_index_topk(const dsa_problem* p, const uint8_t* q_idx, const uint8_t* k_idx, const float* w,
                   int32_t* indices, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Sparse attention, MQA mode of MLA, over the selected latents.
 * For every (b, t, h), over the entries s of indices[b,t,:] with 0 <= s < Lk
 * (other entries, e.g. the -1 padding, are skipped):
 *   z_s = softmax_scale * sum_{d<D_qk} q[b,t,h,d] * kv[b,s,d]
 *   out[b,t,h,:] = sum_s softmax(z)_s * kv[b,s,0:D_v]
 *   lse[b,t,h]   = log(sum_s exp(z_s))             (natural log)
 * The value of a latent is its first D_v columns; the last D_r columns (rope)
 * only enter the scores.  A row with no valid entry gives out = 0, lse = -inf.
 * ("DeepSeek V3.2 and the lightning indexer", "How the lightning indexer
 * works": the main attention runs only over the selected tokens, MLA in its
 * MQA mode with one latent per token shared by all heads.)
 *
 *   q       [B, Lq, H, D_qk] bfloat16 (raw bits)
 *   kv      [B, Lk, D_qk]    bfloat16 latent cache, one row per token shared
 *                             by every head
 *   indices [B, Lq, k]       int32
 *   out     [B, Lq, H, D_v]  float32 output
 *   lse     [B, Lq, H]       float32 output, or NULL
 * One block handles a query row.  Scores and the softmax run in fp32; the
 * probabilities are rounded to bf16 for the value product on bf16 matrix
 * cores with fp32 accumulation.  No workspace.
 */
int dsa_sparse_mla_attn(const dsa_problem* p, const uint16_t* q, const uint16_t* kv,
                        const int32_t* indices, float* out, float* lse, void* stream);

/*
 * dsa_sparse_mla_attn with a workspace that lets it split rows: the same
 * arguments and results, plus
 *   workspace: device scratch, 16-byte aligned, or NULL.  When it holds at
 *              least dsa_workspace_size(p, DSA_OP_SPARSE_MLA_ATTN) bytes and
 *              that size is non-zero (fewer query rows than compute units, as
 *              in decode), each row's selected entries are split over several
 *              blocks whose normalised partial results (and their lse) are
 *              merged by a second kernel; otherwise (NULL, too small, or a size
 *              of 0) it runs exactly as dsa_sparse_mla_attn.  The split keeps
 *              rows x parts x H x (D_v + 1) floats there; contents on return
 *              are unspecified.  Results agree with the unsplit call within
 *              rounding.
 */
int dsa_sparse_mla_attn_ws(const dsa_problem* p, const uint16_t* q, const uint16_t* kv,
                           const int32_t* indices, float* out, float* lse, void* workspace,
                           size_t workspace_bytes, void* stream);

/*
 * Backward of dsa_sparse_mla_attn over fixed indices: the gradients the sparse
 * training stage needs, where every parameter is trained with the selection
 * on (DeepSeek-V3.2 spec sheet, design overview; lightning-indexer post,
 * training section).  No gradient flows into the indices.  Per (b, t, h),
 * with z_i, p = softmax(z) and o as in the forward and g = dout[b,t,h,:]:
 *   D = g . o,  dz_i = p_i (g . v_i - D),
 *   dq[b,t,h,:]  = softmax_scale * sum_i dz_i kv[b,s_i,:]
 *   dkv[b,s_i,:] += softmax_scale * dz_i q[b,t,h,:]   (+ p_i g on the first D_v columns)
 * summed over every (t, h, i) that lists s_i (entries outside [0, Lk) are
 * skipped, a repeated entry is a separate term, as in the forward).
 *
 *   q, kv, indices  as for dsa_sparse_mla_attn
 *   out  [B, Lq, H, D_v]  float32, the forward's output
 *   lse  [B, Lq, H]       float32, the forward's lse (required)
 *   dout [B, Lq, H, D_v]  float32, the upstream gradient
 *   dq   [B, Lq, H, D_qk] float32 output (written)
 *   dkv  [B, Lk, D_qk]    float32, ACCUMULATED into: each listed token's
 *                         total is added once (no atomics on dkv), so the
 *                         caller zeroes it or passes gradients to add to;
 *                         the order in which a token's terms are summed
 *                         varies, hence its last bits may vary between runs
 *   workspace: at least dsa_workspace_size(p, DSA_OP_SPARSE_MLA_ATTN_BWD)
 *              bytes, 256-byte aligned; contents on return are unspecified.
 *              With R = B*Lq and kp = k rounded up to 32, it holds P and dZ
 *              (2 * R*kp*128 bf16), one partial dkv row per (row, entry)
 *              (R*kp*D_qk bf16) and the per-token lists of those entries
 *              (R*k + 3*B*Lk int32, plus one int32 per 4096 tokens), each
 *              part rounded up to 256 bytes.
 * Requires B*Lq*kp and B*Lk below 2^31 (DSA_ERR_UNSUPPORTED otherwise).
 * The products run on bf16 matrix cores with fp32 accumulation; dout, P, dZ
 * and the partial dkv rows are rounded to bf16 (D = dout . o uses the same
 * rounded dout as the products, so a row's dZ sums to zero as it should).  dq and dkv must not alias
 * any input.
 */
int dsa_sparse_mla_attn_bwd(const dsa_problem* p, const uint16_t* q, const uint16_t* kv,
                            const int32_t* indices, const float* out, const float* lse,
                            const float* dout, float* dq, float* dkv, void* workspace,
                            size_t workspace_bytes, void* stream);

/*
 * Target distribution of the indexer's dense warm-up, in which only the
 * indexer is trained so that its softmax matches the main attention's
 * distribution summed over the heads, under a KL loss (DeepSeek-V3.2 spec
 * sheet, design overview and the curriculum row of its training table;
 * lightning-indexer post, training section).  Readings: the main attention is
 * dense over s <= pos(t), and the sum over heads is divided by H so that each
 * row is a distribution:
 *   target[b,t,s] = (1/H) sum_h softmax_s'(softmax_scale * q[b,t,h,:] . kv[b,s',:])[s]
 * for s = 0 .. pos(t) (s < Lk); other entries are left untouched.
 *
 *   q, kv    as for dsa_sparse_mla_attn (topk is not used by this call)
 *   lse_in   [B, Lq, H] float32 or NULL: each head's log-sum-exp (natural
 *            log) of its dense causal scores, if the caller has it (the
 *            dense attention forward of the warm-up computes it); the kernel
 *            then skips its first pass
 *   lse_out  [B, Lq, H] float32 or NULL: receives that lse when lse_in is
 *            NULL (giving both is DSA_ERR_SHAPE); entries of absent rows are
 *            untouched
 *   target   [B, Lq, Lk] float32 output
 * Scores are bf16 products with fp32 accumulation; exponentials in fp32.
 * Without lse_in the kernel computes each head's lse over the row first, so
 * it reads the row's latents twice.  No workspace.
 */
int dsa_warmup_target(const dsa_problem* p, const uint16_t* q, const uint16_t* kv, const float* lse_in,
                      float* lse_out, float* target, void* stream);

/*
 * The warm-up's loss and score gradient (same passages): per query row, over
 * s = 0 .. pos(t) (s < Lk), with pi = softmax(scores[b,t,:]),
 *   loss[b,t]       = sum_s target (log target - log pi)   (terms with target = 0 are 0)
 *   dscores[b,t,s]  = pi_s - target[b,t,s]                  (the gradient of sum_t loss)
 * Entries of dscores past pos(t) are left untouched.
 *
 *   scores   [B, Lq, Lk] float32 (e.g. dsa_index_scores' output)
 *   target   [B, Lq, Lk] float32 (e.g. dsa_warmup_target's output)
 *   loss     [B, Lq]     float32 output
 *   dscores  [B, Lq, Lk] float32 output; may be `scores` itself (in place),
 *            must not overlap target or loss
 * Only batch, q_len, kv_len and q_start of *p are used.  fp32 arithmetic,
 * each row's loss summed in fp64.  No workspace.
 */
int dsa_warmup_kl(const dsa_problem* p, const float* scores, const float* target, float* loss,
                  float* dscores, void* stream);

/*
 * Gradients of dsa_index_scores with respect to its inputs, for a gradient
 * dscores of the scores (e.g. dsa_warmup_kl's): the indexer's backward in its
 * warm-up training (same passages as dsa_warmup_target).  With
 * u = q_I[b,t,j,:] . k_I[b,s,:] and the ReLU's derivative taken as 0 at 0,
 * summed over s = 0 .. pos(t) (s < Lk):
 *   dw[b,t,j]       = sum_s dscores[b,t,s] ReLU(u)
 *   dq_idx[b,t,j,:] = w[b,t,j] sum_s dscores[b,t,s] [u > 0] k_I[b,s,:]
 *   dk_idx[b,s,:]  += sum_(t,j) dscores[b,t,s] w[b,t,j] [u > 0] q_I[b,t,j,:]
 *
 *   q_idx, k_idx, w  as for dsa_index_scores
 *   dscores  [B, Lq, Lk] float32; entries past pos(t) are not read
 *   dq_idx   [B, Lq, H_I, d_I] float32 output (written)
 *   dw       [B, Lq, H_I] float32 output (written)
 *   dk_idx   [B, Lk, d_I] float32, ACCUMULATED into (fp32 atomic adds of
 *            per-block partial sums: the caller zeroes it; the last bits can
 *            vary between runs)
 * u is recomputed on bf16 matrix cores (the e4m3 values are exact in bf16)
 * with fp32 accumulation; dscores * w is rounded to bf16 for the two
 * products; dw is accumulated in fp32.  No workspace.
 */
int dsa_index_scores_bwd(const dsa_problem* p, const uint8_t* q_idx, const uint8_t* k_idx, const float* w,
                         const float* dscores, float* dq_idx, float* dw, float* dk_idx, void* stream);

/*
 * Masked mode for short prefill: the same attention as dsa_sparse_mla_attn,
 * computed densely.  The pages name a masked MHA mode that simulates DSA for
 * short-sequence prefill without specifying it (DeepSeek-V3.2 spec sheet,
 * design overview; "Inference efficiency" table, serving optimisations); the
 * reading taken here: for every (b, t, h), the scores of ALL tokens
 * s = 0 .. pos(t) are computed from contiguous latent rows and those not in
 * the selection are masked out of the softmax, so
 *   out[b,t,h,:], lse[b,t,h] = attention over { s <= pos(t) : s in indices[b,t,:] }
 * Entries that are -1, out of range or past pos(t) are ignored and a repeated
 * entry counts once; for selections made by dsa_topk (distinct, <= pos(t))
 * this equals dsa_sparse_mla_attn within rounding.  A row with no selected
 * entry gives out = 0, lse = -inf.  Work grows with pos(t) rather than k.
 *
 *   q, kv, indices, out, lse: as for dsa_sparse_mla_attn.
 * Requires kv_len <= 65536 (DSA_ERR_UNSUPPORTED otherwise).  No workspace.
 */
int dsa_masked_mha_attn(const dsa_problem* p, const uint16_t* q, const uint16_t* kv,
                        const int32_t* indices, float* out, float* lse, void* stream);

/*
 * dsa_index_scores -> dsa_topk -> dsa_sparse_mla_attn on one stream: the
 * whole sparse attention of a layer, in the order the lightning-indexer post
 * gives it ("How the lightning indexer works": score every preceding token,
 * keep the top k per query, attend over those only).
 * The scores live in the workspace (at least dsa_workspace_size(p,
 * DSA_OP_FORWARD) bytes, 256-byte aligned).  `indices` may be NULL; when given
 * ([B, Lq, k] int32) it receives the selection, otherwise the selection is
 * kept in the workspace, together with the top-k and attention scratch.
 * It runs dsa_index_topk, then dsa_sparse_mla_attn_ws; results are
 * bit-identical to dsa_index_scores, dsa_topk and dsa_sparse_mla_attn_ws
 * called with workspaces of the sizes dsa_workspace_size() reports for them.
 */
int dsa_forward(const dsa_problem* p, const uint8_t* q_idx, const uint8_t* k_idx, const float* w,
                const uint16_t* q, const uint16_t* kv, float* out, float* lse, int32_t* indices,
                void* workspace, size_t workspace_bytes, void* stream);

/*
 * dsa_forward without a workspace, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops such as decode,
 * harnesses that forbid allocation).  Same arguments and results as
 * dsa_forward minus the workspace: the scores, the selection (when `indices`
 * is NULL) and the top-k and attention scratch live in a static device array
 * of 128 MiB that the library holds on every GPU it runs on until the process
 * ends.  Problems whose dsa_workspace_size(p, DSA_OP_FORWARD) exceeds 128 MiB
 * return DSA_ERR_UNSUPPORTED before any launch (the 64-sequence decode over
 * 131,072 tokens needs about 106 MB; long prefills do not fit).  Every call
 * on a device uses that device's one array: calls that overlap on one device
 * (e.g. on two streams) race and give undefined results.  The first call on a
 * device looks up the array's address there (no allocation).
 */
int dsa_forward_noalloc(const dsa_problem* p, const uint8_t* q_idx, const uint8_t* k_idx, const float* w,
                        const uint16_t* q, const uint16_t* kv, float* out, float* lse, int32_t* indices,
                        void* stream);

/* Bytes of device workspace `op` needs for problem `p` (0 if none); returns
 * (size_t)-1 when the problem is invalid (dsa_last_error() says why). */
size_t dsa_workspace_size(const dsa_problem* p, int op);

/* Static text for a status code. */
const char* dsa_status_string(int status);

/* Thread-local text describing the last failing call on this thread. */
const char* dsa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* DSA_H_ */
