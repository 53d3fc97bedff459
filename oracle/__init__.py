"""CPU oracle for the DeepSeek Sparse Attention hot path.

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` are the only callers.  The GPU library never
imports, links or calls this package, and this package imports nothing from it.

The arithmetic lives in ``dsa_oracle.c`` (plain C, OpenMP over query rows,
double precision); this module only builds it with gcc and marshals numpy
arrays.  Every function works on an explicit list of query rows, given by batch
index and absolute position, so large workloads can be checked on a sample.

Sources (cited by page title and section):
  * "DeepSeek V3.2 and the lightning indexer", section "How the lightning
    indexer works": indexer heads, weighted sum of ReLU'd dot products, FP8,
    top-2048 per query, MQA mode of MLA with one selection per query position.
  * DeepSeek-V3.2 spec sheet, design overview and section 2.1: every
    preceding token is scored; fine-grained top-k; MQA-mode MLA latents.
Readings where the pages are silent are listed in the module docstrings of the
functions below.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import time

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# DSA_ORACLE_LIBRARY names another build (the sanitizer test's); unset, the
# in-tree build is used.
_LIB_PATH = os.environ.get("DSA_ORACLE_LIBRARY") or os.path.join(_HERE, "liboracle.so")
_lib = None


def build() -> None:
    src = os.path.join(_HERE, "dsa_oracle.c")
    tmp = _LIB_PATH + ".tmp"
    subprocess.check_call(["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-std=c11",
                           src, "-o", tmp, "-lm"])
    os.replace(tmp, _LIB_PATH)


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        L = ctypes.CDLL(_LIB_PATH)
        i32, i64, vp, f32 = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p, ctypes.c_float
        L.dsa_oracle_e4m3_to_double.argtypes = [ctypes.c_uint8]
        L.dsa_oracle_e4m3_to_double.restype = ctypes.c_double
        L.dsa_oracle_index_scores.argtypes = [i32, i32, i32, i64, vp, vp, vp, vp, vp, vp]
        L.dsa_oracle_index_scores.restype = None
        L.dsa_oracle_topk.argtypes = [i32, i32, i64, vp, vp, vp]
        L.dsa_oracle_topk.restype = None
        L.dsa_oracle_sparse_mla_attn.argtypes = [i32, i32, i32, i32, i32, f32, i64,
                                                 vp, vp, vp, vp, vp, vp]
        L.dsa_oracle_sparse_mla_attn.restype = None
        L.dsa_oracle_masked_mha_attn.argtypes = [i32, i32, i32, i32, i32, f32, i64,
                                                 vp, vp, vp, vp, vp, vp, vp]
        L.dsa_oracle_masked_mha_attn.restype = None
        L.dsa_oracle_sparse_mla_attn_bwd.argtypes = [i32, i32, i32, i32, i32, f32, i64,
                                                     vp, vp, vp, vp, vp, vp, vp]
        L.dsa_oracle_sparse_mla_attn_bwd.restype = None
        L.dsa_oracle_warmup_target.argtypes = [i32, i32, i32, f32, i64, vp, vp, vp, vp, vp]
        L.dsa_oracle_warmup_target.restype = None
        L.dsa_oracle_warmup_kl.argtypes = [i32, i64, vp, vp, vp, vp, vp]
        L.dsa_oracle_warmup_kl.restype = None
        L.dsa_oracle_index_scores_bwd.argtypes = [i32, i32, i32, i64, vp, vp, vp, vp, vp, vp, vp, vp, vp]
        L.dsa_oracle_index_scores_bwd.restype = None
        L.dsa_oracle_max_threads.argtypes = []
        L.dsa_oracle_max_threads.restype = ctypes.c_int
        _lib = L
    return _lib


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a, a.ctypes.data


def max_threads() -> int:
    return int(lib().dsa_oracle_max_threads())


def e4m3_to_float64(codes) -> np.ndarray:
    """OCP FP8 e4m3fn byte -> value, from the format's definition."""
    codes = np.asarray(codes, dtype=np.uint8).ravel()
    f = lib().dsa_oracle_e4m3_to_double
    return np.array([f(int(c)) for c in codes], dtype=np.float64)


def index_scores(k_idx, q_idx_rows, w_rows, row_batch, row_pos, fill=np.nan) -> np.ndarray:
    """Lightning-indexer scores of the given query rows.

    k_idx      [B, Lk, d_I] uint8 (e4m3fn)
    q_idx_rows [R, H_I, d_I] uint8 (e4m3fn)
    w_rows     [R, H_I] float32
    row_batch, row_pos  [R] int32 (absolute position pos(t) = q_start + t)
    Returns [R, Lk] float32 with I[r, s] for s <= pos_r and `fill` elsewhere.
    Causal set reading: s ranges over 0..pos(t) inclusive of the query's own
    token ("every preceding token" read inclusively, so the first token has a
    candidate and dense-equivalence at L <= k is standard causal attention).
    """
    k_idx = np.ascontiguousarray(k_idx, dtype=np.uint8)
    B, Lk, dI = k_idx.shape
    q_idx_rows, qp = _c(q_idx_rows, np.uint8)
    R, HI, dI2 = q_idx_rows.shape
    assert dI2 == dI
    w_rows, wp = _c(w_rows, np.float32)
    assert w_rows.shape == (R, HI)
    rb, rbp = _c(row_batch, np.int32)
    rp, rpp = _c(row_pos, np.int32)
    assert rb.shape == (R,) and rp.shape == (R,)
    assert (rb >= 0).all() and (rb < B).all() and (rp >= 0).all()
    out = np.full((R, Lk), fill, dtype=np.float32)
    lib().dsa_oracle_index_scores(Lk, HI, dI, R, rbp, rpp, qp, wp, k_idx.ctypes.data, out.ctypes.data)
    return out


def on_score_grid(q_idx, k_idx, w) -> bool:
    """True when every decoded q_I / k_I value is a multiple of 1/4 with
    magnitude <= 4 and every weight a multiple of 1/4 with magnitude <= 1 (the
    value grids of the synthetic workloads)."""
    table = e4m3_to_float64(np.arange(256))
    ok_code = np.zeros(256, dtype=bool)
    fin = np.isfinite(table)
    ok_code[fin] = (np.abs(table[fin]) <= 4.0) & (table[fin] * 4 == np.round(table[fin] * 4))
    if not ok_code[np.asarray(q_idx, dtype=np.uint8)].all():
        return False
    if not ok_code[np.asarray(k_idx, dtype=np.uint8)].all():
        return False
    w = np.asarray(w, dtype=np.float64)
    return bool(((np.abs(w) <= 1.0) & (w * 4 == np.round(w * 4))).all())


def index_scores_blas(k_idx, q_idx_rows, w_rows, row_batch, row_pos, fill=np.nan,
                      rows_per_block: int = 32) -> np.ndarray:
    """The same lightning-indexer definition as index_scores, evaluated with
    library matrix products in double precision, for checking whole outputs of
    large workloads (arguments and result as for index_scores).

    Steps, in the definition's order ("DeepSeek V3.2 and the lightning
    indexer", "How the lightning indexer works"): decode the FP8 codes; the
    per-head dot products D[r,j,s] = q_I[r,j,:] . k_I[b_r,s,:] as one matrix
    product; the ReLU; the weighted head sum I[r,s] = sum_j w[r,j] ReLU(D[r,j,s])
    as a batched product; +0 for -0; one rounding to fp32.

    Exactness (why the library's summation order cannot matter): it accepts
    only inputs on the workloads' grids (on_score_grid), and needs
    H_I * d_I <= 8192.  Then every product q*k is a multiple of 2^-4 below 2^4
    in magnitude, every partial sum of a dot product a multiple of 2^-4 below
    2^11, every term w * ReLU(D) a multiple of 2^-6, and every partial sum of
    the head sum a multiple of 2^-6 below 2^17 in magnitude: at most 24
    significant bits, so each double-precision sum and the final fp32 rounding
    are exact, and the result equals index_scores bit for bit.  Other inputs
    raise ValueError.  Rows are processed a block at a time only to bound
    memory; each row's value is its own definition.
    """
    import torch

    k_idx = np.ascontiguousarray(k_idx, dtype=np.uint8)
    B, Lk, dI = k_idx.shape
    q_idx_rows = np.ascontiguousarray(q_idx_rows, dtype=np.uint8)
    R, HI, dI2 = q_idx_rows.shape
    assert dI2 == dI
    w_rows = np.ascontiguousarray(w_rows, dtype=np.float32)
    assert w_rows.shape == (R, HI)
    rb = np.asarray(row_batch, dtype=np.int64)
    rp = np.asarray(row_pos, dtype=np.int64)
    assert rb.shape == (R,) and rp.shape == (R,)
    assert (rb >= 0).all() and (rb < B).all() and (rp >= 0).all()
    if HI * dI > 8192 or not on_score_grid(q_idx_rows, k_idx, w_rows):
        raise ValueError("index_scores_blas is exact only on the 0.25-step grids with H_I * d_I <= 8192")
    table = torch.from_numpy(e4m3_to_float64(np.arange(256)))
    out = np.full((R, Lk), fill, dtype=np.float32)
    for b in np.unique(rb):
        keys = table[torch.from_numpy(k_idx[b].astype(np.int64))]                 # [Lk, dI]
        rows = np.nonzero(rb == b)[0]
        rows = rows[np.argsort(rp[rows], kind="stable")]
        for i0 in range(0, len(rows), rows_per_block):
            blk = rows[i0:i0 + rows_per_block]
            n = int(min(rp[blk].max() + 1, Lk))
            q = table[torch.from_numpy(q_idx_rows[blk].astype(np.int64))]         # [r, HI, dI]
            d = torch.from_numpy(q.reshape(-1, dI).numpy() @ keys[:n].numpy().T)  # [r*HI, n]
            d.clamp_(min=0.0)                                                      # ReLU
            wt = torch.from_numpy(w_rows[blk].astype(np.float64))[:, None, :]      # [r, 1, HI]
            score = torch.bmm(wt, d.view(len(blk), HI, n))[:, 0, :] + 0.0         # [r, n], -0 -> +0
            score = score.to(torch.float32).numpy()
            for j, r in enumerate(blk):
                m = int(min(rp[r] + 1, Lk))
                out[r, :m] = score[j, :m]
    return out


def topk(scores_rows, row_pos, k: int) -> np.ndarray:
    """Top-k selection per row over candidates s <= pos_r.

    Order (score desc, index asc): ties go to the lower index (reading: the
    pages do not say).  Output [R, k] int32 ascending, padded with -1 when the
    row has fewer than k candidates.
    """
    scores_rows, sp = _c(scores_rows, np.float32)
    R, Lk = scores_rows.shape
    rp, rpp = _c(row_pos, np.int32)
    assert rp.shape == (R,)
    out = np.empty((R, k), dtype=np.int32)
    lib().dsa_oracle_topk(Lk, k, R, rpp, sp, out.ctypes.data)
    return out


def sparse_mla_attn(kv, q_rows, indices, row_batch, d_latent: int, softmax_scale: float):
    """Sparse MQA-mode attention over the selected latents, in double precision.

    kv      [B, Lk, D_v + D_r] uint16 (bf16 bits)
    q_rows  [R, H, D_v + D_r] uint16 (bf16 bits)
    indices [R, k] int32 (entries outside [0, Lk) are skipped)
    Value = the first d_latent columns of each latent row (reading of
    "value dim taken from the latent").  Returns (out [R, H, D_v] float32,
    lse [R, H] float32).
    """
    kv = np.ascontiguousarray(kv, dtype=np.uint16)
    B, Lk, Dqk = kv.shape
    q_rows, qp = _c(q_rows, np.uint16)
    R, H, Dqk2 = q_rows.shape
    assert Dqk2 == Dqk and 0 < d_latent <= Dqk
    indices, ip = _c(indices, np.int32)
    assert indices.shape[0] == R
    k = indices.shape[1]
    rb, rbp = _c(row_batch, np.int32)
    assert (rb >= 0).all() and (rb < B).all()
    out = np.empty((R, H, d_latent), dtype=np.float32)
    lse = np.empty((R, H), dtype=np.float32)
    lib().dsa_oracle_sparse_mla_attn(Lk, H, d_latent, Dqk - d_latent, k, float(softmax_scale), R,
                                     rbp, qp, kv.ctypes.data, ip, out.ctypes.data, lse.ctypes.data)
    return out, lse


def sparse_mla_attn_bwd(kv, q_rows, indices, row_batch, dout_rows, d_latent: int,
                        softmax_scale: float, batch: int):
    """Gradients of sparse_mla_attn over fixed indices, in double precision.

    dout_rows [R, H, D_v] is the upstream gradient of the output.  Returns
    (dq [R, H, D_v + D_r] float64, dkv [batch, Lk, D_v + D_r] float64), dkv
    summed over the given rows only.  With o = sum_i p_i v_i: D = dout . o,
    dz_i = p_i (dout . v_i - D), dq = scale sum_i dz_i kv_i,
    dkv[s_i] += scale dz_i q + p_i dout (value columns)."""
    kv = np.ascontiguousarray(kv, dtype=np.uint16)
    B, Lk, Dqk = kv.shape
    assert batch == B
    q_rows, qp = _c(q_rows, np.uint16)
    R, H, Dqk2 = q_rows.shape
    assert Dqk2 == Dqk and 0 < d_latent <= Dqk
    indices, ip = _c(indices, np.int32)
    k = indices.shape[1]
    rb, rbp = _c(row_batch, np.int32)
    g, gp = _c(dout_rows, np.float64)
    assert g.shape == (R, H, d_latent) and indices.shape[0] == R
    dq = np.empty((R, H, Dqk), dtype=np.float64)
    dkv = np.zeros((B, Lk, Dqk), dtype=np.float64)
    lib().dsa_oracle_sparse_mla_attn_bwd(Lk, H, d_latent, Dqk - d_latent, k, float(softmax_scale), R,
                                         rbp, qp, kv.ctypes.data, ip, gp, dq.ctypes.data,
                                         dkv.ctypes.data)
    return dq, dkv


def warmup_target(kv, q_rows, row_batch, row_pos, softmax_scale: float, fill=np.nan) -> np.ndarray:
    """The dense warm-up's target distribution in double precision (DeepSeek-V3.2
    spec sheet, design overview: the main attention distribution summed over
    the heads): target[r, s] = mean over heads of the softmax over
    s' <= pos_r of softmax_scale * q . kv[s'], for s <= pos_r; `fill` after.
    kv [B, Lk, Dqk] bf16 bits, q_rows [R, H, Dqk] bf16 bits."""
    kv = np.ascontiguousarray(kv, dtype=np.uint16)
    B, Lk, Dqk = kv.shape
    q_rows, qp = _c(q_rows, np.uint16)
    R, H, Dqk2 = q_rows.shape
    assert Dqk2 == Dqk
    rb, rbp = _c(row_batch, np.int32)
    rpos, rpp = _c(row_pos, np.int32)
    assert rb.shape == (R,) and rpos.shape == (R,) and (rb >= 0).all() and (rb < B).all()
    assert (rpos >= 0).all()
    out = np.full((R, Lk), fill, dtype=np.float64)
    lib().dsa_oracle_warmup_target(Lk, H, Dqk, float(softmax_scale), R, rbp, rpp, qp, kv.ctypes.data,
                                   out.ctypes.data)
    return out


def warmup_kl(scores_rows, target_rows, row_pos, fill=np.nan):
    """KL(target || softmax(scores)) per row over s <= pos_r and its gradient
    with respect to the scores, softmax(scores) - target, in double precision
    (the dense warm-up's indexer objective).  scores_rows, target_rows [R, Lk]
    float32 (entries past pos_r are not read).  Returns (loss [R], dscores
    [R, Lk] with `fill` past pos_r)."""
    I, Ip = _c(scores_rows, np.float32)
    P, Pp = _c(target_rows, np.float32)
    R, Lk = I.shape
    assert P.shape == (R, Lk)
    rpos, rpp = _c(row_pos, np.int32)
    assert rpos.shape == (R,) and (rpos >= 0).all()
    loss = np.empty(R, dtype=np.float64)
    d = np.full((R, Lk), fill, dtype=np.float64)
    lib().dsa_oracle_warmup_kl(Lk, R, rpp, Ip, Pp, loss.ctypes.data, d.ctypes.data)
    return loss, d


def index_scores_bwd(k_idx, q_idx_rows, w_rows, row_batch, row_pos, dscores_rows):
    """Gradients of the indexer scores with respect to q_I, w and k_I for a
    gradient dscores_rows [R, Lk] of the scores (entries past pos_r unused), in
    double precision; the ReLU's derivative is taken as 0 at 0.  Returns
    (dq_idx [R, H_I, d_I], dw [R, H_I], dk_idx [B, Lk, d_I]); dk_idx sums the
    given rows only."""
    k_idx = np.ascontiguousarray(k_idx, dtype=np.uint8)
    B, Lk, dI = k_idx.shape
    q, qp = _c(q_idx_rows, np.uint8)
    R, HI, dI2 = q.shape
    assert dI2 == dI
    w, wp = _c(w_rows, np.float32)
    assert w.shape == (R, HI)
    rb, rbp = _c(row_batch, np.int32)
    rpos, rpp = _c(row_pos, np.int32)
    assert rb.shape == (R,) and rpos.shape == (R,) and (rb >= 0).all() and (rb < B).all()
    g, gp = _c(dscores_rows, np.float64)
    assert g.shape == (R, Lk)
    dq = np.empty((R, HI, dI), dtype=np.float64)
    dw = np.empty((R, HI), dtype=np.float64)
    dk = np.zeros((B, Lk, dI), dtype=np.float64)
    lib().dsa_oracle_index_scores_bwd(Lk, HI, dI, R, rbp, rpp, qp, wp, k_idx.ctypes.data, gp,
                                      dq.ctypes.data, dw.ctypes.data, dk.ctypes.data)
    return dq, dw, dk


def masked_mha_attn(kv, q_rows, indices, row_batch, row_pos, d_latent: int, softmax_scale: float):
    """Masked mode for short prefill, in double precision: dense causal attention
    over s = 0 .. pos with the tokens outside the row's indices masked to -inf
    (DeepSeek-V3.2 spec sheet, design overview and "Inference efficiency":
    a masked MHA mode simulating DSA for short-sequence prefill).  Arguments as
    for sparse_mla_attn plus row_pos [R]; entries outside [0, min(pos+1, Lk))
    are ignored and a listed token counts once.  Returns (out, lse)."""
    kv = np.ascontiguousarray(kv, dtype=np.uint16)
    B, Lk, Dqk = kv.shape
    q_rows, qp = _c(q_rows, np.uint16)
    R, H, Dqk2 = q_rows.shape
    assert Dqk2 == Dqk and 0 < d_latent <= Dqk
    indices, ip = _c(indices, np.int32)
    assert indices.shape[0] == R
    k = indices.shape[1]
    rb, rbp = _c(row_batch, np.int32)
    rpos, rpp = _c(row_pos, np.int32)
    assert (rb >= 0).all() and (rb < B).all() and rpos.shape == (R,) and (rpos >= 0).all()
    out = np.empty((R, H, d_latent), dtype=np.float32)
    lse = np.empty((R, H), dtype=np.float32)
    lib().dsa_oracle_masked_mha_attn(Lk, H, d_latent, Dqk - d_latent, k, float(softmax_scale), R,
                                     rbp, rpp, qp, kv.ctypes.data, ip, out.ctypes.data,
                                     lse.ctypes.data)
    return out, lse


def forward(k_idx, q_idx_rows, w_rows, q_rows, kv, row_batch, row_pos, k: int, d_latent: int,
            softmax_scale: float):
    """Indexer -> top-k -> sparse attention for the given rows.
    Returns dict(scores, indices, out, lse, seconds)."""
    t0 = time.perf_counter()
    s = index_scores(k_idx, q_idx_rows, w_rows, row_batch, row_pos)
    t1 = time.perf_counter()
    idx = topk(s, row_pos, k)
    t2 = time.perf_counter()
    out, lse = sparse_mla_attn(kv, q_rows, idx, row_batch, d_latent, softmax_scale)
    t3 = time.perf_counter()
    return dict(scores=s, indices=idx, out=out, lse=lse,
                seconds=dict(index=t1 - t0, topk=t2 - t1, attn=t3 - t2, total=t3 - t0))
