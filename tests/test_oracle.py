"""Pins for the CPU oracle (no GPU needed).

Each test ties the oracle to something other than itself: a library routine
that a special case reduces to (torch's FP8 decode, matmul, relu, lexsort,
scaled_dot_product_attention, logsumexp), a closed form, or an invariant that
the definition implies.  Together they fix the whole formula: one-hot head
weights reduce the indexer to ReLU(matmul); linearity in the weights then fixes
the weighted head sum; the causal and top-k pins fix the candidate set and the
order; dense equivalence fixes attention when nothing is dropped.

Sources: "DeepSeek V3.2 and the lightning indexer" (section "How the lightning
indexer works", training section) and the DeepSeek-V3.2 spec sheet (design
overview, section 2.1, the training table's curriculum row).
"""
import math

import numpy as np
import pytest
import torch

import dsa_inputs
import oracle

RNG = np.random.default_rng


def enc_e4m3(vals) -> np.ndarray:
    """Encode exactly representable values with torch's own float8_e4m3fn cast."""
    t = torch.tensor(np.asarray(vals, dtype=np.float32)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy().copy()


def dec_e4m3_torch(codes) -> np.ndarray:
    t = torch.from_numpy(np.asarray(codes, dtype=np.uint8).copy()).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def grid(rng, shape, lo=-4.0, hi=4.0, step=0.25):
    n = int(round((hi - lo) / step)) + 1
    return lo + step * rng.integers(0, n, size=shape)


def bf16_bits(x) -> np.ndarray:
    t = torch.tensor(np.asarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def bf16_vals(bits) -> np.ndarray:
    t = torch.from_numpy(np.asarray(bits, dtype=np.uint16).view(np.int16).copy()).view(torch.bfloat16)
    return t.to(torch.float64).numpy()


# ---------------------------------------------------------------------------
# FP8 format
# ---------------------------------------------------------------------------

def test_e4m3_decode_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.e4m3_to_float64(codes)
    ref = dec_e4m3_torch(codes)
    nan = np.isnan(ref)
    assert (np.isnan(ours) == nan).all()
    assert nan.sum() == 2  # 0x7F and 0xFF
    np.testing.assert_array_equal(ours[~nan], ref[~nan])
    # sign of zero is kept by the decode itself
    assert math.copysign(1.0, ours[0x80]) == -1.0


def test_generator_grid_values_are_exact_grid_points():
    codes = dsa_inputs.e4m3_grid(7, dsa_inputs.TID_Q_IDX, 0, 200_000)
    vals = dec_e4m3_torch(codes)
    u = vals * 4 + 16
    assert np.all(u == np.round(u)) and u.min() == 0 and u.max() == 32
    hist = np.bincount(u.astype(int), minlength=33)
    exp = len(codes) / 33
    chi2 = ((hist - exp) ** 2 / exp).sum()
    assert chi2 < 80  # 32 dof; p ~ 1e-5
    w = dsa_inputs.f32_grid(7, dsa_inputs.TID_W, 0, 90_000, 9, -1.0, 0.25)
    uw = w * 4 + 4
    assert np.all(uw == np.round(uw)) and uw.min() == 0 and uw.max() == 8
    hist = np.bincount(uw.astype(int), minlength=9)
    chi2 = ((hist - 1e4) ** 2 / 1e4).sum()
    assert chi2 < 40


def test_generator_normal_moments_and_slices():
    x = bf16_vals(dsa_inputs.bf16_normal(3, dsa_inputs.TID_KV, 0, 400_000))
    assert abs(x.mean()) < 0.01 and abs(x.std() - 1) < 0.01
    # a slice equals the same range of the full tensor (counter-based)
    full = dsa_inputs.bf16_normal(3, dsa_inputs.TID_KV, 0, 1000)
    part = dsa_inputs.bf16_normal(3, dsa_inputs.TID_KV, 333, 500)
    np.testing.assert_array_equal(full[333:833], part)
    wl = dsa_inputs.WORKLOADS["tiny"]
    np.testing.assert_array_equal(dsa_inputs.q_idx(wl)[[5, 77]], dsa_inputs.q_idx(wl, rows=[5, 77]))
    np.testing.assert_array_equal(dsa_inputs.q(wl)[[0, 255]], dsa_inputs.q(wl, rows=[0, 255]))


# ---------------------------------------------------------------------------
# Lightning indexer
# ---------------------------------------------------------------------------

def _indexer_case(rng, R=6, Lk=40, HI=4, dI=32, qv=None, kv_=None, w=None):
    qv = grid(rng, (R, HI, dI)) if qv is None else qv
    kv_ = grid(rng, (1, Lk, dI)) if kv_ is None else kv_
    w = grid(rng, (R, HI), -1, 1) if w is None else w
    pos = np.full(R, Lk - 1, dtype=np.int32)
    rb = np.zeros(R, dtype=np.int32)
    return qv, kv_, np.asarray(w, np.float32), rb, pos


def _scores(qv, kv_, w, rb, pos):
    return oracle.index_scores(enc_e4m3(kv_), enc_e4m3(qv), w, rb, pos)


@pytest.mark.parametrize("sign", [1.0, -1.0, 0.5])
def test_indexer_one_hot_weight_is_relu_matmul(sign):
    """w = sign * e_j: I = sign * ReLU(q_j . k), compared with torch matmul + relu."""
    rng = RNG(1)
    R, Lk, HI, dI = 5, 33, 4, 32
    for j in range(HI):
        w = np.zeros((R, HI)); w[:, j] = sign
        qv, kv_, w32, rb, pos = _indexer_case(rng, R, Lk, HI, dI, w=w)
        got = _scores(qv, kv_, w32, rb, pos)
        ref = sign * torch.relu(torch.from_numpy(qv[:, j, :]) @ torch.from_numpy(kv_[0]).T).numpy()
        np.testing.assert_array_equal(got, ref.astype(np.float32))
        assert not np.signbit(got[got == 0]).any(), "zero scores must be +0"


def test_indexer_nonnegative_dots_are_plain_matmul():
    """q >= 0 and k >= 0 make every dot product >= 0, so ReLU is the identity and
    I = sum_j w_j (q_j . k) = (sum_j w_j q_j) . k  -- one matmul."""
    rng = RNG(2)
    R, Lk, HI, dI = 4, 24, 4, 32
    qv = grid(rng, (R, HI, dI), 0, 4)
    kv_ = grid(rng, (1, Lk, dI), 0, 4)
    w = grid(rng, (R, HI), -1, 1)
    got = _scores(qv, kv_, w.astype(np.float32), np.zeros(R, np.int32), np.full(R, Lk - 1, np.int32))
    qw = np.einsum("rj,rjd->rd", w, qv)
    ref = (torch.from_numpy(qw) @ torch.from_numpy(kv_[0]).T).numpy()
    np.testing.assert_array_equal(got, ref.astype(np.float32))


def test_indexer_linear_in_weights():
    """I(w1 + w2) = I(w1) + I(w2) exactly on the grid: the ReLU is applied to each
    head's dot product before weighting (not to the weighted sum)."""
    rng = RNG(3)
    qv, kv_, _, rb, pos = _indexer_case(rng, R=6, Lk=50, HI=4, dI=32)
    w1 = grid(rng, (6, 4), -0.5, 0.5).astype(np.float32)
    w2 = grid(rng, (6, 4), -0.5, 0.5).astype(np.float32)
    a = _scores(qv, kv_, w1, rb, pos)
    b = _scores(qv, kv_, w2, rb, pos)
    c = _scores(qv, kv_, w1 + w2, rb, pos)
    np.testing.assert_array_equal(c, a + b)
    # applying ReLU after the head sum would break this for mixed-sign heads
    assert (c != np.maximum(a + b, 0)).any() or (a + b >= 0).all()


def test_indexer_positive_homogeneity_and_zero_query():
    rng = RNG(4)
    qv, kv_, w, rb, pos = _indexer_case(rng, R=4, Lk=30)
    a = _scores(qv, kv_, w, rb, pos)
    b = _scores(2 * qv, kv_, w, rb, pos)  # |2q| <= 8 stays exact in e4m3
    np.testing.assert_array_equal(b, 2 * a)
    z = _scores(0 * qv, kv_, w, rb, pos)
    assert (z == 0).all() and not np.signbit(z).any()


def test_indexer_nonnegative_for_nonnegative_weights():
    rng = RNG(5)
    qv, kv_, _, rb, pos = _indexer_case(rng, R=8, Lk=64)
    w = grid(rng, (8, 4), 0, 1).astype(np.float32)
    s = _scores(qv, kv_, w, rb, pos)
    assert (s >= 0).all()


def test_indexer_causal_set_and_batch():
    """Only s <= pos is written (inclusive of the query's own token); each row
    reads its own sequence's keys."""
    rng = RNG(6)
    B, Lk, HI, dI = 3, 20, 4, 32
    kv_ = grid(rng, (B, Lk, dI))
    rows = [(0, 0), (1, 7), (2, 19), (1, 19)]
    rb = np.array([r[0] for r in rows], np.int32)
    pos = np.array([r[1] for r in rows], np.int32)
    qv = grid(rng, (len(rows), HI, dI))
    w = grid(rng, (len(rows), HI), -1, 1).astype(np.float32)
    s = oracle.index_scores(enc_e4m3(kv_), enc_e4m3(qv), w, rb, pos)
    for i, (b, p) in enumerate(rows):
        assert np.isfinite(s[i, : p + 1]).all()
        assert np.isnan(s[i, p + 1:]).all()
        one = oracle.index_scores(enc_e4m3(kv_[b:b + 1]), enc_e4m3(qv[i:i + 1]), w[i:i + 1],
                                  np.zeros(1, np.int32), np.array([p], np.int32))
        np.testing.assert_array_equal(one[0, : p + 1], s[i, : p + 1])
    # head permutation (q and w together) leaves the score unchanged
    perm = np.array([2, 0, 3, 1])
    s2 = oracle.index_scores(enc_e4m3(kv_), enc_e4m3(qv[:, perm]), w[:, perm], rb, pos)
    np.testing.assert_array_equal(np.nan_to_num(s2, nan=7.0), np.nan_to_num(s, nan=7.0))


def test_indexer_exact_on_grid_full_range():
    """Worst-case magnitudes on the grid (|q| = |k| = 4, d_I = 128, 64 heads,
    |w| = 1) stay exact: the fp32 output equals the exact integer sum."""
    R, Lk, HI, dI = 2, 3, 64, 128
    qv = np.full((R, HI, dI), 4.0); qv[1, ::2] = -4.0
    kv_ = np.full((1, Lk, dI), 4.0); kv_[0, 1, :] = -3.75; kv_[0, 2, ::3] = 0.25
    w = np.ones((R, HI), np.float32); w[1, 1::2] = -0.75
    s = _scores(qv, kv_, w, np.zeros(R, np.int32), np.full(R, Lk - 1, np.int32))
    assert s[0, 0] == 64 * 128 * 16  # 2^17
    # head sum of ReLU'd integer dot products, done with Python integers (x16 units)
    q16 = (qv * 4).astype(int); k16 = (kv_[0] * 4).astype(int)
    for r in range(R):
        for t in range(Lk):
            tot = 0
            for j in range(HI):
                dot = int(np.dot(q16[r, j], k16[t]))
                tot += int(w[r, j] * 4) * max(dot, 0)
            assert s[r, t] == tot / 64.0


# ---------------------------------------------------------------------------
# Top-k
# ---------------------------------------------------------------------------

def _lexsort_topk(row, n, k):
    idx = np.arange(n)
    order = np.lexsort((idx, -row[:n].astype(np.float64)))  # score desc, then index asc
    keep = np.sort(order[: min(k, n)])
    return np.concatenate([keep, -np.ones(k - len(keep), dtype=np.int64)])


def test_topk_matches_lexsort_with_heavy_ties():
    rng = RNG(7)
    R, Lk, k = 40, 300, 17
    scores = rng.integers(-5, 6, size=(R, Lk)).astype(np.float32)  # 11 values -> many ties
    pos = rng.integers(0, Lk, size=R).astype(np.int32)
    pos[:3] = [0, k - 1, k]
    got = oracle.topk(scores, pos, k)
    for r in range(R):
        np.testing.assert_array_equal(got[r], _lexsort_topk(scores[r], pos[r] + 1, k))


def test_topk_invariants_and_tie_rule():
    rng = RNG(8)
    R, Lk, k = 30, 500, 64
    scores = (rng.integers(0, 40, size=(R, Lk)) * 0.5).astype(np.float32)
    pos = rng.integers(k, Lk, size=R).astype(np.int32)
    idx = oracle.topk(scores, pos, k)
    for r in range(R):
        sel = idx[r]
        assert (np.diff(sel) > 0).all() and sel.min() >= 0 and sel.max() <= pos[r]
        rest = np.setdiff1d(np.arange(pos[r] + 1), sel)
        thr = scores[r, sel].min()
        assert thr >= scores[r, rest].max()
        tied_out = rest[scores[r, rest] == thr]
        tied_in = sel[scores[r, sel] == thr]
        if len(tied_out):
            assert tied_in.max() < tied_out.min(), "ties must go to the lower index"


def test_topk_short_rows_select_all_and_pad():
    scores = np.random.default_rng(9).normal(size=(3, 10)).astype(np.float32)
    pos = np.array([0, 4, 9], np.int32)
    idx = oracle.topk(scores, pos, 8)
    np.testing.assert_array_equal(idx[0], [0] + [-1] * 7)
    np.testing.assert_array_equal(idx[1], [0, 1, 2, 3, 4, -1, -1, -1])
    assert (idx[2] >= 0).all()


def test_topk_ignores_entries_after_pos_and_signed_zero_ties():
    scores = np.zeros((2, 6), np.float32)
    scores[0, 3:] = np.inf  # beyond pos: never read
    idx = oracle.topk(scores, np.array([2, 5], np.int32), 1)
    assert idx[0, 0] == 0
    s = np.array([[-0.0, 0.0, -1.0]], np.float32)
    idx = oracle.topk(s, np.array([2], np.int32), 1)
    assert idx[0, 0] == 0  # -0 == +0 as values; the lower index wins


# ---------------------------------------------------------------------------
# Sparse attention (MQA mode)
# ---------------------------------------------------------------------------

def _attn_case(rng, L=24, H=4, Dv=16, Dr=8):
    kv_ = bf16_bits(rng.normal(size=(1, L, Dv + Dr)))
    q_ = bf16_bits(rng.normal(size=(L, H, Dv + Dr)))
    return kv_, q_


def test_attention_equals_dense_causal_sdpa_when_nothing_is_dropped():
    """With k >= pos+1 for every row, the selection is the whole causal prefix and
    sparse MQA attention equals dense causal attention (torch SDPA, float64)."""
    rng = RNG(10)
    L, H, Dv, Dr, k = 24, 4, 16, 8, 32
    kv_, q_ = _attn_case(rng, L, H, Dv, Dr)
    idx = np.array([list(range(t + 1)) + [-1] * (k - t - 1) for t in range(L)], np.int32)
    scale = 1 / math.sqrt(Dv + Dr)
    out, lse = oracle.sparse_mla_attn(kv_, q_, idx, np.zeros(L, np.int32), Dv, scale)
    Q = torch.from_numpy(bf16_vals(q_)).permute(1, 0, 2)          # [H, L, D]
    K = torch.from_numpy(bf16_vals(kv_[0])).expand(H, L, Dv + Dr)  # shared by all heads
    V = K[..., :Dv]
    ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V, is_causal=True, scale=scale)
    np.testing.assert_allclose(out, ref.permute(1, 0, 2).numpy(), rtol=0, atol=2e-6)
    logits = (Q @ K.transpose(-1, -2)) * scale
    mask = torch.ones(L, L, dtype=torch.bool).triu(1)
    ref_lse = torch.logsumexp(logits.masked_fill(mask, -math.inf), dim=-1).T
    np.testing.assert_allclose(lse, ref_lse.numpy(), rtol=1e-6, atol=1e-6)


def test_attention_closed_forms():
    rng = RNG(11)
    L, H, Dv, Dr, k = 20, 3, 8, 4, 6
    kv_, q_ = _attn_case(rng, L, H, Dv, Dr)
    idx = np.stack([np.sort(rng.choice(L, size=k, replace=False)) for _ in range(4)]).astype(np.int32)
    rb = np.zeros(4, np.int32)
    # q = 0: uniform weights -> mean of the selected value rows
    zq = np.zeros((4, H, Dv + Dr), np.uint16)
    out, lse = oracle.sparse_mla_attn(kv_, zq, idx, rb, Dv, 0.3)
    V = bf16_vals(kv_[0])[:, :Dv]
    for r in range(4):
        np.testing.assert_allclose(out[r], np.broadcast_to(V[idx[r]].mean(0), (H, Dv)), atol=1e-6)
        np.testing.assert_allclose(lse[r], math.log(k), rtol=1e-6)
    # constant value columns -> that constant, whatever the scores
    kc = kv_.copy(); kc[0, :, :Dv] = bf16_bits(np.full((L, Dv), 1.5))
    out, _ = oracle.sparse_mla_attn(kc, q_[:4], idx, rb, Dv, 0.2)
    np.testing.assert_allclose(out, 1.5, rtol=1e-6)
    # a single selected token -> exactly its value row
    one = np.full((1, k), -1, np.int32); one[0, 0] = 0
    out, _ = oracle.sparse_mla_attn(kv_, q_[:1], one, rb[:1], Dv, 0.2)
    np.testing.assert_array_equal(out[0], np.broadcast_to(V[0].astype(np.float32), (H, Dv)))


def test_attention_index_order_and_invalid_entries():
    rng = RNG(12)
    L, H, Dv, Dr, k = 30, 2, 8, 8, 10
    kv_, q_ = _attn_case(rng, L, H, Dv, Dr)
    sel = np.sort(rng.choice(L, size=7, replace=False)).astype(np.int32)
    a = np.concatenate([sel, [-1, -1, -1]]).astype(np.int32)[None]
    b = np.concatenate([sel[::-1], [L + 5, -7, -1]]).astype(np.int32)[None]
    oa, la = oracle.sparse_mla_attn(kv_, q_[:1], a, np.zeros(1, np.int32), Dv, 0.25)
    ob, lb = oracle.sparse_mla_attn(kv_, q_[:1], b, np.zeros(1, np.int32), Dv, 0.25)
    np.testing.assert_allclose(oa, ob, rtol=1e-6, atol=1e-7)
    np.testing.assert_allclose(la, lb, rtol=1e-6)
    empty = np.full((1, k), -1, np.int32)
    oe, le = oracle.sparse_mla_attn(kv_, q_[:1], empty, np.zeros(1, np.int32), Dv, 0.25)
    assert (oe == 0).all() and np.isneginf(le).all()


def test_attention_value_is_latent_prefix_not_rope():
    """Changing only the rope columns of the cache, with q's rope part zero,
    leaves the output unchanged; changing latent columns changes it."""
    rng = RNG(13)
    L, H, Dv, Dr = 16, 2, 8, 8
    kv_, q_ = _attn_case(rng, L, H, Dv, Dr)
    q0 = q_.copy(); q0[:, :, Dv:] = 0
    idx = np.arange(L, dtype=np.int32)[None]
    o1, _ = oracle.sparse_mla_attn(kv_, q0[:1], idx, np.zeros(1, np.int32), Dv, 0.3)
    k2 = kv_.copy(); k2[0, :, Dv:] = bf16_bits(rng.normal(size=(L, Dr)) * 50)
    o2, _ = oracle.sparse_mla_attn(k2, q0[:1], idx, np.zeros(1, np.int32), Dv, 0.3)
    np.testing.assert_array_equal(o1, o2)
    k3 = kv_.copy(); k3[0, 3, 0] = bf16_bits([9.0])[0]
    o3, _ = oracle.sparse_mla_attn(k3, q0[:1], idx, np.zeros(1, np.int32), Dv, 0.3)
    assert not np.array_equal(o1, o3)


# Masked mode for short prefill (dense causal softmax with a selection mask)

def test_masked_mode_full_selection_is_dense_causal_sdpa():
    """Selecting every token of the causal prefix leaves nothing masked: the
    dense masked softmax is then dense causal attention (torch SDPA, float64)."""
    rng = RNG(14)
    L, H, Dv, Dr, k = 24, 4, 16, 8, 32
    kv_, q_ = _attn_case(rng, L, H, Dv, Dr)
    idx = np.array([list(range(t + 1)) + [-1] * (k - t - 1) for t in range(L)], np.int32)
    scale = 1 / math.sqrt(Dv + Dr)
    out, lse = oracle.masked_mha_attn(kv_, q_, idx, np.zeros(L, np.int32), np.arange(L, dtype=np.int32),
                                      Dv, scale)
    Q = torch.from_numpy(bf16_vals(q_)).permute(1, 0, 2)
    K = torch.from_numpy(bf16_vals(kv_[0])).expand(H, L, Dv + Dr)
    ref = torch.nn.functional.scaled_dot_product_attention(Q, K, K[..., :Dv], is_causal=True, scale=scale)
    np.testing.assert_allclose(out, ref.permute(1, 0, 2).numpy(), rtol=0, atol=2e-6)
    logits = (Q @ K.transpose(-1, -2)) * scale
    ref_lse = torch.logsumexp(logits.masked_fill(torch.ones(L, L, dtype=torch.bool).triu(1), -math.inf),
                              dim=-1).T
    np.testing.assert_allclose(lse, ref_lse.numpy(), rtol=1e-6, atol=1e-6)


def test_masked_mode_equals_sparse_on_topk_selections():
    """On selections made by the top-k (distinct, at or before pos(t)) the dense
    masked softmax and the sparse softmax over the selected latents are the same
    attention, computed two ways."""
    wl = dsa_inputs.WORKLOADS["tiny"]
    rows = np.arange(wl.q_len)
    rb, pos = dsa_inputs.row_batch_pos(wl, rows)
    qi = dsa_inputs.q_idx(wl).reshape(len(rows), wl.idx_heads, wl.idx_dim)
    s = oracle.index_scores(dsa_inputs.k_idx(wl), qi, dsa_inputs.w(wl).reshape(len(rows), -1), rb, pos)
    idx = oracle.topk(s, pos, wl.topk)
    kv_ = dsa_inputs.kv(wl)
    q_ = dsa_inputs.q(wl).reshape(len(rows), wl.heads, -1)
    o1, l1 = oracle.sparse_mla_attn(kv_, q_, idx, rb, wl.d_latent, wl.softmax_scale)
    o2, l2 = oracle.masked_mha_attn(kv_, q_, idx, rb, pos, wl.d_latent, wl.softmax_scale)
    np.testing.assert_allclose(o2, o1, rtol=0, atol=1e-6)
    np.testing.assert_allclose(l2, l1, rtol=1e-6, atol=1e-6)


def test_masked_mode_ignores_repeats_late_and_invalid_entries():
    rng = RNG(15)
    L, H, Dv, Dr, k = 30, 2, 8, 8, 12
    kv_, q_ = _attn_case(rng, L, H, Dv, Dr)
    pos = np.array([20], np.int32)
    sel = np.sort(rng.choice(21, size=6, replace=False)).astype(np.int32)
    clean = np.concatenate([sel, [-1] * (k - 6)]).astype(np.int32)[None]
    # the same tokens listed twice, plus entries past pos, past Lk and negative
    noisy = np.concatenate([sel[::-1], sel[:3], [25, L + 3, -4]]).astype(np.int32)[None]
    assert noisy.shape == (1, k)
    rb = np.zeros(1, np.int32)
    o1, l1 = oracle.sparse_mla_attn(kv_, q_[:1], clean, rb, Dv, 0.25)
    o2, l2 = oracle.masked_mha_attn(kv_, q_[:1], noisy, rb, pos, Dv, 0.25)
    np.testing.assert_allclose(o2, o1, rtol=0, atol=1e-6)
    np.testing.assert_allclose(l2, l1, rtol=1e-6)
    empty = np.full((1, k), -1, np.int32); empty[0, 0] = 25  # only a token past pos
    oe, le = oracle.masked_mha_attn(kv_, q_[:1], empty, rb, pos, Dv, 0.25)
    assert (oe == 0).all() and np.isneginf(le).all()


# Backward of the sparse attention over fixed indices

def _fwd_loss(qv, kvv, idx, g, Dv, scale):
    """sum(dout * out) of the forward definition, in float64 (for finite
    differences): per row and head, softmax over the listed entries."""
    R, H, _ = qv.shape
    tot = 0.0
    for r in range(R):
        sel = [s for s in idx[r] if 0 <= s < kvv.shape[0]]
        if not sel:
            continue
        K = kvv[sel]                                  # [n, Dqk]
        z = scale * (qv[r] @ K.T)                     # [H, n]
        z = z - z.max(1, keepdims=True)
        p = np.exp(z); p /= p.sum(1, keepdims=True)
        tot += float((g[r] * (p @ K[:, :Dv])).sum())
    return tot


def test_attention_backward_matches_finite_differences():
    """The analytic gradients against central differences of the forward
    definition (every q entry and every kv entry of a small case, with a
    repeated index and an invalid one)."""
    rng = RNG(16)
    L, H, Dv, Dr, k, R = 12, 3, 4, 4, 6, 3
    kv_ = bf16_bits(rng.normal(size=(1, L, Dv + Dr)))
    q_ = bf16_bits(rng.normal(size=(R, H, Dv + Dr)))
    idx = np.array([[0, 3, 5, 7, -1, 11], [2, 2, 9, 4, 1, 6], [10, 8, 0, 1, 5, L + 2]], np.int32)
    g = rng.normal(size=(R, H, Dv))
    scale = 0.7
    dq, dkv = oracle.sparse_mla_attn_bwd(kv_, q_, idx, np.zeros(R, np.int32), g, Dv, scale, 1)
    qv, kvv = bf16_vals(q_).astype(np.float64), bf16_vals(kv_[0]).astype(np.float64)
    eps = 1e-6
    num_q = np.zeros_like(qv)
    for i in np.ndindex(qv.shape):
        a = qv.copy(); a[i] += eps
        b = qv.copy(); b[i] -= eps
        num_q[i] = (_fwd_loss(a, kvv, idx, g, Dv, scale) - _fwd_loss(b, kvv, idx, g, Dv, scale)) / (2 * eps)
    num_kv = np.zeros_like(kvv)
    for i in np.ndindex(kvv.shape):
        a = kvv.copy(); a[i] += eps
        b = kvv.copy(); b[i] -= eps
        num_kv[i] = (_fwd_loss(qv, a, idx, g, Dv, scale) - _fwd_loss(qv, b, idx, g, Dv, scale)) / (2 * eps)
    np.testing.assert_allclose(dq, num_q, rtol=1e-6, atol=1e-8)
    np.testing.assert_allclose(dkv[0], num_kv, rtol=1e-6, atol=1e-8)
    assert (dkv[0, [s for s in range(L) if s not in idx]] == 0).all()  # unlisted rows get nothing


def test_attention_backward_closed_forms():
    rng = RNG(17)
    L, H, Dv, Dr, k = 10, 2, 4, 4, 5
    kv_ = bf16_bits(rng.normal(size=(1, L, Dv + Dr)))
    q_ = bf16_bits(rng.normal(size=(2, H, Dv + Dr)))
    g = rng.normal(size=(2, H, Dv))
    # one selected token: p = 1, so dz = 0: dq = 0 and dkv = dout on the value columns
    one = np.array([[4, -1, -1, -1, -1], [4, -1, -1, -1, -1]], np.int32)
    dq, dkv = oracle.sparse_mla_attn_bwd(kv_, q_, one, np.zeros(2, np.int32), g, Dv, 0.5, 1)
    assert (dq == 0).all()
    np.testing.assert_allclose(dkv[0, 4, :Dv], g.sum((0, 1)), rtol=1e-12)
    assert (dkv[0, 4, Dv:] == 0).all()
    # sum_i dz_i = 0: the rope columns (which only the scores reach) sum to zero over the keys
    idx = np.stack([rng.choice(L, size=k, replace=False) for _ in range(2)]).astype(np.int32)
    _, dkv = oracle.sparse_mla_attn_bwd(kv_, q_, idx, np.zeros(2, np.int32), g, Dv, 0.5, 1)
    np.testing.assert_allclose(dkv[0, :, Dv:].sum(0), 0.0, atol=1e-12)


# ---------------------------------------------------------------------------
# Dense warm-up objective
# ---------------------------------------------------------------------------

def test_warmup_target_is_head_mean_of_sdpa_weights():
    """With one-hot value columns the attention output of each head is its
    probability vector, so torch's SDPA (fp64, causal) gives the target as the
    mean of its outputs over the heads."""
    rng = RNG(20)
    L, H, Dr = 12, 3, 4
    onehot = np.eye(L)
    kvv = np.concatenate([onehot, rng.normal(size=(L, Dr))], axis=1)
    kv_ = bf16_bits(kvv)[None]
    q_ = bf16_bits(rng.normal(size=(L, H, L + Dr)))
    scale = 0.75  # exact in fp32, the type the oracle takes it in
    t = oracle.warmup_target(kv_, q_, np.zeros(L, np.int32), np.arange(L, dtype=np.int32), scale, fill=0.0)
    Q = torch.from_numpy(bf16_vals(q_)).permute(1, 0, 2)
    K = torch.from_numpy(bf16_vals(kv_[0])).expand(H, L, L + Dr)
    o = torch.nn.functional.scaled_dot_product_attention(Q, K, K[..., :L], is_causal=True, scale=scale)
    np.testing.assert_allclose(t, o.mean(0).numpy(), atol=1e-14, rtol=0)


def test_warmup_target_special_cases():
    rng = RNG(21)
    L, H, D = 9, 4, 8
    kv_ = bf16_bits(rng.normal(size=(1, L, D)))
    rb, pos = np.zeros(L, np.int32), np.arange(L, dtype=np.int32)
    # zero queries: uniform over the causal range
    t = oracle.warmup_target(kv_, np.zeros((L, H, D), np.uint16), rb, pos, 0.5, fill=0.0)
    for r in range(L):
        np.testing.assert_allclose(t[r, : r + 1], 1.0 / (r + 1), rtol=1e-15)
        assert (t[r, r + 1:] == 0).all()
    # identical heads: one head's softmax (torch, fp64)
    q1 = bf16_bits(rng.normal(size=(L, 1, D)))
    tq = oracle.warmup_target(kv_, np.repeat(q1, H, axis=1), rb, pos, 0.5, fill=0.0)
    z = 0.5 * bf16_vals(q1[:, 0]) @ bf16_vals(kv_[0]).T
    z = torch.from_numpy(z).masked_fill(torch.triu(torch.ones(L, L, dtype=torch.bool), 1), -math.inf)
    np.testing.assert_allclose(tq, torch.softmax(z, -1).numpy(), atol=1e-15)
    # rows sum to one; head order does not matter
    q_ = bf16_bits(rng.normal(size=(L, H, D)))
    t = oracle.warmup_target(kv_, q_, rb, pos, 0.5, fill=0.0)
    np.testing.assert_allclose(t.sum(1), 1.0, rtol=1e-14)
    tp = oracle.warmup_target(kv_, q_[:, ::-1], rb, pos, 0.5, fill=0.0)
    np.testing.assert_allclose(tp, t, rtol=1e-14, atol=1e-300)


def test_warmup_kl_matches_scipy_entropy_and_gradient():
    from scipy.special import rel_entr  # p log(p / q) termwise, 0 where p = 0, no renormalising
    rng = RNG(22)
    R, Lk = 5, 16
    pos = np.array([0, 3, 7, 15, 10], np.int32)
    I = rng.normal(size=(R, Lk)).astype(np.float32) * 3
    P = rng.random(size=(R, Lk)).astype(np.float32)
    P[1, 2] = 0.0  # a zero target entry contributes nothing
    for r in range(R):
        P[r, pos[r] + 1:] = 0
        P[r] /= P[r].sum()
    loss, d = oracle.warmup_kl(I, P, pos)
    for r in range(R):
        n = pos[r] + 1
        pi = torch.softmax(torch.from_numpy(I[r, :n].astype(np.float64)), 0).numpy()
        assert loss[r] == pytest.approx(rel_entr(P[r, :n].astype(np.float64), pi).sum(), rel=1e-12, abs=1e-15)
        np.testing.assert_allclose(d[r, :n], pi - P[r, :n], atol=1e-15)
        assert np.isnan(d[r, n:]).all()
        # softmax sums to one, so the gradient sums to 1 - sum(P) (P is fp32)
        assert d[r, :n].sum() == pytest.approx(1.0 - P[r, :n].astype(np.float64).sum(), abs=1e-14)
    assert loss[0] == 0.0 and (loss >= 0).all()
    # the gradient is the derivative of the loss (central differences)
    r, h = 3, 1e-3
    for s in range(pos[r] + 1):
        Ip, Im = I.copy(), I.copy()
        Ip[r, s] += h
        Im[r, s] -= h
        fd = (oracle.warmup_kl(Ip, P, pos)[0][r] - oracle.warmup_kl(Im, P, pos)[0][r]) / (float(Ip[r, s]) - float(Im[r, s]))
        assert fd == pytest.approx(d[r, s], abs=2e-6)


def test_warmup_kl_zero_at_match_and_shift_invariant():
    rng = RNG(23)
    R, Lk = 4, 12
    pos = np.full(R, Lk - 1, np.int32)
    I = rng.normal(size=(R, Lk)).astype(np.float32)
    P = torch.softmax(torch.from_numpy(I.astype(np.float64)), -1).numpy().astype(np.float32)
    loss, d = oracle.warmup_kl(I, P, pos)
    assert np.abs(loss).max() < 1e-7 and np.abs(d).max() < 1e-7  # P rounded to fp32
    P2 = rng.random(size=(R, Lk)).astype(np.float32)
    P2 /= P2.sum(1, keepdims=True)
    l1, d1 = oracle.warmup_kl(I, P2, pos)
    l2, d2 = oracle.warmup_kl(I + np.float32(5.0), P2, pos)
    np.testing.assert_allclose(l1, l2, rtol=1e-6)
    np.testing.assert_allclose(d1, d2, atol=1e-6)


def test_index_scores_bwd_matches_autograd():
    """dq_I, dw and dk_I against torch autograd of the indexer formula on the
    decoded values (fp64), with exact zeros of q.k on the grid (where the ReLU's
    derivative is 0 in both)."""
    rng = RNG(24)
    R, Lk, HI, dI = 6, 20, 4, 16
    qv = grid(rng, (R, HI, dI), -2, 2, 0.5)
    qv[0, 0] = 0.0  # u = 0 for a whole head
    kv_ = grid(rng, (2, Lk, dI), -2, 2, 0.5)
    w = grid(rng, (R, HI), -1, 1, 0.25).astype(np.float32)
    rb = np.array([0, 0, 1, 1, 0, 1], np.int32)
    pos = np.array([0, 5, 19, 11, 19, 3], np.int32)
    g = rng.normal(size=(R, Lk))
    dq, dw, dk = oracle.index_scores_bwd(enc_e4m3(kv_), enc_e4m3(qv), w, rb, pos, g)
    Q = torch.tensor(qv, dtype=torch.float64, requires_grad=True)
    K = torch.tensor(kv_, dtype=torch.float64, requires_grad=True)
    W = torch.tensor(w, dtype=torch.float64, requires_grad=True)
    u = torch.einsum("rjd,rsd->rjs", Q, K[torch.from_numpy(rb).long()])
    I = (W[..., None] * torch.relu(u)).sum(1)
    mask = torch.arange(Lk)[None, :] <= torch.from_numpy(pos)[:, None]
    (I * torch.from_numpy(g) * mask).sum().backward()
    np.testing.assert_allclose(dq, Q.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dw, W.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dk, K.grad.numpy(), atol=1e-12)
    assert (dq[0, 0] == 0).all()


# ---------------------------------------------------------------------------
# Whole path on the tiny workload
# ---------------------------------------------------------------------------

def test_forward_tiny_counts_and_dense_equivalence():
    wl = dsa_inputs.WORKLOADS["tiny"]
    rows = np.arange(wl.q_len)
    rb, pos = dsa_inputs.row_batch_pos(wl, rows)
    res = oracle.forward(dsa_inputs.k_idx(wl), dsa_inputs.q_idx(wl), dsa_inputs.w(wl),
                         dsa_inputs.q(wl), dsa_inputs.kv(wl), rb, pos, wl.topk, wl.d_latent,
                         wl.softmax_scale)
    idx = res["indices"]
    assert int((idx >= 0).sum()) == wl.selected_pairs()
    assert int(np.isfinite(res["scores"]).sum()) == wl.causal_pairs()
    # rows with pos + 1 <= k select their whole prefix -> dense causal attention there
    t = wl.topk - 1
    Q = torch.from_numpy(bf16_vals(dsa_inputs.q(wl)[: t + 1])).permute(1, 0, 2)
    K = torch.from_numpy(bf16_vals(dsa_inputs.kv(wl)[0, : t + 1])).expand(wl.heads, t + 1, wl.d_qk)
    ref = torch.nn.functional.scaled_dot_product_attention(
        Q, K, K[..., : wl.d_latent], is_causal=True, scale=wl.softmax_scale)
    np.testing.assert_allclose(res["out"][: t + 1], ref.permute(1, 0, 2).numpy(), atol=2e-6, rtol=0)


def test_workload_pair_counts_closed_form():
    """Pair counts used for the algorithmic FLOP/byte figures."""
    c = dsa_inputs.WORKLOADS
    assert c["prefill32k"].causal_pairs() == 32768 * 32769 // 2
    assert c["prefill32k"].selected_pairs() == 2048 * 2049 // 2 + (32768 - 2048) * 2048
    assert c["decode"].causal_pairs() == 64 * 131072
    assert c["decode"].selected_pairs() == 64 * 2048
    assert c["chunked"].causal_pairs() == sum(range(122881, 131073))
    assert c["tiny"].selected_pairs() == 64 * 65 // 2 + (256 - 64) * 64
    assert c["decode1m"].causal_pairs() == 4 * 2 ** 20
    assert c["decode1m"].selected_pairs() == 4 * 2048
    assert c["chunked1m"].causal_pairs() == sum(range(2 ** 20 - 4096 + 1, 2 ** 20 + 1))
    assert c["chunked1m"].selected_pairs() == 4096 * 2048
    assert c["prefill2k"].selected_pairs() == c["prefill2k"].causal_pairs() == 2048 * 2049 // 2


# ---------------------------------------------------------------------------
# The matrix-product evaluation of the indexer (for whole outputs at size)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name,rows", [("tiny", None), ("prefill4k", [0, 1, 2047, 2048, 3001, 4095]),
                                       ("chunked", [0, 4000, 8191])])
def test_indexer_blas_equals_the_c_definition_bit_for_bit(name, rows):
    """index_scores_blas evaluates the same definition with library products;
    on the workload grids it must equal the C oracle bit for bit, including
    the NaN fill past pos(t) and +0 for zero scores."""
    import torch  # noqa: F401  (the evaluation uses torch's CPU kernels)
    wl = dsa_inputs.WORKLOADS[name]
    rows = np.arange(wl.batch * wl.q_len) if rows is None else np.asarray(rows)
    rb, pos = dsa_inputs.row_batch_pos(wl, rows)
    k_idx = dsa_inputs.k_idx(wl)
    qi, w = dsa_inputs.q_idx(wl, rows), dsa_inputs.w(wl, rows)
    a = oracle.index_scores(k_idx, qi, w, rb, pos)
    b = oracle.index_scores_blas(k_idx, qi, w, rb, pos, rows_per_block=3)
    np.testing.assert_array_equal(a.view(np.uint32), b.view(np.uint32))
    assert (b.view(np.uint32) != 0x80000000).all()


def test_indexer_blas_extremes_ragged_heads_and_batches():
    """The largest magnitudes the grid allows (|I| = 2^17: every value +-4, every
    weight +-1), a ragged head count and width, two sequences with rows in
    shuffled order, and w < 0 against zero dot products (-0 terms)."""
    rng = RNG(5)
    B, Lk, HI, dI, R = 2, 70, 5, 96, 9
    k = grid(rng, (B, Lk, dI))
    k[0, :10] = 4.0
    k[1, 5] = 0.0
    q = grid(rng, (R, HI, dI))
    q[0] = 4.0
    w = grid(rng, (R, HI), -1, 1)
    w[0] = 1.0
    w[1] = -1.0
    rb = np.array([0, 1, 1, 0, 1, 0, 0, 1, 0], np.int32)
    pos = np.array([9, 69, 5, 0, 33, 69, 12, 40, 2], np.int32)
    a = oracle.index_scores(enc_e4m3(k), enc_e4m3(q), w.astype(np.float32), rb, pos)
    b = oracle.index_scores_blas(enc_e4m3(k), enc_e4m3(q), w.astype(np.float32), rb, pos)
    np.testing.assert_array_equal(a.view(np.uint32), b.view(np.uint32))
    assert a[0, 0] == 5 * 96 * 16.0  # five heads of 96 products of 4 * 4, weights 1


def test_indexer_blas_refuses_inputs_off_the_grid():
    rng = RNG(6)
    k = grid(rng, (1, 20, 32))
    q = grid(rng, (2, 4, 32))
    w = grid(rng, (2, 4), -1, 1).astype(np.float32)
    rb, pos = np.zeros(2, np.int32), np.array([10, 19], np.int32)
    for kk, qq, ww in [(k * 1.5, q, w), (k, q + 0.125, w), (k, q, w * 0.5 + 0.125), (k * 2, q, w)]:
        with pytest.raises(ValueError):
            oracle.index_scores_blas(enc_e4m3(kk), enc_e4m3(qq), ww.astype(np.float32), rb, pos)
