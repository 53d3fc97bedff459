"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Bar (from the workload definitions): indexer scores and top-k indices
bit-exact, sparse-attention output and log-sum-exp within max-abs 1e-2 (fp32).
The small and edge cases here are compared in full; the full-size workloads
are in test_gpu_full_outputs.py.
"""
import math

import numpy as np
import pytest
import torch

import dsa_inputs
import oracle
from gpu_util import Inputs, check_rows, dev, log, run_stages

pytestmark = pytest.mark.gpu

ATOL = 1e-2


@pytest.fixture(scope="module")
def dsa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_attention_02_amd as m
    return m


def _full_compare(dsa, wl, label):
    log(f"[{label}] shapes B={wl.batch} Lq={wl.q_len} Lk={wl.kv_len} q_start={wl.q_start} "
        f"HI={wl.idx_heads} dI={wl.idx_dim} k={wl.topk} H={wl.heads} Dv={wl.d_latent}+{wl.d_rope}")
    inp = Inputs.make(wl)
    d = inp.device()
    prob = dsa.Problem.from_workload(wl)
    sentinel = float("nan")
    scores, indices, out, lse = run_stages(prob, d, wl, fill_scores=sentinel)
    # entries after pos(t) are never written
    s = scores.cpu().numpy()
    pos = wl.q_start + np.arange(wl.q_len)
    after = np.arange(wl.kv_len)[None, :] > pos[:, None]
    assert np.isnan(s[:, after]).all(), "scores written past pos(t)"
    rows = np.arange(wl.batch * wl.q_len)
    err, lerr = check_rows(inp, rows, scores, indices, out, lse, ATOL, label)
    log(f"[{label}] all {len(rows)} rows: scores/indices exact, attn max-abs {err:.3e}, lse {lerr:.3e}")
    return inp, d, prob, scores, indices, out, lse


def test_tiny_full(dsa):
    wl = dsa_inputs.WORKLOADS["tiny"]
    inp, d, prob, scores, indices, out, lse = _full_compare(dsa, wl, "tiny")
    # dsa_forward == the three calls, bit for bit
    out2 = torch.empty_like(out)
    lse2 = torch.empty_like(lse)
    idx2 = torch.empty_like(indices)
    ws_bytes = dsa.workspace_size(prob, dsa.DSA_OP_FORWARD)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    dsa.dsa_forward(prob, d["q_idx"], d["k_idx"], d["w"], d["q"], d["kv"], out2, lse2, idx2, ws)
    torch.cuda.synchronize()
    assert torch.equal(idx2, indices)
    assert torch.equal(out2.view(torch.int32), out.view(torch.int32))
    assert torch.equal(lse2.view(torch.int32), lse.view(torch.int32))
    # forward without exporting indices
    out3 = torch.empty_like(out)
    dsa.dsa_forward(prob, d["q_idx"], d["k_idx"], d["w"], d["q"], d["kv"], out3, None, None, ws)
    torch.cuda.synchronize()
    assert torch.equal(out3.view(torch.int32), out.view(torch.int32))
    # a second run is bit-identical (no races)
    s2, i2, o2, l2 = run_stages(prob, d, wl, fill_scores=float("nan"))
    assert torch.equal(s2.view(torch.int32), scores.view(torch.int32))
    assert torch.equal(i2, indices) and torch.equal(o2.view(torch.int32), out.view(torch.int32))


EDGE = {
    # ragged everything: tails in query tiles, key stages, chunks of 32, heads
    "ragged": dsa_inputs.Workload("ragged", 11, 2, 77, 300, 223, 5, 64, 50, 20, 64, 16),
    "single_token": dsa_inputs.Workload("single", 12, 1, 1, 1, 0, 4, 32, 64, 8, 64, 16),
    "k_above_len": dsa_inputs.Workload("kbig", 13, 1, 40, 40, 0, 4, 32, 64, 8, 64, 16),
    "wide_indexer": dsa_inputs.Workload("wide", 14, 1, 130, 300, 170, 64, 96, 100, 16, 64, 16),
    "decode_small": dsa_inputs.Workload("dec", 15, 3, 1, 1000, 999, 64, 128, 128, 16, 64, 16),
    "few_queries": dsa_inputs.Workload("few", 16, 2, 5, 700, 695, 8, 128, 64, 24, 64, 16),
    "mla_small": dsa_inputs.Workload("mla", 17, 1, 200, 200, 0, 64, 128, 96, 128, 512, 64),
    # 100 of the 128 head slots: one 16-head tile part-filled, one absent
    "mla_partial_heads": dsa_inputs.Workload("mlah", 20, 1, 150, 180, 30, 64, 128, 96, 100, 512, 64),
    # long rows that the indexer splits over several blocks (prefill: 4 key
    # ranges of ~20 64-key stages; decode: 8 ranges of ~10 256-key stages),
    # each with a part-filled last stage
    "split_prefill": dsa_inputs.Workload("splitp", 18, 1, 12, 5000, 4988, 64, 128, 256, 16, 64, 16),
    "split_decode": dsa_inputs.Workload("splitd", 19, 2, 1, 20000, 19999, 64, 128, 256, 16, 64, 16),
}


@pytest.mark.parametrize("name", list(EDGE))
def test_edge_shapes_full(dsa, name):
    _full_compare(dsa, EDGE[name], name)


def test_topk_ties_and_signed_zero(dsa):
    """Heavy ties, exact zeros of both signs, and all-equal rows through dsa_topk."""
    rng = np.random.default_rng(3)
    B, Lq, Lk, k = 1, 300, 1500, 96
    wl = dsa_inputs.Workload("ties", 0, B, Lq, Lk, Lk - Lq, 4, 32, k, 8, 64, 16)
    s = rng.integers(-3, 4, size=(B, Lq, Lk)).astype(np.float32)
    s[s == 0] = np.where(rng.random(int((s == 0).sum())) < 0.5, -0.0, 0.0)
    s[0, :10] = 1.0  # all-equal rows
    prob = dsa.Problem.from_workload(wl)
    idx = torch.empty((B, Lq, k), dtype=torch.int32, device="cuda")
    dsa.dsa_topk(prob, dev(s), idx)
    torch.cuda.synchronize()
    pos = (wl.q_start + np.arange(Lq)).astype(np.int32)
    ref = oracle.topk(s.reshape(Lq, Lk), pos, k)
    np.testing.assert_array_equal(idx.cpu().numpy().reshape(Lq, k), ref)


@pytest.mark.parametrize("k", [2048, 64])
def test_topk_sampled_threshold_paths(dsa, k):
    """Rows of up to 32K candidates are first cut down with a threshold taken
    from a stride-16 sample; these rows drive every outcome of that step: the
    normal case, a sample that overshoots (fewer than k keys clear the
    threshold), one that undershoots (more keys than the candidate buffer),
    an all-equal row and heavy ties, each against the oracle."""
    rng = np.random.default_rng(11 + k)
    B, Lq, Lk = 1, 8, 20000
    q_start = Lk - Lq
    wl = dsa_inputs.Workload("sampled", 0, B, Lq, Lk, q_start, 4, 32, k, 8, 64, 16)
    s = rng.standard_normal((B, Lq, Lk)).astype(np.float32)       # row 0: normal path
    comb = (np.arange(Lk) % 16) == 0
    s[0, 1] = np.where(comb, 5.0 + rng.random(Lk), rng.random(Lk)).astype(np.float32)   # sample overshoots
    s[0, 2] = np.where(comb, rng.random(Lk), 5.0 + rng.random(Lk)).astype(np.float32)   # sample undershoots
    s[0, 3] = 1.5                                                   # all equal
    s[0, 4] = rng.integers(0, 3, Lk).astype(np.float32)            # three values, heavy ties
    s[0, 5] = (rng.integers(-20, 21, Lk) * 0.125).astype(np.float32)  # quantised
    s[0, 6, :] = -0.0                                               # signed zeros with a few spikes
    s[0, 6, rng.choice(Lk, 50, replace=False)] = 0.0
    s[0, 6, rng.choice(Lk, 30, replace=False)] = 2.0
    prob = dsa.Problem.from_workload(wl)
    ws_bytes = dsa.workspace_size(prob, dsa.DSA_OP_TOPK)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device="cuda")
    idx = torch.empty((B, Lq, k), dtype=torch.int32, device="cuda")
    dsa.dsa_topk(prob, dev(s), idx, ws, ws_bytes)
    torch.cuda.synchronize()
    pos = (q_start + np.arange(Lq)).astype(np.int32)
    ref = oracle.topk(np.ascontiguousarray(s[0]), pos, k)
    np.testing.assert_array_equal(idx.cpu().numpy()[0], ref)


@pytest.mark.parametrize("k,Lk,Lq", [(64, 40000, 6), (2048, 40000, 4), (100, 65536, 3),
                                     (64, 40000, 1024)])
def test_topk_two_stage_long_rows(dsa, k, Lk, Lq):
    """Rows longer than one block holds go through per-segment selection and a
    merge; quantised scores put ties across segment boundaries, one row ends
    exactly on a segment boundary and one just after it.  A few rows use 8K-key
    segments; 2048 rows (enough blocks) use 32K-key segments."""
    rng = np.random.default_rng(k + Lk + Lq)
    B = 2
    q_start = Lk - Lq
    wl = dsa_inputs.Workload("long", 0, B, Lq, Lk, q_start, 4, 32, k, 8, 64, 16)
    s = rng.integers(-40, 41, size=(B, Lq, Lk), dtype=np.int8).astype(np.float32) * 0.25
    s[0, 0, 8192 - 5:8192 + 5] = 10.0   # a tie straddling the first narrow segment boundary
    s[0, 1, 32768 - 5:32768 + 5] = 10.0  # ... and the first wide one
    s[1, -1, :] = 3.0                    # an all-equal row: the k lowest indices win
    prob = dsa.Problem.from_workload(wl)
    ws_bytes = dsa.workspace_size(prob, dsa.DSA_OP_TOPK)
    assert ws_bytes > 0
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    idx = torch.empty((B, Lq, k), dtype=torch.int32, device="cuda")
    dsa.dsa_topk(prob, dev(s), idx, ws, ws_bytes)
    torch.cuda.synchronize()
    pos = (q_start + np.arange(Lq)).astype(np.int32)
    got = idx.cpu().numpy()
    for b in range(B):
        ref = oracle.topk(np.ascontiguousarray(s[b]), pos, k)
        np.testing.assert_array_equal(got[b], ref)
    np.testing.assert_array_equal(got[1, -1], np.arange(k))


@pytest.mark.parametrize("Lk", [131072, 40001])
def test_topk_few_rows_cut_and_flagged_rows(dsa, Lk):
    """Few long rows are first selected from a cut taken on a sample of each
    row (the first 64 keys of every 1024): the keys at or above it are kept
    in 4096-key splits and selected exactly, and a row the cut cannot settle
    is flagged and redone in two stages.  Row 0 is random (settled by the
    cut); in row 1 the sampled keys are the row's lowest, so the cut lets
    nearly every key through and the splits overflow; in row 2 they are its
    highest, so fewer than k keys pass; row 3 is all equal.  Lk = 40001 also
    takes the scalar loads and a partial last run."""
    rng = np.random.default_rng(Lk)
    k, B, Lq = 2048, 4, 1
    q_start = Lk - 1
    wl = dsa_inputs.Workload("few", 0, B, Lq, Lk, q_start, 4, 32, k, 8, 64, 16)
    s = (rng.standard_normal((B, Lq, Lk)) * 100.0).astype(np.float32)
    sampled = (np.arange(Lk) % 1024) < 64
    ns = int(sampled.sum())
    s[1, 0, sampled] = (-1000.0 + rng.standard_normal(ns)).astype(np.float32)
    s[2, 0, sampled] = (1000.0 + rng.standard_normal(ns)).astype(np.float32)
    s[2, 0, ~sampled] = rng.standard_normal(Lk - ns).astype(np.float32)
    s[3] = 5.0
    prob = dsa.Problem.from_workload(wl)
    ws_bytes = dsa.workspace_size(prob, dsa.DSA_OP_TOPK)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    idx = torch.full((B, Lq, k), -7, dtype=torch.int32, device="cuda")
    log(f"[few rows] Lk={Lk} k={k} rows={B * Lq} workspace {ws_bytes} bytes")
    dsa.dsa_topk(prob, dev(s), idx, ws, ws_bytes)
    torch.cuda.synchronize()
    pos = (q_start + np.arange(Lq)).astype(np.int32)
    got = idx.cpu().numpy()
    for b in range(B):
        ref = oracle.topk(np.ascontiguousarray(s[b]), pos, k)
        np.testing.assert_array_equal(got[b], ref)
    np.testing.assert_array_equal(got[3, 0], np.arange(k))


def test_topk_two_stage_needs_workspace(dsa):
    wl = dsa_inputs.Workload("long", 0, 1, 2, 40000, 39998, 4, 32, 64, 8, 64, 16)
    prob = dsa.Problem.from_workload(wl)
    scores = torch.zeros((1, 2, 40000), dtype=torch.float32, device="cuda")
    idx = torch.empty((1, 2, 64), dtype=torch.int32, device="cuda")
    with pytest.raises(dsa.DsaError) as e:
        dsa.dsa_topk(prob, scores, idx)
    assert e.value.status == -4


def test_attention_split_matches_unsplit(dsa):
    """Few rows (decode-like): with a workspace each row's entries are split over
    several blocks and merged; the result matches the oracle and the unsplit path."""
    B, Lk, k = 6, 5000, 2048
    wl = dsa_inputs.Workload("split", 31, B, 1, Lk, Lk - 1, 4, 32, k, 128, 512, 64)
    inp = Inputs.make(wl)
    rng = np.random.default_rng(5)
    idx = np.full((B, 1, k), -1, np.int32)
    for b in range(B - 1):
        n = [k, 1500, 37, k, 900][b]
        idx[b, 0, :n] = np.sort(rng.choice(Lk, n, replace=False))
    # the last row has no valid entry
    prob = dsa.Problem.from_workload(wl)
    ws_bytes = dsa.workspace_size(prob, dsa.DSA_OP_SPARSE_MLA_ATTN)
    assert ws_bytes > 0
    d = inp.device()
    outs = []
    for use_ws in (True, False):
        out = torch.empty((B, 1, 128, 512), dtype=torch.float32, device="cuda")
        lse = torch.empty((B, 1, 128), dtype=torch.float32, device="cuda")
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda") if use_ws else None
        dsa.dsa_sparse_mla_attn_ws(prob, d["q"], d["kv"], dev(idx), out, lse, ws, ws_bytes if use_ws else 0)
        torch.cuda.synchronize()
        outs.append((out.cpu().numpy()[:, 0], lse.cpu().numpy()[:, 0]))
    rb = np.arange(B, dtype=np.int32)
    ref_o, ref_l = oracle.sparse_mla_attn(inp.kv, inp.q, idx[:, 0], rb, 512, wl.softmax_scale)
    for o, l in outs:
        assert np.abs(o - ref_o).max() <= ATOL
        fin = np.isfinite(ref_l)
        assert np.abs(l[fin] - ref_l[fin]).max() <= ATOL
        assert (o[-1] == 0).all() and np.isneginf(l[-1]).all()
    assert np.abs(outs[0][0] - outs[1][0]).max() <= 2e-3


def test_attention_invalid_entries_and_empty_rows(dsa):
    wl = dsa_inputs.Workload("inv", 21, 1, 6, 120, 114, 4, 32, 64, 16, 64, 16)
    inp = Inputs.make(wl)
    rng = np.random.default_rng(4)
    idx = np.full((1, 6, 64), -1, np.int32)
    idx[0, 0, :30] = np.sort(rng.choice(120, 30, replace=False))
    idx[0, 1, ::2] = rng.choice(120, 32, replace=False)        # unsorted, -1 in between
    idx[0, 2, :5] = [3, 500, -7, 119, 2 ** 30]                  # out-of-range entries skipped
    idx[0, 3, 40:] = np.arange(24)                              # only the last chunk valid
    idx[0, 5, 63] = 7                                           # one valid entry in the tail
    # row 4 stays all -1: out = 0, lse = -inf
    prob = dsa.Problem.from_workload(wl)
    d = inp.device()
    out = torch.empty((1, 6, 16, 64), dtype=torch.float32, device="cuda")
    lse = torch.empty((1, 6, 16), dtype=torch.float32, device="cuda")
    dsa.dsa_sparse_mla_attn(prob, d["q"], d["kv"], dev(idx), out, lse)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle.sparse_mla_attn(inp.kv, inp.q, idx[0], np.zeros(6, np.int32), 64,
                                          wl.softmax_scale)
    o = out.cpu().numpy()[0]
    l = lse.cpu().numpy()[0]
    assert np.abs(o - ref_o).max() <= ATOL
    assert (o[4] == 0).all() and np.isneginf(l[4]).all()
    fin = np.isfinite(ref_l)
    assert np.abs(l[fin] - ref_l[fin]).max() <= ATOL


def test_attention_dense_equivalence(dsa):
    """When every row keeps its whole causal prefix (pos+1 <= k), the sparse path is
    dense causal MQA attention: compare with torch SDPA in float64 on the CPU."""
    wl = dsa_inputs.Workload("dense", 22, 1, 64, 64, 0, 4, 32, 64, 32, 512, 64)
    inp = Inputs.make(wl)
    prob = dsa.Problem.from_workload(wl)
    _, indices, out, _ = run_stages(prob, inp.device(), wl)
    Q = torch.from_numpy(inp.q.view(np.int16).copy()).view(torch.bfloat16).double().permute(1, 0, 2)
    K = torch.from_numpy(inp.kv[0].view(np.int16).copy()).view(torch.bfloat16).double()
    K = K.expand(wl.heads, wl.kv_len, wl.d_qk)
    ref = torch.nn.functional.scaled_dot_product_attention(
        Q, K, K[..., : wl.d_latent], is_causal=True, scale=wl.softmax_scale)
    err = (out[0].cpu().double() - ref.permute(1, 0, 2)).abs().max().item()
    assert err <= ATOL, err


@pytest.mark.parametrize("k,Lk,Lq,B", [
    (50, 40000, 5, 2),       # k % 4 != 0: no segment plan; one block per row re-reads the row per pass
    (64, 40001, 6, 2),       # Lk % 4 != 0, few rows: 8K-key segments with scalar loads
    (64, 40001, 1024, 2),    # Lk % 4 != 0, many rows: 32K-key segments with scalar loads
    (2048, 1048580, 2, 1),   # over 2^20 candidates at k = 2048: no plan holds them, streamed rows
    (96, 5001, 40, 1),       # rows of <= 32K candidates with Lk % 4 != 0: registers, scalar loads
])
def test_topk_remaining_paths(dsa, k, Lk, Lq, B):
    """The selection paths the workloads do not reach, against the oracle, with
    quantised scores (ties everywhere, including across segment boundaries) and
    one all-equal row."""
    log(f"[topk paths] k={k} Lk={Lk} Lq={Lq} B={B}")
    rng = np.random.default_rng(k * 7 + Lk % 1000 + Lq)
    q_start = Lk - Lq
    wl = dsa_inputs.Workload("paths", 0, B, Lq, Lk, q_start, 4, 32, k, 8, 64, 16)
    s = (rng.integers(-60, 61, size=(B, Lq, Lk), dtype=np.int8).astype(np.float32) * 0.5)
    s[0, 0, 8190:8200] = 40.0
    s[-1, -1, :] = -0.0
    s[-1, -1, rng.choice(Lk, 7, replace=False)] = 0.0
    prob = dsa.Problem.from_workload(wl)
    ws_bytes = dsa.workspace_size(prob, dsa.DSA_OP_TOPK)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda") if ws_bytes else None
    idx = torch.empty((B, Lq, k), dtype=torch.int32, device="cuda")
    dsa.dsa_topk(prob, dev(s), idx, ws, ws_bytes)
    torch.cuda.synchronize()
    pos = (q_start + np.arange(Lq)).astype(np.int32)
    got = idx.cpu().numpy()
    for b in range(B):
        ref = oracle.topk(np.ascontiguousarray(s[b]), pos, k)
        np.testing.assert_array_equal(got[b], ref)
    np.testing.assert_array_equal(got[-1, -1], np.arange(k))


@pytest.mark.parametrize("shape", ["tiny", "mla"])
def test_attention_invalid_entries_masked_chunks_and_empty_rows(dsa, shape):
    """Hand-built selections through dsa_sparse_mla_attn at both latent shapes:
    -1 and out-of-range entries, unsorted lists, rows whose valid entries sit
    only in the last chunk (leading chunks wholly invalid), and an empty row."""
    if shape == "tiny":
        wl = dsa_inputs.Workload("inv_t", 23, 1, 6, 300, 294, 4, 32, 96, 16, 64, 16)
    else:
        wl = dsa_inputs.Workload("inv_m", 24, 1, 6, 300, 294, 4, 32, 96, 128, 512, 64)
    log(f"[invalid {shape}] H={wl.heads} Dv={wl.d_latent}+{wl.d_rope} k={wl.topk}")
    inp = Inputs.make(wl)
    rng = np.random.default_rng(4)
    k = wl.topk
    idx = np.full((1, 6, k), -1, np.int32)
    idx[0, 0, :70] = np.sort(rng.choice(300, 70, replace=False))
    idx[0, 1, ::3] = rng.choice(300, 32, replace=False)          # unsorted, -1 in between
    idx[0, 2, :6] = [3, 500, -7, 299, 2 ** 30, 0]                  # out-of-range entries skipped
    idx[0, 3, 64:] = np.arange(32)                                 # only the last chunk valid
    idx[0, 5, k - 1] = 7                                           # one valid entry in the tail
    # row 4 stays all -1: out = 0, lse = -inf
    prob = dsa.Problem.from_workload(wl)
    d = inp.device()
    out = torch.full((1, 6, wl.heads, wl.d_latent), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full((1, 6, wl.heads), float("nan"), dtype=torch.float32, device="cuda")
    dsa.dsa_sparse_mla_attn(prob, d["q"], d["kv"], dev(idx), out, lse)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle.sparse_mla_attn(inp.kv, inp.q, idx[0], np.zeros(6, np.int32), wl.d_latent,
                                          wl.softmax_scale)
    o = out.cpu().numpy()[0]
    l = lse.cpu().numpy()[0]
    assert np.abs(o - ref_o).max() <= ATOL
    assert (o[4] == 0).all() and np.isneginf(l[4]).all()
    fin = np.isfinite(ref_l)
    assert np.array_equal(fin, np.isfinite(l))
    assert np.abs(l[fin] - ref_l[fin]).max() <= ATOL


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def test_attention_score_range_far_above_the_first_chunk(dsa):
    """Late selected tokens whose scores exceed every earlier one by far more
    than 2^32 in probability (a latent row that is a large multiple of the
    query), at the MLA shape: the result must still be the softmax of the
    whole selection, for split and unsplit rows."""
    B, Lk, k = 3, 4000, 2048
    wl = dsa_inputs.Workload("range", 33, B, 1, Lk, Lk - 1, 4, 32, k, 128, 512, 64)
    log(f"[score range] B={B} Lk={Lk} k={k}")
    inp = Inputs.make(wl)
    kv = inp.kv.copy()
    q = inp.q.copy()
    rng = np.random.default_rng(8)
    idx = np.sort(np.stack([rng.choice(Lk, k, replace=False) for _ in range(B)]), axis=1).astype(np.int32)
    qv = torch.from_numpy(q.view(np.int16).copy()).view(torch.bfloat16).float()
    for b_ in range(B):
        # row b_: a selected token near the end aligned with head 5's query, 8x larger
        s_big = int(idx[b_, k - 40 + 10 * b_])
        kv[b_, s_big] = (8.0 * qv[b_, 5]).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    prob = dsa.Problem.from_workload(wl)
    kv_d = dev(kv)
    q_d = dev(q)
    ref_o, ref_l = oracle.sparse_mla_attn(kv, q, idx, np.arange(B, dtype=np.int32), 512, wl.softmax_scale)
    assert ref_l[:, 5].min() > 100.0  # the big score dominates head 5
    # The big token's value row is 8x a query row (|v| up to ~36), so the
    # absolute error that the rounding of the probabilities to bf16 for the
    # value product brings (relative 2^-9 each, 2^-8 allowed) grows with |v|:
    # per element, 2^-8 * sum_s p_s |v_sd| + 1e-3, p the exact probabilities.
    bound = np.empty_like(ref_o, dtype=np.float64)
    for b_ in range(B):
        sel = bf16_to_f64(kv[b_, idx[b_]])                      # [k, 576]
        z = wl.softmax_scale * (bf16_to_f64(q[b_]) @ sel.T)      # [H, k]
        pr = np.exp(z - ref_l[b_].astype(np.float64)[:, None])
        bound[b_] = 2.0 ** -8 * (pr @ np.abs(sel[:, :512])) + 1e-3
    ws_bytes = dsa.workspace_size(prob, dsa.DSA_OP_SPARSE_MLA_ATTN)
    for use_ws in (False, True):
        out = torch.empty((B, 1, 128, 512), dtype=torch.float32, device="cuda")
        lse = torch.empty((B, 1, 128), dtype=torch.float32, device="cuda")
        ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device="cuda")
        dsa.dsa_sparse_mla_attn_ws(prob, q_d, kv_d, dev(idx.reshape(B, 1, k)), out, lse, ws if use_ws else None,
                                   ws_bytes if use_ws else 0)
        torch.cuda.synchronize()
        o = out.cpu().numpy()[:, 0]
        l = lse.cpu().numpy()[:, 0]
        err = np.abs(o - ref_o)
        lerr = np.abs(l - ref_l).max()
        log(f"[score range] split={use_ws}: max-abs {err.max():.2e}, worst error/bound {(err / bound).max():.3f}, "
            f"lse {lerr:.2e} (lse up to {ref_l.max():.1f})")
        assert (err <= bound).all() and lerr <= ATOL * max(1.0, float(np.abs(ref_l).max()) / 100.0)
