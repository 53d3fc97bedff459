"""dsa_index_topk on the GPU: the indexer and the top-k in one call.

For rows longer than 32768 keys in a multi-query problem the call scores a key
sample, takes a threshold per row from it, lets the indexer write only the
keys at or above it, and selects among those; rows whose candidates cannot be
trusted are redone through the full score row.  The bar is the one the
header states: indices bit-identical to dsa_index_scores followed by
dsa_topk, on every row, and equal to the oracle's selection (the indexer
ranking of "DeepSeek V3.2 and the lightning indexer", "How the lightning
indexer works", with the lower-index tie rule) on the rows checked there.

Cases:
  * crafted caches that defeat the sample: informative keys only off the
    sampled positions (the threshold is too low and the candidates overflow
    their slots), only on them (too high: fewer than k candidates), every
    key equal (every row one big tie), one sequence of two tied, and a cache
    longer than the last query position;
  * a prefill past 32K keys from position 0, whose first k rows select their
    whole prefix while the last ones have 33,000 keys;
  * the chunked prefill (8192 queries at positions 122880..131071) and the
    chunked prefill over a 1M-token context, every row, plus dsa_forward on
    the former against the three stages.
Each case prints its name and shape before it touches the GPU.
"""
import numpy as np
import pytest
import torch

import dsa_inputs
import oracle
from gpu_util import Inputs, dev, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dsa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_attention_02_amd as m
    return m


def unfused(dsa, prob, wl, d):
    """dsa_index_scores then dsa_topk; returns (scores, indices)."""
    scores = torch.full((wl.batch, wl.q_len, wl.kv_len), float("nan"), dtype=torch.float32, device="cuda")
    idx = torch.empty((wl.batch, wl.q_len, wl.topk), dtype=torch.int32, device="cuda")
    dsa.dsa_index_scores(prob, d["q_idx"], d["k_idx"], d["w"], scores)
    tws = dsa.workspace_size(prob, dsa.DSA_OP_TOPK)
    tw = torch.empty(max(tws, 1), dtype=torch.uint8, device="cuda")
    dsa.dsa_topk(prob, scores, idx, tw, tws)
    torch.cuda.synchronize()
    return scores, idx


def index_topk(dsa, prob, wl, d, fill=-7):
    ws_bytes = dsa.workspace_size(prob, dsa.DSA_OP_INDEX_TOPK)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    idx = torch.full((wl.batch, wl.q_len, wl.topk), fill, dtype=torch.int32, device="cuda")
    dsa.dsa_index_topk(prob, d["q_idx"], d["k_idx"], d["w"], idx, ws, ws_bytes)
    torch.cuda.synchronize()
    del ws
    return idx


def assert_same_rows(label, got, ref):
    g = got.reshape(got.shape[0] * got.shape[1], -1)
    r = ref.reshape(g.shape)
    bad = (g != r).any(-1)
    if bool(bad.any()):
        row = int(torch.nonzero(bad)[0])
        slot = int(torch.nonzero(g[row] != r[row])[0])
        raise AssertionError(f"{label}: {int(bad.sum())} rows differ from the unfused path; first row {row} "
                             f"slot {slot}: fused={int(g[row, slot])} unfused={int(r[row, slot])}")


def oracle_rows(label, inp, rows, idx):
    wl = inp.wl
    rows = np.asarray(rows, dtype=np.int64)
    flat = idx.reshape(-1, wl.topk)
    for i0 in range(0, len(rows), 8):
        r = rows[i0:i0 + 8]
        rb, pos = dsa_inputs.row_batch_pos(wl, r)
        s_or = oracle.index_scores_blas(inp.k_idx, inp.q_idx[r], inp.w[r], rb, pos)
        want = oracle.topk(s_or, pos, wl.topk)
        got = flat.index_select(0, torch.from_numpy(r).cuda()).cpu().numpy()
        for j in range(len(r)):
            if not np.array_equal(got[j], want[j]):
                slot = int(np.nonzero(got[j] != want[j])[0][0])
                raise AssertionError(f"{label}: row {r[j]} slot {slot}: gpu={got[j, slot]} "
                                     f"oracle={want[j, slot]}")


def crafted(name, seed, batch, q_len, kv_len, q_start, edit):
    wl = dsa_inputs.Workload(name, seed, batch, q_len, kv_len, q_start, 64, 128, 2048, 8, 64, 16)
    k = dsa_inputs.k_idx(wl).copy()
    edit(k)
    return Inputs(wl, k, dsa_inputs.q_idx(wl), dsa_inputs.w(wl), np.zeros(0, np.uint16), np.zeros(0, np.uint16))


def _off_sample(k):
    k[:, np.arange(k.shape[1]) % 16 == 0] = 0   # zero keys score exactly 0


def _on_sample(k):
    k[:, np.arange(k.shape[1]) % 16 != 0] = 0


def _all_equal(k):
    k[:, :] = k[:, 5:6]


def _one_tied(k):
    k[1, :] = k[1, 7]


CRAFTED = [
    ("informative keys off the sample", 51, 1, 64, 40000, 39936, _off_sample),
    ("informative keys on the sample", 52, 1, 64, 40000, 39936, _on_sample),
    ("every key equal", 53, 1, 64, 40000, 39936, _all_equal),
    ("one sequence tied", 54, 2, 40, 50000, 49960, _one_tied),
    ("cache longer than the queries", 55, 1, 96, 90000, 40000, lambda k: None),
]


@pytest.mark.timeout(300)
@pytest.mark.parametrize("case", CRAFTED, ids=[c[0] for c in CRAFTED])
def test_crafted_caches(dsa, case):
    label = case[0]
    inp = crafted(*case)
    wl = inp.wl
    assert min(wl.q_start + wl.q_len, wl.kv_len) > 32768, "long enough rows for the sampled path"
    log(f"[{label}] B={wl.batch} Lq={wl.q_len} Lk={wl.kv_len} q_start={wl.q_start}")
    d = dict(q_idx=dev(inp.q_idx), k_idx=dev(inp.k_idx), w=dev(inp.w))
    prob = dsa.Problem.from_workload(wl)
    got = index_topk(dsa, prob, wl, d)
    _, ref = unfused(dsa, prob, wl, d)
    assert_same_rows(label, got, ref)
    oracle_rows(label, inp, np.arange(wl.batch * wl.q_len), got)
    log(f"[{label}] all {wl.batch * wl.q_len} rows identical to the unfused path and the oracle")


@pytest.mark.timeout(600)
def test_prefill_past_32k_from_position_zero(dsa):
    """Rows of every length in one sampled-path call: the first k rows select
    their whole prefix (no threshold), the last ones have 33,000 keys."""
    wl = dsa_inputs.Workload("prefill33k", 56, 1, 33000, 33000, 0, 64, 128, 2048, 8, 64, 16)
    log(f"[prefill33k] B=1 Lq={wl.q_len} Lk={wl.kv_len} q_start=0")
    inp = Inputs(wl, dsa_inputs.k_idx(wl), dsa_inputs.q_idx(wl), dsa_inputs.w(wl),
                 np.zeros(0, np.uint16), np.zeros(0, np.uint16))
    d = dict(q_idx=dev(inp.q_idx), k_idx=dev(inp.k_idx), w=dev(inp.w))
    prob = dsa.Problem.from_workload(wl)
    plain = (4 * wl.q_len * wl.kv_len + 255) // 256 * 256 + dsa.workspace_size(prob, dsa.DSA_OP_TOPK)
    assert dsa.workspace_size(prob, dsa.DSA_OP_INDEX_TOPK) > plain, "the sampled path is taken"
    got = index_topk(dsa, prob, wl, d)
    torch.cuda.empty_cache()
    scores, ref = unfused(dsa, prob, wl, d)
    del scores
    torch.cuda.empty_cache()
    assert_same_rows("prefill33k", got, ref)
    rows = sorted({0, 1, 2046, 2047, 2048, 2049, 20000, 32767, 32768, 32999})
    oracle_rows("prefill33k", inp, rows, got)
    log(f"[prefill33k] every row identical to the unfused path; rows {rows} equal the oracle")


@pytest.mark.timeout(900)
def test_chunked_every_row_and_forward(dsa):
    wl = dsa_inputs.WORKLOADS["chunked"]
    log(f"[chunked] B={wl.batch} Lq={wl.q_len} Lk={wl.kv_len} q_start={wl.q_start}: inputs")
    inp = Inputs.make(wl)
    d = inp.device()
    prob = dsa.Problem.from_workload(wl)
    log("[chunked] dsa_index_topk and the unfused path")
    got = index_topk(dsa, prob, wl, d)
    scores, ref = unfused(dsa, prob, wl, d)
    del scores
    torch.cuda.empty_cache()
    assert_same_rows("chunked", got, ref)
    oracle_rows("chunked", inp, dsa_inputs.sample_rows(wl, 12), got)
    log("[chunked] every row identical to the unfused path; sampled rows equal the oracle")
    # dsa_forward runs the same selection, then the attention of the stages
    aws_bytes = dsa.workspace_size(prob, dsa.DSA_OP_SPARSE_MLA_ATTN)
    aws = torch.empty(aws_bytes, dtype=torch.uint8, device="cuda") if aws_bytes else None
    out = torch.empty((1, wl.q_len, wl.heads, wl.d_latent), dtype=torch.float32, device="cuda")
    lse = torch.empty((1, wl.q_len, wl.heads), dtype=torch.float32, device="cuda")
    log("[chunked] stages' attention and dsa_forward")
    dsa.dsa_sparse_mla_attn_ws(prob, d["q"], d["kv"], ref, out, lse, aws, aws_bytes)
    fws = torch.empty(dsa.workspace_size(prob, dsa.DSA_OP_FORWARD), dtype=torch.uint8, device="cuda")
    out_f, lse_f = torch.empty_like(out), torch.empty_like(lse)
    idx_f = torch.full_like(ref, -7)
    dsa.dsa_forward(prob, d["q_idx"], d["k_idx"], d["w"], d["q"], d["kv"], out_f, lse_f, idx_f, fws)
    torch.cuda.synchronize()
    assert torch.equal(idx_f, ref)
    assert torch.equal(out_f.view(torch.int32), out.view(torch.int32))
    assert torch.equal(lse_f.view(torch.int32), lse.view(torch.int32))
    log("[chunked] dsa_forward: indices, output and lse bit-identical to the stages")
    del fws, d
    torch.cuda.empty_cache()


@pytest.mark.timeout(900)
def test_chunked_1m_every_row(dsa):
    wl = dsa_inputs.WORKLOADS["chunked1m"]
    log(f"[chunked1m] B={wl.batch} Lq={wl.q_len} Lk={wl.kv_len} q_start={wl.q_start}: inputs")
    inp = Inputs(wl, dsa_inputs.k_idx(wl), dsa_inputs.q_idx(wl), dsa_inputs.w(wl),
                 np.zeros(0, np.uint16), np.zeros(0, np.uint16))
    d = dict(q_idx=dev(inp.q_idx), k_idx=dev(inp.k_idx), w=dev(inp.w))
    prob = dsa.Problem.from_workload(wl)
    log("[chunked1m] dsa_index_topk")
    got = index_topk(dsa, prob, wl, d)
    torch.cuda.empty_cache()
    log("[chunked1m] unfused path")
    scores, ref = unfused(dsa, prob, wl, d)
    del scores
    torch.cuda.empty_cache()
    assert_same_rows("chunked1m", got, ref)
    oracle_rows("chunked1m", inp, [0, 1, wl.q_len // 2, wl.q_len - 1], got)
    log("[chunked1m] every row identical to the unfused path; 4 rows equal the oracle")
    del d
    torch.cuda.empty_cache()
