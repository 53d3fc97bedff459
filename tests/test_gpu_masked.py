"""GPU parity of the masked mode for short prefill (dense causal attention with
the non-selected tokens masked) against the CPU oracle's dense masked softmax,
and against the sparse kernel on the same selections.

Bar: max-abs 1e-2 on out and lse (fp32), as for the sparse attention."""
import numpy as np
import pytest
import torch

import dsa_inputs
import oracle
from gpu_util import Inputs, dev, log, run_stages
from test_gpu_parity import EDGE

pytestmark = pytest.mark.gpu

ATOL = 1e-2


@pytest.fixture(scope="module")
def dsa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_attention_02_amd as m
    return m


def _masked(dsa, prob, wl, d, indices):
    out = torch.full((wl.batch, wl.q_len, wl.heads, wl.d_latent), float("nan"), dtype=torch.float32,
                     device="cuda")
    lse = torch.full((wl.batch, wl.q_len, wl.heads), float("nan"), dtype=torch.float32, device="cuda")
    dsa.dsa_masked_mha_attn(prob, d["q"], d["kv"], indices, out, lse)
    torch.cuda.synchronize()
    return out, lse


def _compare(inp, wl, rows, indices_np, out, lse, label):
    rb, pos = dsa_inputs.row_batch_pos(wl, rows)
    q_rows = inp.q.reshape(wl.batch * wl.q_len, wl.heads, -1)[rows]
    o_or, l_or = oracle.masked_mha_attn(inp.kv, q_rows, indices_np[rows], rb, pos, wl.d_latent,
                                        wl.softmax_scale)
    o_gpu = out.reshape(-1, wl.heads, wl.d_latent)[torch.from_numpy(rows).cuda()].cpu().numpy()
    l_gpu = lse.reshape(-1, wl.heads)[torch.from_numpy(rows).cuda()].cpu().numpy()
    err = float(np.abs(o_gpu - o_or).max())
    fin = np.isfinite(l_or)
    assert np.array_equal(fin, np.isfinite(l_gpu)), f"{label}: lse finiteness differs"
    lerr = float(np.abs(l_gpu[fin] - l_or[fin]).max()) if fin.any() else 0.0
    log(f"[{label}] masked mode, {len(rows)} rows: out max-abs {err:.3e}, lse {lerr:.3e}")
    assert err <= ATOL and lerr <= ATOL, f"{label}: out {err}, lse {lerr}"


@pytest.mark.parametrize("name", ["tiny", "ragged", "single_token", "k_above_len", "mla_small",
                                  "mla_partial_heads", "decode_small", "few_queries", "split_prefill"])
def test_masked_mode_matches_oracle(dsa, name):
    wl = dsa_inputs.WORKLOADS[name] if name in dsa_inputs.WORKLOADS else EDGE[name]
    log(f"[{name}] B={wl.batch} Lq={wl.q_len} Lk={wl.kv_len} q_start={wl.q_start} k={wl.topk} "
        f"H={wl.heads} Dv={wl.d_latent}+{wl.d_rope}")
    inp = Inputs.make(wl)
    d = inp.device()
    prob = dsa.Problem.from_workload(wl)
    _, indices, out_s, lse_s = run_stages(prob, d, wl)
    out, lse = _masked(dsa, prob, wl, d, indices)
    rows = np.arange(wl.batch * wl.q_len)
    _compare(inp, wl, rows, indices.reshape(-1, wl.topk).cpu().numpy(), out, lse, name)
    # The sparse kernel on the same selection computes the same attention.  Both
    # round P to bf16 against a running maximum that moves at different chunks,
    # so outputs agree to the attention bar, not bit for bit; lse comes from the
    # unrounded fp32 sums and agrees more closely.
    assert float((out - out_s).abs().max()) <= ATOL
    fin = torch.isfinite(lse_s)
    assert torch.equal(fin, torch.isfinite(lse)) and float((lse - lse_s)[fin].abs().max()) <= 1e-3


def test_masked_mode_leading_masked_chunks_and_noisy_entries(dsa):
    """Selections built by hand: rows whose first selected token lies many chunks
    in (every score of the leading chunks is masked), rows with repeated entries,
    entries past pos(t), past the cache and negative, and a row with nothing
    selected."""
    wl = dsa_inputs.Workload("maskhand", 21, 2, 6, 700, 694, 4, 32, 40, 16, 64, 16)
    inp = Inputs.make(wl)
    d = inp.device()
    prob = dsa.Problem.from_workload(wl)
    rng = np.random.default_rng(5)
    R = wl.batch * wl.q_len
    _, pos = dsa_inputs.row_batch_pos(wl, np.arange(R))
    idx = np.full((R, wl.topk), -1, np.int32)
    for r in range(R):
        p = int(pos[r])
        if r == 0:
            sel = np.arange(p - 4, p + 1)                       # only the last 5 tokens
        elif r == 1:
            sel = np.array([p])                                  # only the diagonal
        elif r == 2:
            sel = np.array([], np.int64)                         # nothing selected
        else:
            sel = np.sort(rng.choice(p + 1, size=20, replace=False))
        extra = []
        if r % 3 == 0 and len(sel):
            extra = [sel[0], sel[-1], p + 1, wl.kv_len + 9, -3]  # repeats, late, out of range
        row = np.concatenate([sel, extra]).astype(np.int32)
        idx[r, :len(row)] = row
    indices = dev(idx.reshape(wl.batch, wl.q_len, wl.topk))
    out, lse = _masked(dsa, prob, wl, d, indices)
    _compare(inp, wl, np.arange(R), idx, out, lse, "maskhand")
    assert bool((out.reshape(R, wl.heads, -1)[2] == 0).all())
    assert bool(torch.isneginf(lse.reshape(R, wl.heads)[2]).all())


@pytest.mark.parametrize("name", ["prefill2k", "prefill4k"])
def test_masked_mode_prefill_sampled(dsa, name):
    """The 2K and 4K prefill workloads: masked and sparse kernels on the
    pipeline's own selection, every row, plus the oracle on sampled rows."""
    wl = dsa_inputs.WORKLOADS[name]
    inp = Inputs.make(wl)
    d = inp.device()
    prob = dsa.Problem.from_workload(wl)
    _, indices, out_s, lse_s = run_stages(prob, d, wl)
    out, lse = _masked(dsa, prob, wl, d, indices)
    diff = float((out - out_s).abs().max())
    ldiff = float((lse - lse_s).abs().max())
    log(f"[{name}] masked vs sparse, all rows: out max-abs {diff:.3e}, lse {ldiff:.3e}")
    assert diff <= ATOL and ldiff <= 1e-3
    rows = np.array([0, 1, 1023, 2046, 2047, wl.q_len - 1])
    _compare(inp, wl, rows, indices.reshape(-1, wl.topk).cpu().numpy(), out, lse, name)
