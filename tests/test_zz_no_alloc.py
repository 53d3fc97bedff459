"""dsa_forward_noalloc (the forward on the library's static scratch, for
callers that cannot allocate) against dsa_forward with a caller workspace,
through the C ABI: two calls in a row, the second on a smaller problem, each
bit-identical to dsa_forward (which the full-output tests hold to the oracle),
plus the oracle itself on a few rows of the second; and the size limit."""
import numpy as np
import pytest
import torch

import dsa_inputs
import oracle
from gpu_util import Inputs, log

pytestmark = pytest.mark.gpu

SCRATCH_BYTES = 128 << 20


@pytest.fixture(scope="module")
def dsa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_attention_02_amd as m
    return m


def _outputs(wl):
    B, Lq = wl.batch, wl.q_len
    out = torch.full((B, Lq, wl.heads, wl.d_latent), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full((B, Lq, wl.heads), float("nan"), dtype=torch.float32, device="cuda")
    idx = torch.full((B, Lq, wl.topk), -7, dtype=torch.int32, device="cuda")
    return out, lse, idx


def _both(dsa, wl, export_indices=True):
    log(f"[no-alloc] {wl.name}: B={wl.batch} Lq={wl.q_len} Lk={wl.kv_len} k={wl.topk}")
    inp = Inputs.make(wl)
    d = inp.device()
    prob = dsa.Problem.from_workload(wl)
    need = dsa.workspace_size(prob, dsa.DSA_OP_FORWARD)
    assert need <= SCRATCH_BYTES
    o1, l1, i1 = _outputs(wl)
    o2, l2, i2 = _outputs(wl)
    dsa.dsa_forward_noalloc(prob, d["q_idx"], d["k_idx"], d["w"], d["q"], d["kv"], o1, l1,
                            i1 if export_indices else None)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    dsa.dsa_forward(prob, d["q_idx"], d["k_idx"], d["w"], d["q"], d["kv"], o2, l2, i2, ws)
    torch.cuda.synchronize()
    if export_indices:
        assert torch.equal(i1, i2), "indices differ from dsa_forward"
    assert torch.equal(o1.view(torch.int32), o2.view(torch.int32)), "output differs from dsa_forward"
    assert torch.equal(l1.view(torch.int32), l2.view(torch.int32)), "lse differs from dsa_forward"
    log(f"[no-alloc] {wl.name}: bit-identical to dsa_forward (workspace {need} bytes)")
    return inp, o1, l1, i2


def test_forward_noalloc_two_calls_then_smaller(dsa):
    big = dsa_inputs.WORKLOADS["decode"]
    small = dsa_inputs.Workload("decode_small_mla", 41, 8, 1, 20000, 19999, 64, 128, 2048, 128, 512, 64)
    _both(dsa, big)
    inp, out, lse, idx = _both(dsa, small)
    _both(dsa, small, export_indices=False)
    # the oracle on four rows of the smaller call
    rows = np.array([0, 3, 5, 7])
    rb, pos = dsa_inputs.row_batch_pos(small, rows)
    ref = oracle.forward(inp.k_idx, inp.q_idx[rows], inp.w[rows], inp.q[rows], inp.kv, rb, pos, small.topk,
                         small.d_latent, small.softmax_scale)
    np.testing.assert_array_equal(idx.reshape(-1, small.topk).cpu().numpy()[rows], ref["indices"])
    err = np.abs(out.reshape(-1, small.heads, small.d_latent).cpu().numpy()[rows] - ref["out"]).max()
    lerr = np.abs(lse.reshape(-1, small.heads).cpu().numpy()[rows] - ref["lse"]).max()
    assert err <= 1e-2 and lerr <= 1e-2, (err, lerr)
    log(f"[no-alloc] oracle rows {rows.tolist()}: indices exact, attention max-abs {err:.2e}")


def test_forward_noalloc_sampled_selection(dsa):
    """A prefill-shaped problem with rows past 32K keys: the forward's
    selection takes the sampled path (the indexer writes only candidate
    keys), here inside the static scratch."""
    wl = dsa_inputs.Workload("long_rows_mla", 42, 1, 64, 40000, 39936, 64, 128, 2048, 128, 512, 64)
    prob = dsa.Problem.from_workload(wl)
    plain = (4 * wl.q_len * wl.kv_len + 255) // 256 * 256 + dsa.workspace_size(prob, dsa.DSA_OP_TOPK)
    assert dsa.workspace_size(prob, dsa.DSA_OP_INDEX_TOPK) > plain, "the sampled path is taken"
    inp, out, lse, idx = _both(dsa, wl)
    rows = np.array([0, 31, 63])
    rb, pos = dsa_inputs.row_batch_pos(wl, rows)
    ref = oracle.forward(inp.k_idx, inp.q_idx[rows], inp.w[rows], inp.q[rows], inp.kv, rb, pos, wl.topk,
                         wl.d_latent, wl.softmax_scale)
    np.testing.assert_array_equal(idx.reshape(-1, wl.topk).cpu().numpy()[rows], ref["indices"])
    err = np.abs(out.reshape(-1, wl.heads, wl.d_latent).cpu().numpy()[rows] - ref["out"]).max()
    assert err <= 1e-2, err
    log(f"[no-alloc] sampled selection: oracle rows {rows.tolist()} indices exact, attention max-abs {err:.2e}")


def test_forward_noalloc_rejects_problems_beyond_the_scratch(dsa):
    wl = dsa_inputs.WORKLOADS["prefill32k"]
    prob = dsa.Problem.from_workload(wl)
    assert dsa.workspace_size(prob, dsa.DSA_OP_FORWARD) > SCRATCH_BYTES
    fake = 1 << 20  # never dereferenced: the size check comes before any launch
    with pytest.raises(dsa.DsaError) as e:
        dsa.dsa_forward_noalloc(prob, fake, fake, fake, fake, fake, fake, None, None, stream=0)
    assert e.value.status == -3 and "static scratch" in str(e.value)
