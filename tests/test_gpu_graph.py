"""The forward (dsa_forward) and the attention backward captured in one HIP
graph and replayed: every replay must reproduce the eager results (the
forward and dq bit for bit; dkv, whose per-token sums run in a varying order,
within 1e-5 of its scale).  The library enqueues kernels only (no memset, no
allocation); dkv is cleared inside the graph by a fill kernel.  The outputs
are overwritten between replays so that a replay that did nothing fails."""
import numpy as np
import pytest
import torch

import dsa_inputs
from gpu_util import Inputs, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dsa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_attention_02_amd as m
    return m


def test_forward_and_backward_replay_in_a_graph(dsa):
    wl = dsa_inputs.WORKLOADS["prefill4k"]
    inp = Inputs.make(wl)
    d = inp.device()
    prob = dsa.Problem.from_workload(wl)
    B, Lq, Lk, H = wl.batch, wl.q_len, wl.kv_len, wl.heads
    f32 = dict(dtype=torch.float32, device="cuda")
    out = torch.empty((B, Lq, H, wl.d_latent), **f32)
    lse = torch.empty((B, Lq, H), **f32)
    idx = torch.empty((B, Lq, wl.topk), dtype=torch.int32, device="cuda")
    fws_b = dsa.workspace_size(prob, dsa.DSA_OP_FORWARD)
    fws = torch.empty(fws_b, dtype=torch.uint8, device="cuda")
    g = torch.from_numpy(np.random.default_rng(4).normal(size=(B, Lq, H, wl.d_latent)).astype(np.float32)).cuda()
    dq = torch.empty((B, Lq, H, wl.d_qk), **f32)
    dkv = torch.empty((B, Lk, wl.d_qk), **f32)
    bws_b = dsa.workspace_size(prob, dsa.DSA_OP_SPARSE_MLA_ATTN_BWD)
    bws = torch.empty(bws_b, dtype=torch.uint8, device="cuda")

    def step():
        dsa.dsa_forward(prob, d["q_idx"], d["k_idx"], d["w"], d["q"], d["kv"], out, lse, idx, fws, fws_b)
        dkv.zero_()
        dsa.dsa_sparse_mla_attn_bwd(prob, d["q"], d["kv"], idx, out, lse, g, dq, dkv, bws, bws_b)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()  # eager, on the stream the capture will use
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    ref = [t.clone() for t in (out, lse, idx, dq, dkv)]

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for rep in range(3):
        for t in (out, lse, dq, dkv):
            t.fill_(float("nan"))  # eager work between replays
        idx.fill_(-7)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref[0]) and torch.equal(lse, ref[1]) and torch.equal(idx, ref[2]), rep
        assert torch.equal(dq, ref[3]), rep
        err = float((dkv - ref[4]).abs().max())
        scale = float(ref[4].abs().max())
        log(f"[graph replay {rep}] forward and dq identical; dkv max diff {err:.2e} of {scale:.2e}")
        assert err <= 1e-5 * scale, rep
    del graph
    torch.cuda.empty_cache()
