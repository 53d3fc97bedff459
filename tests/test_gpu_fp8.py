"""The FP8 format on the GPU: every finite OCP e4m3fn code through the indexer
and its backward, against the oracle.

The workload inputs all lie on the 0.25-step grid of [-4, 4]; these cases
drive the rest of the format (subnormals m * 2^-9, magnitudes up to 448, both
zeros) through the FP8 matrix cores of dsa_index_scores and the e4m3 -> bf16
conversion of dsa_index_scores_bwd.  The pages name only "FP8" for the
indexer ("DeepSeek V3.2 and the lightning indexer", "How the lightning
indexer works"); the reading taken is OCP e4m3fn with scale 1, and these tests
confirm the GPU reads the codes that way.

Exact cases: one-hot keys and one active indexer head per query (the others
weigh 0), with powers of two on the other side of every product, so every
score and every gradient element is a single exactly representable term and
the GPU must match the oracle bit for bit.  A dense random full-range case is
compared within an fp32 accumulation bound.
"""
import numpy as np
import pytest
import torch

import dsa_inputs
import oracle
from gpu_util import dev, log

pytestmark = pytest.mark.gpu

NAN_CODES = (0x7F, 0xFF)
FINITE = np.array([c for c in range(256) if c not in NAN_CODES], dtype=np.uint8)


@pytest.fixture(scope="module")
def dsa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_attention_02_amd as m
    return m


def e4m3_pow2(e: int, negative: bool = False) -> int:
    """The e4m3fn code of +-2^e, -9 <= e <= 8 (subnormal below 2^-6)."""
    assert -9 <= e <= 8
    code = (1 << (e + 9)) if e < -6 else ((e + 7) << 3)
    return code | (0x80 if negative else 0)


def exact_case():
    """Keys 0..255 are one-hot at d = s % 128 holding code s (NaN codes -> 0);
    keys 256..511 one-hot powers of two; keys 512..767 zero.  Query row t has
    one active head j = t % 64 with a power-of-two weight; its vector holds
    powers of two (rows < 128) or the codes d + 128*((t//64) % 2) (rows >= 128);
    the other heads hold random finite codes and weigh 0."""
    rng = np.random.default_rng(2024)
    HI, dI, Lq, Lk = 64, 128, 256, 768
    q_start = Lk - Lq
    k = np.zeros((1, Lk, dI), np.uint8)
    for s in range(256):
        k[0, s, s % dI] = 0 if s in NAN_CODES else s
    for s in range(256, 512):
        k[0, s, s % dI] = e4m3_pow2((s % 7) - 3, negative=(s // 7) % 2 == 1)
    q = rng.choice(FINITE, size=(Lq, HI, dI)).astype(np.uint8)
    w = np.zeros((Lq, HI), np.float32)
    for t in range(Lq):
        j = t % HI
        w[t, j] = np.float32(2.0 ** ((t % 5) - 2) * (-1 if t % 11 == 0 else 1))
        if t < 128:
            q[t, j] = [e4m3_pow2(((t + d) % 5) - 2, negative=(t + d) % 3 == 0) for d in range(dI)]
        else:
            codes = np.arange(dI) + 128 * ((t // 64) % 2)
            q[t, j] = np.where(np.isin(codes, NAN_CODES), 0, codes)
    wl = dsa_inputs.Workload("fp8codes", 0, 1, Lq, Lk, q_start, HI, dI, 64, 8, 64, 16)
    active_q = {int(c) for t in range(128, Lq) for c in q[t, t % HI]}
    active_k = {int(k[0, s, s % dI]) for s in range(256)}
    assert set(FINITE.tolist()) <= active_q, "every finite code on the query side"
    assert set(FINITE.tolist()) <= active_k, "every finite code on the key side"
    return wl, q, k, w


def _scores(dsa, wl, q, k, w):
    prob = dsa.Problem.from_workload(wl)
    scores = torch.full((1, wl.q_len, wl.kv_len), float("nan"), dtype=torch.float32, device="cuda")
    dsa.dsa_index_scores(prob, dev(q.reshape(1, wl.q_len, wl.idx_heads, wl.idx_dim)), dev(k),
                         dev(w.reshape(1, wl.q_len, wl.idx_heads)), scores)
    torch.cuda.synchronize()
    return scores[0].cpu().numpy()


def test_every_e4m3_code_through_the_indexer(dsa):
    wl, q, k, w = exact_case()
    log(f"[fp8 codes] indexer Lq={wl.q_len} Lk={wl.kv_len} H_I={wl.idx_heads} d_I={wl.idx_dim}")
    got = _scores(dsa, wl, q, k, w)
    rb, pos = dsa_inputs.row_batch_pos(wl, np.arange(wl.q_len))
    ref = oracle.index_scores(k, q, w, rb, pos)
    np.testing.assert_array_equal(got.view(np.uint32), ref.view(np.uint32))
    # the cases are not vacuous: many distinct non-zero scores of both signs
    nz = ref[np.isfinite(ref) & (ref != 0)]
    assert (nz > 0).sum() > 10000 and (nz < 0).sum() > 1000 and np.abs(nz).max() >= 100.0
    assert np.abs(nz).min() <= 2.0 ** -12
    log(f"[fp8 codes] {nz.size} non-zero scores bit-exact, |I| in [{np.abs(nz).min():.3g}, {np.abs(nz).max():.3g}]")


def test_random_full_range_codes_within_fp32_bound(dsa):
    """Dense random finite codes and random fp32 weights: the scores agree with
    the exact value within 2^-15 * A, A = sum_j |w_j| sum_d |q_jd k_sd| (the
    fp32 accumulation bound of a 128-term dot product followed by a 64-term
    weighted sum, with margin)."""
    rng = np.random.default_rng(77)
    HI, dI, Lq, Lk = 64, 128, 64, 600
    wl = dsa_inputs.Workload("fp8rand", 0, 1, Lq, Lk, Lk - Lq, HI, dI, 64, 8, 64, 16)
    q = rng.choice(FINITE, size=(Lq, HI, dI)).astype(np.uint8)
    k = rng.choice(FINITE, size=(1, Lk, dI)).astype(np.uint8)
    w = rng.uniform(-1, 1, size=(Lq, HI)).astype(np.float32)
    log(f"[fp8 random] indexer Lq={Lq} Lk={Lk}")
    got = _scores(dsa, wl, q, k, w)
    rb, pos = dsa_inputs.row_batch_pos(wl, np.arange(Lq))
    ref = oracle.index_scores(k, q, w, rb, pos).astype(np.float64)
    # |q| and |k| are the codes with the sign bit cleared; ReLU of a sum of
    # non-negative products is the sum itself
    A = oracle.index_scores(k & 0x7F, q & 0x7F, np.abs(w), rb, pos).astype(np.float64)
    causal = np.arange(Lk)[None, :] <= pos[:, None]
    err = np.abs(got.astype(np.float64) - ref)[causal]
    bound = (2.0 ** -15 * A)[causal] + 1e-30
    assert (err <= bound).all(), f"worst err/bound {np.max(err / bound):.3f}"
    assert np.isnan(got[~causal]).all()
    log(f"[fp8 random] max err/bound {np.max(err / bound):.3e}, max |I| {np.abs(ref[causal]).max():.3e}")


def test_every_e4m3_code_through_the_indexer_backward(dsa):
    """One non-zero score gradient per query row (at key s = t, a code key) makes
    every element of dw, dq_I and dk_I a single exact term."""
    wl, q, k, w = exact_case()
    Lq, Lk, HI, dI = wl.q_len, wl.kv_len, wl.idx_heads, wl.idx_dim
    rb, pos = dsa_inputs.row_batch_pos(wl, np.arange(Lq))
    g = np.zeros((Lq, Lk), np.float32)
    for t in range(Lq):
        g[t, t] = 2.0 ** ((t % 3) - 1) * (-1 if t % 4 == 1 else 1)
    g = np.where(np.arange(Lk)[None, :] > pos[:, None], np.nan, g).astype(np.float32)
    prob = dsa.Problem.from_workload(wl)
    dq = torch.full((1, Lq, HI, dI), float("nan"), dtype=torch.float32, device="cuda")
    dw = torch.full((1, Lq, HI), float("nan"), dtype=torch.float32, device="cuda")
    dk = torch.zeros((1, Lk, dI), dtype=torch.float32, device="cuda")
    log(f"[fp8 codes] indexer backward Lq={Lq} Lk={Lk}")
    dsa.dsa_index_scores_bwd(prob, dev(q.reshape(1, Lq, HI, dI)), dev(k), dev(w.reshape(1, Lq, HI)),
                             dev(g.reshape(1, Lq, Lk)), dq, dw, dk)
    torch.cuda.synchronize()
    dq_or, dw_or, dk_or = oracle.index_scores_bwd(k, q, w, rb, pos, np.nan_to_num(g.astype(np.float64)))
    for name, got, ref in [("dq_I", dq[0].cpu().numpy(), dq_or), ("dw", dw[0].cpu().numpy(), dw_or),
                           ("dk_I", dk[0].cpu().numpy(), dk_or[0])]:
        assert np.array_equal(ref, ref.astype(np.float32)), f"{name}: reference not exact in fp32"
        bad = got.astype(np.float64) != ref
        assert not bad.any(), f"{name}: {bad.sum()} elements differ, first at {np.argwhere(bad)[0]}"
    assert np.count_nonzero(dk_or) > 1000 and np.count_nonzero(dw_or) > 1000
    log(f"[fp8 codes] indexer backward exact: {np.count_nonzero(dq_or)} dq_I, {np.count_nonzero(dw_or)} dw, "
        f"{np.count_nonzero(dk_or)} dk_I non-zero elements")
