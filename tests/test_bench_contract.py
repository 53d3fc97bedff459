"""The bench's contract on the host (no GPU): it refuses more than one GPU with
a message, and its algorithmic work figures (the numerators of every roofline
it reports) match the closed forms of the 32K prefill written out here from
the workload's sizes."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_algorithmic_work_of_the_32k_prefill():
    sys.path.insert(0, ROOT)
    import bench
    import dsa_inputs

    wl = dsa_inputs.WORKLOADS["prefill32k"]
    L, k, H, HI, dI = 32768, 2048, 128, 64, 128
    causal = L * (L + 1) // 2                       # every s <= t
    selected = k * (k + 1) // 2 + (L - k) * k       # min(t + 1, k) per row
    a = bench.algorithmic(wl)
    # indexer: one d_I-wide dot product per (pair, head), multiply-add = 2 flop
    assert a["index_scores"]["flop"] == 2 * HI * dI * causal
    # top-k: read the causal scores (fp32), write k int32 indices per row
    assert a["topk"]["bytes"] == 4 * causal + 4 * k * L
    # attention: per (selected pair, head) a 576-wide score and a 512-wide value product
    assert a["sparse_mla_attn"]["flop"] == 2 * H * (576 + 512) * selected
    # the gather: one 576-wide bf16 latent row per selected pair
    gather = 2 * 576 * selected
    assert a["sparse_mla_attn"]["bytes"] - gather == L * H * (2 * 576 + 4 * 512 + 4) + 4 * L * k
    assert a["masked_mha_attn"]["flop"] == 2 * H * (576 + 512) * causal


def test_end_to_end_ceiling_of_the_32k_prefill():
    """The step's ceiling is the sum of its kernels' roofline times: the indexer
    at the FP8 peak, the top-k at HBM bandwidth, the attention at the bf16 peak
    (its gather is served by the caches: the 38 MB latent cache fits them)."""
    sys.path.insert(0, ROOT)
    import bench
    import dsa_inputs

    wl = dsa_inputs.WORKLOADS["prefill32k"]
    a = bench.algorithmic(wl)
    L, k = 32768, 2048
    causal = L * (L + 1) // 2
    selected = k * (k + 1) // 2 + (L - k) * k
    t1 = 2 * 64 * 128 * causal / 5.0e15 * 1e3
    t2 = (4 * causal + 4 * k * L) / 8.0e12 * 1e3
    t3 = 2 * 128 * 1088 * selected / 2.5e15 * 1e3
    got = [bench.roofline_ms(n, a[n]) for n in ("index_scores", "topk", "sparse_mla_attn")]
    assert abs(got[0] - t1) < 1e-9 and abs(got[1] - t2) < 1e-9 and abs(got[2] - t3) < 1e-9
    assert 9.2 < sum(got) < 9.4
    # decode over 64 sequences: every gathered latent row comes from HBM
    dec = dsa_inputs.WORKLOADS["decode"]
    ad = bench.algorithmic(dec)
    assert ad["sparse_mla_attn"]["hbm_min_bytes"] == ad["sparse_mla_attn"]["bytes"]
