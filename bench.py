"""Benchmark of the DeepSeek Sparse Attention hot path on one MI355X.

One step = one pass of the whole path over the L=32K prefill workload (batch 1,
32768 query tokens, k=2048, FP8 indexer 64 heads x 128, 128 query heads,
576-wide bf16 latents): dsa_index_topk -> dsa_sparse_mla_attn, launched back
to back on one stream (the launches dsa_forward makes), with HIP events
around each call.  dsa_index_topk is the indexer followed by the top-k (for
rows past 32K keys, the sampled path that writes only candidate keys).
After the timed steps, dsa_index_scores and dsa_topk are timed on their own
(a few calls, events between them, each pair followed by the attention as in
a step) for the indexer's and the top-k's per-kernel figures.  Inputs are seeded, synthetic and resident in HBM before
timing starts.  --workload picks another of the seeded workloads.

Prints one JSON line: query tokens/s, per-kernel times and rooflines, and the
CPU oracle timed on a bounded row sample of the same workload.

--attn masked replaces the sparse attention by dsa_masked_mha_attn (the masked
mode for short prefill: dense over each query's causal range, non-selected
tokens masked); its roofline counts that dense work.

--warmup-objective times the indexer's dense warm-up step instead: the
indexer scores, the target distribution (the main attention summed over the
heads, dense), the KL loss with its score gradient (in place), and the
gradients into the indexer's q_I, w and k_I.

--bwd times the backward of the sparse attention over fixed indices
(dsa_sparse_mla_attn_bwd: dq and dkv for an upstream gradient of the output)
instead; the indices, output and lse come from one untimed forward pass.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

# MI355X published peaks.
PEAK_FP8_TFLOPS = 5000.0    # dense FP8 MFMA
PEAK_BF16_TFLOPS = 2500.0   # dense bf16 MFMA
PEAK_HBM_GBS = 8000.0

KERNEL_SOURCES = {
    "index_scores": "sparse_attention_02_amd/csrc/indexer.hip",
    "topk": "sparse_attention_02_amd/csrc/topk.hip",
    "sparse_mla_attn": "sparse_attention_02_amd/csrc/sparse_mla.hip",
    "masked_mha_attn": "sparse_attention_02_amd/csrc/sparse_mla.hip",
}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")
COPY_BYTES = 1 << 30  # calibration copy: reads and writes exactly this many bytes


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="prefill32k")
    ap.add_argument("--bwd", action="store_true",
                    help="time the attention backward over fixed indices instead of the forward step")
    ap.add_argument("--warmup-objective", action="store_true",
                    help="time the indexer's dense warm-up objective (scores, target, KL) instead")
    ap.add_argument("--warmup-lse", action="store_true",
                    help="with --warmup-objective: give the target kernel each head's dense lse "
                         "(computed once, untimed), as the warm-up's dense attention forward would")
    ap.add_argument("--attn", choices=["sparse", "masked"], default="sparse",
                    help="attention stage: the sparse kernel, or the masked mode for short prefill")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target wall time of the oracle sample")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after the timed steps, run a plain device-to-device copy of "
                         f"{COPY_BYTES >> 20} MiB three times (reference dispatches for scaling "
                         "the FETCH_SIZE / WRITE_SIZE counters of a PMC run)")
    return ap.parse_args()


def source_hash(rel: str) -> str:
    with open(os.path.join(ROOT, rel), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def algorithmic(wl):
    """Algorithmic work per launch (only what the method must do).  `bytes`
    counts every latent row a query gathers; `hbm_min_bytes` is the least HBM
    traffic the kernel needs: each byte of its inputs and outputs once, the
    gather counted at most once per cached latent row (a gather that fits the
    caches costs the cache once; a larger one, e.g. decode over many
    sequences, costs what it gathers)."""
    causal = wl.causal_pairs()
    sel = wl.selected_pairs()
    rows = wl.batch * wl.q_len
    attn_io = rows * wl.heads * (2 * wl.d_qk + 4 * wl.d_latent + 4) + 4.0 * rows * wl.topk
    gathered = 2.0 * wl.d_qk * sel
    cache = 2.0 * wl.d_qk * wl.batch * wl.kv_len
    work = {
        "index_scores": dict(
            flop=2.0 * wl.idx_heads * wl.idx_dim * causal,
            bytes=rows * wl.idx_heads * (wl.idx_dim + 4) + wl.batch * wl.kv_len * wl.idx_dim
            + 4.0 * causal),
        "topk": dict(flop=0.0, bytes=4.0 * causal + 4.0 * wl.topk * rows),
        "sparse_mla_attn": dict(
            flop=2.0 * wl.heads * (wl.d_qk + wl.d_latent) * sel,
            bytes=rows * wl.heads * (2 * wl.d_qk + 4 * wl.d_latent + 4) + 4.0 * rows * wl.topk
            + 2.0 * wl.d_qk * sel),
        # the masked mode scores every causal pair and runs the value product on
        # all of them (masked probabilities are zero); it reads each latent row
        # of the causal range once per query
        "masked_mha_attn": dict(
            flop=2.0 * wl.heads * (wl.d_qk + wl.d_latent) * causal,
            bytes=rows * wl.heads * (2 * wl.d_qk + 4 * wl.d_latent + 4) + 4.0 * rows * wl.topk
            + 2.0 * wl.d_qk * causal),
    }
    for name, w in work.items():
        w["hbm_min_bytes"] = w["bytes"]
    work["sparse_mla_attn"]["hbm_min_bytes"] = attn_io + min(gathered, cache)
    work["masked_mha_attn"]["hbm_min_bytes"] = attn_io + min(2.0 * wl.d_qk * causal, cache)
    return work


KERNEL_PEAK_TFLOPS = {"index_scores": PEAK_FP8_TFLOPS, "sparse_mla_attn": PEAK_BF16_TFLOPS,
                      "masked_mha_attn": PEAK_BF16_TFLOPS, "topk": None}


def roofline_ms(name, w):
    """The kernel's time at its roofline: the larger of its work at the MFMA peak
    of its dtype and its least HBM traffic at the HBM peak."""
    t_mem = w["hbm_min_bytes"] / (PEAK_HBM_GBS * 1e9) * 1e3
    peak = KERNEL_PEAK_TFLOPS[name]
    t_mfma = w["flop"] / (peak * 1e12) * 1e3 if peak and w["flop"] else 0.0
    return max(t_mem, t_mfma)


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def metric_name(wl) -> str:
    if wl.name == "prefill32k":
        return "DSA query tokens/s at L=32K prefill"
    if wl.q_len == 1:
        return f"DSA query tokens/s, {wl.name} ({wl.batch} sequences x 1 query over {wl.kv_len} tokens)"
    return f"DSA query tokens/s, {wl.name} ({wl.batch} x {wl.q_len} queries, positions {wl.q_start}.." \
           f"{wl.q_start + wl.q_len - 1} of {wl.kv_len})"


def bench_bwd(args, wl, dsa, prob, to_dev, q, kv, scores, indices, out, lse, ws, ws_bytes, aws, aws_bytes,
              q_idx, k_idx, w):
    """Backward of the sparse attention: one untimed forward for the indices,
    output and lse, then `steps` timed calls of dsa_sparse_mla_attn_bwd."""
    import numpy as np
    import torch
    stream = torch.cuda.current_stream()
    dsa.dsa_index_scores(prob, q_idx, k_idx, w, scores, stream=stream)
    dsa.dsa_topk(prob, scores, indices, ws, ws_bytes, stream=stream)
    dsa.dsa_sparse_mla_attn_ws(prob, q, kv, indices, out, lse, aws, aws_bytes, stream=stream)
    torch.cuda.synchronize()
    del scores
    torch.cuda.empty_cache()
    rows = wl.batch * wl.q_len
    gen = torch.Generator(device="cuda").manual_seed(11)
    dout = torch.randn((wl.batch, wl.q_len, wl.heads, wl.d_latent), dtype=torch.float32, device="cuda",
                       generator=gen)
    dq = torch.empty((wl.batch, wl.q_len, wl.heads, wl.d_qk), dtype=torch.float32, device="cuda")
    dkv = torch.zeros((wl.batch, wl.kv_len, wl.d_qk), dtype=torch.float32, device="cuda")
    bws_bytes = dsa.workspace_size(prob, dsa.DSA_OP_SPARSE_MLA_ATTN_BWD)
    bws = torch.empty(bws_bytes, dtype=torch.uint8, device="cuda")

    def step():
        dsa.dsa_sparse_mla_attn_bwd(prob, q, kv, indices, out, lse, dout, dq, dkv, bws, bws_bytes,
                                    stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for e in ev:
        e[0].record(stream)
        step()
        e[1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = [a.elapsed_time(b) for a, b in ev]
    sel = wl.selected_pairs()
    # per (selected pair, head): scores 2*Dqk, dout.v 2*Dv, dq 2*Dqk, dkv 2*Dqk + 2*Dv
    flop = 2.0 * wl.heads * sel * (3 * wl.d_qk + 2 * wl.d_latent)
    avg = float(np.mean(ms))
    tf = flop / (avg * 1e-3) / 1e12
    result = {
        "metric": "DSA sparse attention backward query tokens/s",
        "value": rows * args.steps / wall,
        "unit": "query tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall * 1e3 / args.steps,
        "event_ms_per_step": avg,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "batch": wl.batch, "q_len": wl.q_len, "kv_len": wl.kv_len,
                   "topk": wl.topk, "heads": wl.heads, "d_latent": wl.d_latent, "d_rope": wl.d_rope,
                   "pass": "attention backward"},
        "roofline": {"bound": "mfma", "achieved": tf, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": tf / PEAK_BF16_TFLOPS, "kernel": "sparse_mla_attn_bwd", "traffic": None},
        "algorithmic_flop": flop,
        "workspace_bytes": bws_bytes,
        "cpu_baseline": None if args.no_cpu_baseline else cpu_baseline_pass(wl, args.cpu_seconds, "bwd"),
    }
    print(json.dumps(result))


def bench_warmup(args, wl, dsa, prob, q, kv, scores, q_idx, k_idx, w):
    """The dense warm-up objective per step: dsa_index_scores, dsa_warmup_target,
    dsa_warmup_kl (gradient written over the scores)."""
    import numpy as np
    import torch
    stream = torch.cuda.current_stream()
    B, Lq, Lk = wl.batch, wl.q_len, wl.kv_len
    target = torch.empty((B, Lq, Lk), dtype=torch.float32, device="cuda")
    loss = torch.empty((B * Lq,), dtype=torch.float32, device="cuda")
    dq_idx = torch.empty((B, Lq, wl.idx_heads, wl.idx_dim), dtype=torch.float32, device="cuda")
    dw = torch.empty((B, Lq, wl.idx_heads), dtype=torch.float32, device="cuda")
    dk_idx = torch.empty((B, Lk, wl.idx_dim), dtype=torch.float32, device="cuda")
    lse = None
    if args.warmup_lse:
        lse = torch.empty((B, Lq, wl.heads), dtype=torch.float32, device="cuda")
        dsa.dsa_warmup_target(prob, q, kv, target, lse_out=lse, stream=stream)
        torch.cuda.synchronize()

    def step(ev=None):
        dk_idx.zero_()  # accumulated into by the indexer backward
        if ev:
            ev[0].record(stream)
        dsa.dsa_index_scores(prob, q_idx, k_idx, w, scores, stream=stream)
        if ev:
            ev[1].record(stream)
        dsa.dsa_warmup_target(prob, q, kv, target, lse_in=lse, stream=stream)
        if ev:
            ev[2].record(stream)
        dsa.dsa_warmup_kl(prob, scores, target, loss, scores, stream=stream)
        if ev:
            ev[3].record(stream)
        dsa.dsa_index_scores_bwd(prob, q_idx, k_idx, w, scores, dq_idx, dw, dk_idx, stream=stream)
        if ev:
            ev[4].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for ev in events:
        step(ev)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    names = ["index_scores", "warmup_target", "warmup_kl", "index_scores_bwd"]
    per = {n: [ev[j].elapsed_time(ev[j + 1]) for ev in events] for j, n in enumerate(names)}
    pairs = wl.causal_pairs()
    # algorithmic work: one evaluation of every head's scores per causal pair
    # (without a given lse the kernel evaluates them twice: the lse, then the sum)
    t_flop = 2.0 * wl.heads * wl.d_qk * pairs
    k1_flop = 2.0 * wl.idx_heads * wl.idx_dim * pairs
    kl_bytes = 16.0 * pairs  # scores read twice, target read once, gradient written
    t_ms = float(np.mean(per["warmup_target"]))
    kernels = {}
    for n in names:
        a = np.array(per[n])
        kernels[n] = {"avg_ms": float(a.mean()), "median_ms": float(np.median(a)), "min_ms": float(a.min())}
    kernels["index_scores"]["fp8_tflops"] = k1_flop / (kernels["index_scores"]["avg_ms"] * 1e-3) / 1e12
    kernels["warmup_target"]["bf16_tflops"] = t_flop / (t_ms * 1e-3) / 1e12
    kernels["warmup_kl"]["gbps"] = kl_bytes / (kernels["warmup_kl"]["avg_ms"] * 1e-3) / 1e9
    # indexer backward: u once plus the dq_I and dk_I products, 3 * 2 * H_I * d_I
    # per causal pair (the two kernels each recompute u: 4 evaluations run)
    ib_flop = 3.0 * k1_flop
    kernels["index_scores_bwd"]["bf16_tflops"] = ib_flop / (kernels["index_scores_bwd"]["avg_ms"] * 1e-3) / 1e12
    tf = t_flop / (t_ms * 1e-3) / 1e12
    result = {
        "metric": "DSA indexer warm-up objective query tokens/s",
        "value": B * Lq * args.steps / wall,
        "unit": "query tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall * 1e3 / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "batch": B, "q_len": Lq, "kv_len": Lk, "heads": wl.heads,
                   "d_latent": wl.d_latent, "d_rope": wl.d_rope, "idx_heads": wl.idx_heads,
                   "idx_dim": wl.idx_dim, "pass": "dense warm-up step (objective and indexer gradients)",
                   "attention_lse": "given" if args.warmup_lse else "computed"},
        "kernels": kernels,
        "roofline": {"bound": "mfma", "achieved": tf, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": tf / PEAK_BF16_TFLOPS, "kernel": "warmup_target", "traffic": None},
        "cpu_baseline": None if args.no_cpu_baseline else cpu_baseline_pass(wl, args.cpu_seconds, "warmup"),
    }
    print(json.dumps(result))


def traffic_for(kernel: str):
    """HBM bytes per launch from the committed PMC summary, if it was taken on the
    current kernel source; otherwise None."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    e = t.get(kernel)
    if not e or e.get("source_sha256_16") != source_hash(KERNEL_SOURCES[kernel]):
        return None
    return e.get("hbm_bytes_per_launch")


def cpu_baseline(wl, target_s: float):
    """The oracle (as it stands) on an evenly spaced row sample of the workload."""
    import numpy as np

    import dsa_inputs
    import oracle

    k_idx = dsa_inputs.k_idx(wl)
    kv = dsa_inputs.kv(wl)

    def run(n):
        rows = ((np.arange(n) + 0.5) * (wl.batch * wl.q_len) / n).astype(np.int64)
        rb, pos = dsa_inputs.row_batch_pos(wl, rows)
        qi, w, q = dsa_inputs.q_idx(wl, rows), dsa_inputs.w(wl, rows), dsa_inputs.q(wl, rows)
        t0 = time.perf_counter()
        oracle.forward(k_idx, qi, w, q, kv, rb, pos, wl.topk, wl.d_latent, wl.softmax_scale)
        return time.perf_counter() - t0

    threads = oracle.max_threads()
    pilot_n = max(4, threads)
    pilot = run(pilot_n)
    n = int(min(4096, max(pilot_n, pilot_n * target_s / max(pilot, 1e-3))))
    secs = run(n)
    return {"value": n / secs, "unit": "query tokens/s", "cores": threads, "kind": "oracle",
            "cpu_model": cpu_model(), "host_cpus": os.cpu_count(),
            "sample": f"{n} query rows evenly spaced over the {wl.batch * wl.q_len} query rows "
                      f"(indexer + top-k + attention per row, {secs:.1f} s wall)"}


def cpu_baseline_pass(wl, target_s: float, which: str):
    """The oracle (as it stands) timed on an evenly spaced row sample for the
    backward ("bwd": dq and dkv of the sampled rows, their indices from the
    oracle's forward, untimed) or the warm-up step ("warmup": indexer scores,
    target, KL and the indexer gradients of the sampled rows)."""
    import numpy as np

    import dsa_inputs
    import oracle

    k_idx = dsa_inputs.k_idx(wl)
    kv = dsa_inputs.kv(wl)
    rng = np.random.default_rng(3)

    def run(n):
        rows = ((np.arange(n) + 0.5) * (wl.batch * wl.q_len) / n).astype(np.int64)
        rb, pos = dsa_inputs.row_batch_pos(wl, rows)
        qi, w, q = dsa_inputs.q_idx(wl, rows), dsa_inputs.w(wl, rows), dsa_inputs.q(wl, rows)
        if which == "bwd":
            res = oracle.forward(k_idx, qi, w, q, kv, rb, pos, wl.topk, wl.d_latent, wl.softmax_scale)
            g = rng.normal(size=(n, wl.heads, wl.d_latent))
            t0 = time.perf_counter()
            oracle.sparse_mla_attn_bwd(kv, q, res["indices"], rb, g, wl.d_latent, wl.softmax_scale, wl.batch)
            return time.perf_counter() - t0
        t0 = time.perf_counter()
        scores = oracle.index_scores(k_idx, qi, w, rb, pos)
        target = oracle.warmup_target(kv, q, rb, pos, wl.softmax_scale)
        _, d = oracle.warmup_kl(scores, target.astype(np.float32), pos)
        oracle.index_scores_bwd(k_idx, qi, w, rb, pos, np.nan_to_num(d, nan=0.0))
        return time.perf_counter() - t0

    threads = oracle.max_threads()
    pilot_n = max(4, threads)
    pilot = run(pilot_n)
    n = int(min(4096, max(pilot_n, pilot_n * target_s / max(pilot, 1e-3))))
    secs = run(n)
    what = ("attention backward (dq, dkv) per row" if which == "bwd"
            else "indexer scores, target, KL and indexer gradients per row")
    return {"value": n / secs, "unit": "query tokens/s", "cores": threads, "kind": "oracle",
            "cpu_model": cpu_model(), "host_cpus": os.cpu_count(),
            "sample": f"{n} query rows evenly spaced over the {wl.batch * wl.q_len} query rows "
                      f"({what}, {secs:.1f} s wall)"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); "
              "the DSA path here is a single-GPU build.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import dsa_inputs
    import sparse_attention_02_amd as dsa

    wl = dsa_inputs.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def to_dev(a):
        if a.dtype == np.uint16:
            a = a.view(np.int16)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    t_gen = time.perf_counter()
    q_idx = to_dev(dsa_inputs.q_idx(wl))
    k_idx = to_dev(dsa_inputs.k_idx(wl))
    w = to_dev(dsa_inputs.w(wl))
    kv = to_dev(dsa_inputs.kv(wl))
    q = to_dev(dsa_inputs.q(wl))
    t_gen = time.perf_counter() - t_gen
    print(f"[bench] inputs for {wl.name} generated and copied in {t_gen:.1f} s", file=sys.stderr,
          flush=True)

    prob = dsa.Problem.from_workload(wl)
    B, Lq, Lk = wl.batch, wl.q_len, wl.kv_len
    scores = torch.empty((B, Lq, Lk), dtype=torch.float32, device=dev)
    indices = torch.empty((B, Lq, wl.topk), dtype=torch.int32, device=dev)
    out = torch.empty((B, Lq, wl.heads, wl.d_latent), dtype=torch.float32, device=dev)
    lse = torch.empty((B, Lq, wl.heads), dtype=torch.float32, device=dev)
    ws_bytes = dsa.workspace_size(prob, dsa.DSA_OP_TOPK)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    aws_bytes = dsa.workspace_size(prob, dsa.DSA_OP_SPARSE_MLA_ATTN)
    aws = torch.empty(max(aws_bytes, 1), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    if args.warmup_objective:
        bench_warmup(args, wl, dsa, prob, q, kv, scores, q_idx, k_idx, w)
        return
    if args.bwd:
        bench_bwd(args, wl, dsa, prob, to_dev, q, kv, scores, indices, out, lse, ws, ws_bytes, aws,
                  aws_bytes, q_idx, k_idx, w)
        return

    attn_name = "sparse_mla_attn" if args.attn == "sparse" else "masked_mha_attn"
    names = ["index_scores", "topk", attn_name]
    iws_bytes = dsa.workspace_size(prob, dsa.DSA_OP_INDEX_TOPK)
    iws = torch.empty(iws_bytes, dtype=torch.uint8, device=dev)
    # the header's workspace rule: beyond the score matrix and the top-k
    # scratch only when the sampled path is taken
    r256 = lambda n: (n + 255) // 256 * 256
    sampled = iws_bytes > r256(4 * B * Lq * Lk) + r256(ws_bytes)

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        dsa.dsa_index_topk(prob, q_idx, k_idx, w, indices, iws, iws_bytes, stream=stream)
        if ev is not None:
            ev[1].record(stream)
        if args.attn == "sparse":
            dsa.dsa_sparse_mla_attn_ws(prob, q, kv, indices, out, lse, aws, aws_bytes, stream=stream)
        else:
            dsa.dsa_masked_mha_attn(prob, q, kv, indices, out, lse, stream=stream)
        if ev is not None:
            ev[2].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    events = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    print(f"[bench] {args.steps} steps in {wall:.3f} s", file=sys.stderr, flush=True)

    # the indexer and the top-k as separate calls, for their own figures; the
    # attention follows each pair as in a step, so the kernels run under the
    # same load (and clock) as in the timed steps
    n_stage = max(1, min(args.steps, 10))
    stage_idx = torch.empty_like(indices)
    stage_events = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(n_stage)]
    for i in range(-1, n_stage):
        ev = stage_events[i] if i >= 0 else None
        if ev is not None:
            ev[0].record(stream)
        dsa.dsa_index_scores(prob, q_idx, k_idx, w, scores, stream=stream)
        if ev is not None:
            ev[1].record(stream)
        dsa.dsa_topk(prob, scores, stage_idx, ws, ws_bytes, stream=stream)
        if ev is not None:
            ev[2].record(stream)
        if args.attn == "sparse":
            dsa.dsa_sparse_mla_attn_ws(prob, q, kv, stage_idx, out, lse, aws, aws_bytes, stream=stream)
        else:
            dsa.dsa_masked_mha_attn(prob, q, kv, stage_idx, out, lse, stream=stream)
    torch.cuda.synchronize()
    del stage_idx

    if args.copy_calibration:
        src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        print(f"[bench] calibration copies of {COPY_BYTES} bytes done", file=sys.stderr, flush=True)

    per = {n: [] for n in names}
    per["index_topk"] = []
    for ev in events:
        per["index_topk"].append(ev[0].elapsed_time(ev[1]))
        per[attn_name].append(ev[1].elapsed_time(ev[2]))
    for ev in stage_events:
        per["index_scores"].append(ev[0].elapsed_time(ev[1]))
        per["topk"].append(ev[1].elapsed_time(ev[2]))
    step_ms = [ev[0].elapsed_time(ev[2]) for ev in events]
    ms_per_step = wall * 1e3 / args.steps

    work = algorithmic(wl)
    kernels = {}
    for n in names:
        avg_ms = float(np.mean(per[n]))
        k = {"avg_ms": avg_ms, "median_ms": float(np.median(per[n])), "min_ms": float(np.min(per[n])),
             "algorithmic_flop": work[n]["flop"], "algorithmic_bytes": work[n]["bytes"],
             "hbm_min_bytes": work[n]["hbm_min_bytes"], "roofline_ms": roofline_ms(n, work[n]),
             "hbm_bytes_per_launch": traffic_for(n)}
        if work[n]["flop"]:
            tf = work[n]["flop"] / (avg_ms * 1e-3) / 1e12
            peak = PEAK_FP8_TFLOPS if n == "index_scores" else PEAK_BF16_TFLOPS
            k.update(tflops=tf, mfma_peak_tflops=peak, frac_of_mfma_peak=tf / peak)
        gbs = work[n]["bytes"] / (avg_ms * 1e-3) / 1e9
        k.update(algorithmic_gbs=gbs, frac_of_hbm_peak=gbs / PEAK_HBM_GBS)
        kernels[n] = k

    # the step's selection call: the indexer's roofline, plus the top-k's
    # score read when the scores are written out
    sel_roof = kernels["index_scores"]["roofline_ms"] + (0.0 if sampled else kernels["topk"]["roofline_ms"])
    kernels["index_topk"] = {"avg_ms": float(np.mean(per["index_topk"])),
                             "median_ms": float(np.median(per["index_topk"])),
                             "min_ms": float(np.min(per["index_topk"])), "sampled_path": sampled,
                             "roofline_ms": sel_roof, "stage_calls_timed": n_stage}

    dom = max(names, key=lambda n: kernels[n]["avg_ms"])
    kd = kernels[dom]
    if work[dom]["flop"]:
        roof = {"bound": "mfma", "achieved": kd["tflops"], "peak": kd["mfma_peak_tflops"],
                "unit": "TFLOP/s", "frac": kd["frac_of_mfma_peak"]}
    else:
        roof = {"bound": "hbm", "achieved": kd["algorithmic_gbs"], "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": kd["frac_of_hbm_peak"]}
    roof["kernel"] = dom
    roof["traffic"] = kd["hbm_bytes_per_launch"]

    value = wl.batch * wl.q_len * args.steps / wall
    ceiling_ms = sel_roof + kernels[attn_name]["roofline_ms"]
    result = {
        "metric": metric_name(wl),
        "value": value,
        "unit": "query tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "event_ms_per_step": float(np.mean(step_ms)),
        "event_ms_per_step_median": float(np.median(step_ms)),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8/bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "batch": wl.batch, "q_len": wl.q_len, "kv_len": wl.kv_len,
                   "q_start": wl.q_start, "topk": wl.topk, "idx_heads": wl.idx_heads,
                   "idx_dim": wl.idx_dim, "heads": wl.heads, "d_latent": wl.d_latent,
                   "d_rope": wl.d_rope, "attn": args.attn},
        "roofline": roof,
        # the whole step against the sum of its kernels' roofline times
        "end_to_end": {"ceiling_ms": ceiling_ms, "ms_per_step": ms_per_step, "frac": ceiling_ms / ms_per_step,
                       "sampled_selection": sampled,
                       "ceiling_query_tokens_per_s": wl.batch * wl.q_len / (ceiling_ms * 1e-3)},
        "indexer_fp8_tflops": kernels["index_scores"]["tflops"],
        "indexer_frac_of_fp8_peak": kernels["index_scores"]["frac_of_mfma_peak"],
        "indexer_fp8_tflops_median": work["index_scores"]["flop"] / (kernels["index_scores"]["median_ms"] * 1e-3) / 1e12,
        "kernels": kernels,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        del scores, indices, out, lse, q, q_idx, iws
        torch.cuda.empty_cache()
        print("[bench] timing the CPU oracle on a row sample", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds)
    print(json.dumps(result))


if __name__ == "__main__":
    main()
