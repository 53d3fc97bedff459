"""Helpers for the GPU parity tests: inputs on host and device, runs through the
C ABI, and comparisons with the CPU oracle on selected rows."""
from __future__ import annotations

import dataclasses
import sys
from typing import Optional

import numpy as np
import torch

import dsa_inputs
import oracle


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def dev(a: np.ndarray) -> torch.Tensor:
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


@dataclasses.dataclass
class Inputs:
    wl: dsa_inputs.Workload
    k_idx: np.ndarray
    q_idx: np.ndarray
    w: np.ndarray
    q: np.ndarray
    kv: np.ndarray

    @classmethod
    def make(cls, wl) -> "Inputs":
        return cls(wl, dsa_inputs.k_idx(wl), dsa_inputs.q_idx(wl), dsa_inputs.w(wl),
                   dsa_inputs.q(wl), dsa_inputs.kv(wl))

    def device(self):
        return dict(k_idx=dev(self.k_idx), q_idx=dev(self.q_idx), w=dev(self.w), q=dev(self.q),
                    kv=dev(self.kv))


def run_stages(prob, d, wl, fill_scores=float("-inf"), lse=True):
    """The three entry points in order; returns scores, indices, out, lse tensors."""
    import sparse_attention_02_amd as dsa
    B, Lq, Lk = wl.batch, wl.q_len, wl.kv_len
    scores = torch.full((B, Lq, Lk), fill_scores, dtype=torch.float32, device="cuda")
    indices = torch.empty((B, Lq, wl.topk), dtype=torch.int32, device="cuda")
    out = torch.empty((B, Lq, wl.heads, wl.d_latent), dtype=torch.float32, device="cuda")
    lse_t = torch.empty((B, Lq, wl.heads), dtype=torch.float32, device="cuda") if lse else None
    dsa.dsa_index_scores(prob, d["q_idx"], d["k_idx"], d["w"], scores)
    ws_bytes = dsa.workspace_size(prob, dsa.DSA_OP_TOPK)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device="cuda")
    dsa.dsa_topk(prob, scores, indices, ws, ws_bytes)
    aws_bytes = dsa.workspace_size(prob, dsa.DSA_OP_SPARSE_MLA_ATTN)
    aws = torch.empty(aws_bytes, dtype=torch.uint8, device="cuda") if aws_bytes else None
    dsa.dsa_sparse_mla_attn_ws(prob, d["q"], d["kv"], indices, out, lse_t, aws, aws_bytes)
    torch.cuda.synchronize()
    return scores, indices, out, lse_t


def check_rows(inp: Inputs, rows, scores, indices, out, lse, atol=1e-2, label=""):
    """Bit-exact scores and indices and attention within atol on the given flat rows,
    against the oracle (the oracle's own indices feed its attention)."""
    wl = inp.wl
    rows = np.asarray(rows, dtype=np.int64)
    rb, pos = dsa_inputs.row_batch_pos(wl, rows)
    Lk = wl.kv_len
    s_or = oracle.index_scores(inp.k_idx, inp.q_idx[rows], inp.w[rows], rb, pos)
    rt = torch.from_numpy(rows).cuda()
    s_gpu = scores.reshape(-1, Lk).index_select(0, rt).cpu().numpy()
    for i, r in enumerate(rows):
        n = min(int(pos[i]) + 1, Lk)
        a = s_gpu[i, :n].view(np.uint32)
        b = s_or[i, :n].view(np.uint32)
        if not np.array_equal(a, b):
            bad = np.nonzero(a != b)[0]
            raise AssertionError(f"{label} scores row {r}: {len(bad)} mismatches, first s={bad[0]} "
                                 f"gpu={s_gpu[i, bad[0]]!r} oracle={s_or[i, bad[0]]!r}")
    idx_or = oracle.topk(s_or, pos, wl.topk)
    idx_gpu = indices.reshape(-1, wl.topk).index_select(0, rt).cpu().numpy()
    for i, r in enumerate(rows):
        if not np.array_equal(idx_gpu[i], idx_or[i]):
            bad = np.nonzero(idx_gpu[i] != idx_or[i])[0]
            raise AssertionError(f"{label} indices row {r}: {len(bad)} slots differ, first slot "
                                 f"{bad[0]}: gpu={idx_gpu[i, bad[0]]} oracle={idx_or[i, bad[0]]}")
    out_or, lse_or = oracle.sparse_mla_attn(inp.kv, inp.q[rows], idx_or, rb, wl.d_latent,
                                            wl.softmax_scale)
    out_gpu = out.reshape(-1, wl.heads, wl.d_latent).index_select(0, rt).cpu().numpy()
    err = float(np.abs(out_gpu - out_or).max())
    assert err <= atol, f"{label} attention max-abs error {err} > {atol}"
    lerr = 0.0
    if lse is not None:
        lse_gpu = lse.reshape(-1, wl.heads).index_select(0, rt).cpu().numpy()
        lerr = float(np.abs(lse_gpu - lse_or).max())
        assert lerr <= atol, f"{label} lse max-abs error {lerr} > {atol}"
    return err, lerr


def check_selection_properties(wl, scores, indices):
    """Properties of the GPU selection that hold at any size, checked on every row:
    ascending valid prefix, count = min(pos+1, k), values <= pos, -1 padding,
    min(selected scores) >= max(unselected candidate scores), and the tie rule:
    among the candidates whose score equals the row's smallest selected score,
    every selected index is below every unselected one.
    Entries of `scores` past pos are not read.  Returns the number of rows
    where the tie rule binds (an unselected candidate ties the threshold)."""
    B, Lq, Lk, k = wl.batch, wl.q_len, wl.kv_len, wl.topk
    dev = scores.device
    pos = torch.arange(Lq, device=dev, dtype=torch.int64) + wl.q_start
    n_exp = torch.clamp(torch.clamp(pos + 1, max=Lk), max=k)              # [Lq]
    idx = indices.to(torch.int64)                                          # [B, Lq, k]
    valid = idx >= 0
    assert torch.equal(valid.sum(-1), n_exp.expand(B, Lq)), "selected count != min(pos+1, k)"
    slot = torch.arange(k, device=dev)
    assert torch.equal(valid, (slot[None, None, :] < n_exp[None, :, None]).expand(B, Lq, k)), \
        "padding is not a -1 suffix"
    assert bool(((idx <= pos[None, :, None]) | ~valid).all()), "selected index beyond pos"
    d = idx[..., 1:] - idx[..., :-1]
    assert bool(((d > 0) | ~valid[..., 1:]).all()), "indices not strictly ascending"
    # threshold and tie properties, processed in row blocks to bound memory
    rows_per = max(1, (1 << 27) // (Lk * 4))
    col = torch.arange(Lk, device=dev, dtype=torch.int64)
    big = torch.iinfo(torch.int64).max
    n_tied_rows = 0
    for b in range(B):
        for t0 in range(0, Lq, rows_per):
            t1 = min(Lq, t0 + rows_per)
            s = scores[b, t0:t1]
            ii = idx[b, t0:t1]
            vv = valid[b, t0:t1]
            safe = torch.where(vv, ii, torch.zeros_like(ii))
            sel = torch.gather(s, 1, safe)
            sel = torch.where(vv, sel, torch.full_like(sel, float("inf")))
            min_sel = sel.min(1).values
            # -1 slots point at column 0 with a zero count, so they mark nothing
            chosen = torch.zeros(s.shape, dtype=torch.int32, device=dev)
            chosen.scatter_add_(1, safe, vv.to(torch.int32))
            chosen = chosen > 0
            cand = col[None, :] <= pos[t0:t1, None]
            rest = torch.where(chosen | ~cand, torch.full_like(s, float("-inf")), s)
            max_rest = rest.max(1).values
            assert bool((min_sel >= max_rest).all()), f"threshold property fails in batch {b} rows {t0}..{t1}"
            tied = cand & (s == min_sel[:, None])
            hi_sel = torch.where(tied & chosen, col[None, :], torch.full_like(col, -1)[None, :]).max(1).values
            lo_rest = torch.where(tied & ~chosen, col[None, :], torch.full_like(col, big)[None, :]).min(1).values
            assert bool((hi_sel < lo_rest).all()), f"tie rule fails in batch {b} rows {t0}..{t1}"
            n_tied_rows += int((lo_rest < big).sum())
    return n_tied_rows
