"""The GPU tests' property check of a selection, run on the CPU: it accepts the
oracle's selections and rejects selections with a planted mistake (a tie
broken towards the higher index, a better candidate left out, a wrong count,
an unsorted row).  This keeps the all-rows check of the large workloads
honest."""
import numpy as np
import pytest
import torch

import dsa_inputs
import oracle
from gpu_util import check_selection_properties

WL = dsa_inputs.Workload("checks", 0, 2, 40, 300, 260, 4, 32, 64, 8, 64, 16)


def _case():
    rng = np.random.default_rng(9)
    s = rng.integers(-3, 4, size=(WL.batch, WL.q_len, WL.kv_len)).astype(np.float32)
    pos = (WL.q_start + np.arange(WL.q_len)).astype(np.int32)
    idx = np.stack([oracle.topk(s[b], pos, WL.topk) for b in range(WL.batch)])
    return s, idx


def test_oracle_selection_passes_and_ties_bind():
    s, idx = _case()
    n = check_selection_properties(WL, torch.from_numpy(s), torch.from_numpy(idx))
    assert n > 0  # the tie rule is exercised


def _planted(kind):
    s, idx = _case()
    b, t = 1, 17
    row, sel = s[b, t], idx[b, t].copy()
    thr = row[sel].min()
    tied_out = [c for c in range(WL.q_start + t + 1) if row[c] == thr and c not in sel]
    if kind == "tie":          # swap the highest selected tied index for a higher unselected one
        hi = max(c for c in sel if row[c] == thr)
        cand = [c for c in tied_out if c > hi]
        sel[list(sel).index(hi)] = cand[0]
    elif kind == "threshold":  # replace a selected entry above the threshold by an unselected tie
        above = [i for i, c in enumerate(sel) if row[c] > thr]
        sel[above[0]] = tied_out[0]
    elif kind == "order":
        sel[[3, 4]] = sel[[4, 3]]
    elif kind == "count":
        sel[-1] = -1
    idx[b, t] = np.sort(sel) if kind in ("tie", "threshold") else sel
    return s, idx


@pytest.mark.parametrize("kind", ["tie", "threshold", "order", "count"])
def test_planted_mistakes_are_caught(kind):
    s, idx = _planted(kind)
    with pytest.raises(AssertionError):
        check_selection_properties(WL, torch.from_numpy(s), torch.from_numpy(idx))
