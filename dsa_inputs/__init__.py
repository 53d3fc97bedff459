"""Seeded synthetic workloads for the DeepSeek Sparse Attention hot path.

This module only describes workloads and draws random inputs; it holds none of
the method's arithmetic.  The CPU oracle and the GPU library both consume the
arrays it returns, so every comparison is made on identical bytes.

Workloads (DeepSeek-V3.2 DSA as described in "DeepSeek V3.2 and the lightning
indexer" (section "How the lightning indexer works") and the DeepSeek-V3.2 spec
sheet (design overview, section 2.1)): a lightning indexer with FP8 queries and
keys, top-k with k = 2048, and MLA in MQA mode over 576-wide bf16 latents
(512 latent + 64 rope); the trained and deployed context is 131,072 tokens
(spec sheet, "Context" table).  Shapes and value grids:

  tiny      L=256, k=64, indexer 4 heads x 32, 8 query heads, latent 64 + rope 16
  prefill4k L=4096, k=2048, indexer 64 x 128, 128 heads, latent 512 + rope 64
  prefill32k L=32768, otherwise as prefill4k
  decode    64 sequences, one new query each against a 131,072-token cache
  chunked   8192 new queries (positions 122880..131071) over a 131,072 context

Indexer q/k values lie on the 0.25-step grid of [-4, 4] (FP8 e4m3), the head
weights on the 0.25-step grid of [-1, 1] (fp32), and q / kv are N(0,1) in bf16.
"""
from __future__ import annotations

import ctypes
import dataclasses
import math
import os
import subprocess
from typing import Dict, Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# DSA_INPUTS_LIBRARY names another build (the sanitizer test's); unset, the
# in-tree build is used.
_LIB_PATH = os.environ.get("DSA_INPUTS_LIBRARY") or os.path.join(_HERE, "libdsa_inputs.so")

# Tensor ids: each tensor of a workload draws from its own stream.
TID_Q_IDX, TID_K_IDX, TID_W, TID_Q, TID_KV = 1, 2, 3, 4, 5


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    batch: int
    q_len: int
    kv_len: int
    q_start: int
    idx_heads: int
    idx_dim: int
    topk: int
    heads: int
    d_latent: int
    d_rope: int

    @property
    def d_qk(self) -> int:
        return self.d_latent + self.d_rope

    @property
    def softmax_scale(self) -> float:
        return 1.0 / math.sqrt(self.d_qk)

    def positions(self) -> np.ndarray:
        return self.q_start + np.arange(self.q_len, dtype=np.int64)

    def causal_pairs(self) -> int:
        """Number of (query, key) pairs with key <= pos, summed over the batch."""
        p = self.positions()
        return int(self.batch * np.minimum(p + 1, self.kv_len).sum())

    def selected_pairs(self) -> int:
        p = self.positions()
        return int(self.batch * np.minimum(np.minimum(p + 1, self.kv_len), self.topk).sum())

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS: Dict[str, Workload] = {
    "tiny": Workload("tiny", 0, 1, 256, 256, 0, 4, 32, 64, 8, 64, 16),
    "prefill4k": Workload("prefill4k", 1, 1, 4096, 4096, 0, 64, 128, 2048, 128, 512, 64),
    "prefill32k": Workload("prefill32k", 2, 1, 32768, 32768, 0, 64, 128, 2048, 128, 512, 64),
    "decode": Workload("decode", 3, 64, 1, 131072, 131071, 64, 128, 2048, 128, 512, 64),
    "chunked": Workload("chunked", 4, 1, 8192, 131072, 122880, 64, 128, 2048, 128, 512, 64),
    # 1M-token contexts (the indexer's surviving quadratic term at long context)
    "decode1m": Workload("decode1m", 5, 4, 1, 1048576, 1048575, 64, 128, 2048, 128, 512, 64),
    "chunked1m": Workload("chunked1m", 6, 1, 4096, 1048576, 1044480, 64, 128, 2048, 128, 512, 64),
    # short prefill, every row selects its whole causal prefix (L <= k): the
    # regime of the masked mode
    "prefill2k": Workload("prefill2k", 7, 1, 2048, 2048, 0, 64, 128, 2048, 128, 512, 64),
}


def _build() -> None:
    src = os.path.join(_HERE, "gen.c")
    tmp = _LIB_PATH + ".tmp"
    subprocess.check_call(["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-std=c11", src, "-o", tmp, "-lm"])
    os.replace(tmp, _LIB_PATH)


_lib = None


def lib(rebuild: bool = False):
    global _lib
    if rebuild or not os.path.exists(_LIB_PATH):
        _build()
        _lib = None
    if _lib is None:
        L = ctypes.CDLL(_LIB_PATH)
        u64, i64, i32, vp = ctypes.c_uint64, ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p
        L.dsa_gen_e4m3_grid.argtypes = [u64, u64, i64, i64, vp]
        L.dsa_gen_f32_grid.argtypes = [u64, u64, i64, i64, i32, ctypes.c_double, ctypes.c_double, vp]
        L.dsa_gen_bf16_normal.argtypes = [u64, u64, i64, i64, vp]
        for f in (L.dsa_gen_e4m3_grid, L.dsa_gen_f32_grid, L.dsa_gen_bf16_normal):
            f.restype = None
        _lib = L
    return _lib


def e4m3_grid(seed: int, tid: int, offset: int, n: int) -> np.ndarray:
    out = np.empty(n, dtype=np.uint8)
    lib().dsa_gen_e4m3_grid(seed, tid, offset, n, out.ctypes.data)
    return out


def f32_grid(seed: int, tid: int, offset: int, n: int, npoints: int, lo: float, step: float) -> np.ndarray:
    out = np.empty(n, dtype=np.float32)
    lib().dsa_gen_f32_grid(seed, tid, offset, n, npoints, lo, step, out.ctypes.data)
    return out


def bf16_normal(seed: int, tid: int, offset: int, n: int) -> np.ndarray:
    out = np.empty(n, dtype=np.uint16)
    lib().dsa_gen_bf16_normal(seed, tid, offset, n, out.ctypes.data)
    return out


# ---------------------------------------------------------------------------
# Whole tensors and single query rows of a workload
# ---------------------------------------------------------------------------

def k_idx(wl: Workload) -> np.ndarray:
    """Indexer key cache [B, Lk, d_I], e4m3fn bytes."""
    n = wl.batch * wl.kv_len * wl.idx_dim
    return e4m3_grid(wl.seed, TID_K_IDX, 0, n).reshape(wl.batch, wl.kv_len, wl.idx_dim)


def kv(wl: Workload) -> np.ndarray:
    """Latent cache [B, Lk, D_v + D_r], bf16 bits."""
    n = wl.batch * wl.kv_len * wl.d_qk
    return bf16_normal(wl.seed, TID_KV, 0, n).reshape(wl.batch, wl.kv_len, wl.d_qk)


def _row_block(wl: Workload, tid: int, per_row: int, rows: Optional[Sequence[int]], gen) -> np.ndarray:
    total_rows = wl.batch * wl.q_len
    if rows is None:
        return gen(0, total_rows * per_row).reshape(total_rows, per_row)
    out = np.empty((len(rows), per_row), dtype=gen(0, 0).dtype)
    for i, r in enumerate(rows):
        if not 0 <= r < total_rows:
            raise IndexError(f"row {r} outside 0..{total_rows - 1}")
        out[i] = gen(int(r) * per_row, per_row)
    return out


def q_idx(wl: Workload, rows: Optional[Sequence[int]] = None) -> np.ndarray:
    """Indexer queries, e4m3fn bytes: [B*Lq, H_I, d_I] (or only the listed flat rows b*Lq+t)."""
    per = wl.idx_heads * wl.idx_dim
    a = _row_block(wl, TID_Q_IDX, per, rows, lambda o, n: e4m3_grid(wl.seed, TID_Q_IDX, o, n))
    return a.reshape(-1, wl.idx_heads, wl.idx_dim)


def w(wl: Workload, rows: Optional[Sequence[int]] = None) -> np.ndarray:
    """Indexer head weights, fp32 [B*Lq, H_I] on the 0.25-step grid of [-1, 1]."""
    a = _row_block(wl, TID_W, wl.idx_heads, rows,
                   lambda o, n: f32_grid(wl.seed, TID_W, o, n, 9, -1.0, 0.25))
    return a.reshape(-1, wl.idx_heads)


def q(wl: Workload, rows: Optional[Sequence[int]] = None) -> np.ndarray:
    """MQA-mode queries, bf16 bits [B*Lq, H, D_v + D_r]."""
    per = wl.heads * wl.d_qk
    a = _row_block(wl, TID_Q, per, rows, lambda o, n: bf16_normal(wl.seed, TID_Q, o, n))
    return a.reshape(-1, wl.heads, wl.d_qk)


def row_batch_pos(wl: Workload, rows: Sequence[int]):
    """Batch index and absolute position of flat query rows r = b*Lq + t."""
    r = np.asarray(rows, dtype=np.int64)
    return (r // wl.q_len).astype(np.int32), (wl.q_start + r % wl.q_len).astype(np.int32)


def sample_rows(wl: Workload, n_random: int, seed: int = 12345) -> np.ndarray:
    """Deterministic row sample: row 0, rows around k-2..k, the last row of each
    sequence, plus n_random uniform rows."""
    total = wl.batch * wl.q_len
    fixed = {0, total - 1}
    for t in (wl.topk - 2, wl.topk - 1, wl.topk, wl.q_len - 1):
        if 0 <= t < wl.q_len:
            fixed.add(t)
    rng = np.random.default_rng(seed)
    rand = rng.integers(0, total, size=n_random) if n_random > 0 else []
    return np.array(sorted(fixed.union(int(x) for x in rand)), dtype=np.int64)
