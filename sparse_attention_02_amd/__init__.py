"""Python binding of libdsa.so — the DeepSeek Sparse Attention hot path on MI355X.

Argument marshalling only: every function passes raw device pointers of torch
tensors and the current HIP stream to the C ABI declared in include/dsa.h and
raises DsaError on a non-zero status.  All computation happens in the HIP
kernels; there is no CPU fallback, and importing this module fails loudly when
the built library is missing (build it with ``python -m
sparse_attention_02_amd.build`` or ``__graft_entry__.build()``).
"""
from __future__ import annotations

import ctypes
import dataclasses
import math
import os
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
# DSA_LIBRARY names another build of the same library (the sanitizer test
# loads a host-instrumented one); unset, the in-tree build is used.
LIB_PATH = os.environ.get("DSA_LIBRARY") or os.path.join(_HERE, "libdsa.so")

DSA_OP_INDEX_SCORES, DSA_OP_TOPK, DSA_OP_SPARSE_MLA_ATTN, DSA_OP_FORWARD = 0, 1, 2, 3
DSA_OP_SPARSE_MLA_ATTN_BWD = 4
DSA_OP_INDEX_TOPK = 5
STATUS = {0: "DSA_OK", -1: "DSA_ERR_NULL", -2: "DSA_ERR_SHAPE", -3: "DSA_ERR_UNSUPPORTED",
          -4: "DSA_ERR_WORKSPACE", -5: "DSA_ERR_ALIGN", -6: "DSA_ERR_HIP"}


class DsaError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{STATUS.get(status, status)}: {detail}")
        self.status = status


class _Problem(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("batch", "q_len", "kv_len", "q_start", "idx_heads", "idx_dim", "topk",
                 "heads", "d_latent", "d_rope")] + [("softmax_scale", ctypes.c_float)]


@dataclasses.dataclass(frozen=True)
class Problem:
    """Mirror of struct dsa_problem (include/dsa.h)."""
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
    softmax_scale: Optional[float] = None

    def c(self) -> _Problem:
        scale = self.softmax_scale
        if scale is None:
            scale = 1.0 / math.sqrt(self.d_latent + self.d_rope)
        return _Problem(self.batch, self.q_len, self.kv_len, self.q_start, self.idx_heads,
                        self.idx_dim, self.topk, self.heads, self.d_latent, self.d_rope, scale)

    @classmethod
    def from_workload(cls, wl) -> "Problem":
        return cls(wl.batch, wl.q_len, wl.kv_len, wl.q_start, wl.idx_heads, wl.idx_dim,
                   wl.topk, wl.heads, wl.d_latent, wl.d_rope, wl.softmax_scale)


def _load():
    # torch ships its own HIP runtime with the same soname as the system one.
    # Import it first so libdsa.so binds to the runtime that owns torch's
    # device memory and streams (loading libdsa.so first would pull the system
    # runtime into the process and leave torch on a mismatched stack).
    import torch  # noqa: F401
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python -m sparse_attention_02_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER(_Problem)
    vp, sz, i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
    L.dsa_index_scores.argtypes = [P, vp, vp, vp, vp, vp]
    L.dsa_topk.argtypes = [P, vp, vp, vp, sz, vp]
    L.dsa_index_topk.argtypes = [P, vp, vp, vp, vp, vp, sz, vp]
    L.dsa_sparse_mla_attn.argtypes = [P, vp, vp, vp, vp, vp, vp]
    L.dsa_sparse_mla_attn_ws.argtypes = [P, vp, vp, vp, vp, vp, vp, sz, vp]
    L.dsa_masked_mha_attn.argtypes = [P, vp, vp, vp, vp, vp, vp]
    L.dsa_sparse_mla_attn_bwd.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.dsa_forward.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.dsa_forward_noalloc.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    L.dsa_warmup_target.argtypes = [P, vp, vp, vp, vp, vp, vp]
    L.dsa_warmup_kl.argtypes = [P, vp, vp, vp, vp, vp]
    L.dsa_index_scores_bwd.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp]
    for f in (L.dsa_index_scores, L.dsa_topk, L.dsa_index_topk, L.dsa_sparse_mla_attn, L.dsa_sparse_mla_attn_ws,
              L.dsa_masked_mha_attn,
              L.dsa_sparse_mla_attn_bwd, L.dsa_forward, L.dsa_forward_noalloc, L.dsa_warmup_target,
              L.dsa_warmup_kl,
              L.dsa_index_scores_bwd):
        f.restype = i32
    L.dsa_workspace_size.argtypes = [P, i32]
    L.dsa_workspace_size.restype = sz
    L.dsa_status_string.argtypes = [i32]
    L.dsa_status_string.restype = ctypes.c_char_p
    L.dsa_last_error.argtypes = []
    L.dsa_last_error.restype = ctypes.c_char_p
    return L


lib = _load()


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status: int) -> None:
    if status != 0:
        raise DsaError(status, lib.dsa_last_error().decode())


def workspace_size(problem: Problem, op: int) -> int:
    n = lib.dsa_workspace_size(ctypes.byref(problem.c()), op)
    if n == ctypes.c_size_t(-1).value:
        raise DsaError(-2, lib.dsa_last_error().decode())
    return n


def dsa_index_scores(problem: Problem, q_idx, k_idx, w, scores, stream=None) -> None:
    """scores[b,t,s] for s <= pos(t) (include/dsa.h: dsa_index_scores)."""
    _check(lib.dsa_index_scores(ctypes.byref(problem.c()), _ptr(q_idx), _ptr(k_idx), _ptr(w),
                                _ptr(scores), _stream(stream)))


def dsa_topk(problem: Problem, scores, indices, workspace=None, workspace_bytes: int = 0,
             stream=None) -> None:
    """indices[b,t,:] = ascending top-k of row (b,t), -1 padded (include/dsa.h: dsa_topk)."""
    if workspace is not None and not isinstance(workspace, int) and workspace_bytes == 0:
        workspace_bytes = workspace.numel() * workspace.element_size()
    _check(lib.dsa_topk(ctypes.byref(problem.c()), _ptr(scores), _ptr(indices), _ptr(workspace),
                        workspace_bytes, _stream(stream)))


def dsa_index_topk(problem: Problem, q_idx, k_idx, w, indices, workspace, workspace_bytes: int = 0,
                   stream=None) -> None:
    """Indexer scores and top-k without necessarily materialising the scores
    (include/dsa.h: dsa_index_topk); workspace from
    dsa_workspace_size(problem, DSA_OP_INDEX_TOPK)."""
    if workspace is not None and not isinstance(workspace, int) and workspace_bytes == 0:
        workspace_bytes = workspace.numel() * workspace.element_size()
    _check(lib.dsa_index_topk(ctypes.byref(problem.c()), _ptr(q_idx), _ptr(k_idx), _ptr(w), _ptr(indices),
                              _ptr(workspace), workspace_bytes, _stream(stream)))


def dsa_sparse_mla_attn(problem: Problem, q, kv, indices, out, lse=None, stream=None) -> None:
    """Sparse MQA-mode attention over the selected latents, one block per row
    (include/dsa.h: dsa_sparse_mla_attn)."""
    _check(lib.dsa_sparse_mla_attn(ctypes.byref(problem.c()), _ptr(q), _ptr(kv), _ptr(indices),
                                   _ptr(out), _ptr(lse), _stream(stream)))


def dsa_sparse_mla_attn_ws(problem: Problem, q, kv, indices, out, lse=None, workspace=None,
                           workspace_bytes: int = 0, stream=None) -> None:
    """The same with a workspace that lets few rows split over several blocks
    (include/dsa.h: dsa_sparse_mla_attn_ws; size from
    dsa_workspace_size(problem, DSA_OP_SPARSE_MLA_ATTN))."""
    if workspace is not None and not isinstance(workspace, int) and workspace_bytes == 0:
        workspace_bytes = workspace.numel() * workspace.element_size()
    _check(lib.dsa_sparse_mla_attn_ws(ctypes.byref(problem.c()), _ptr(q), _ptr(kv), _ptr(indices),
                                      _ptr(out), _ptr(lse), _ptr(workspace), workspace_bytes,
                                      _stream(stream)))


def dsa_sparse_mla_attn_bwd(problem: Problem, q, kv, indices, out, lse, dout, dq, dkv,
                            workspace, workspace_bytes: int = 0, stream=None) -> None:
    """dq (written) and dkv (accumulated into) of the sparse attention over fixed
    indices (include/dsa.h: dsa_sparse_mla_attn_bwd)."""
    if workspace is not None and not isinstance(workspace, int) and workspace_bytes == 0:
        workspace_bytes = workspace.numel() * workspace.element_size()
    _check(lib.dsa_sparse_mla_attn_bwd(ctypes.byref(problem.c()), _ptr(q), _ptr(kv), _ptr(indices),
                                       _ptr(out), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dkv),
                                       _ptr(workspace), workspace_bytes, _stream(stream)))


def dsa_warmup_target(problem: Problem, q, kv, target, lse_in=None, lse_out=None, stream=None) -> None:
    """The warm-up target: the main attention's distribution summed over the heads
    and divided by H, dense over s <= pos(t); lse_in skips the kernel's lse pass,
    lse_out receives it (include/dsa.h: dsa_warmup_target)."""
    _check(lib.dsa_warmup_target(ctypes.byref(problem.c()), _ptr(q), _ptr(kv), _ptr(lse_in), _ptr(lse_out),
                                 _ptr(target), _stream(stream)))


def dsa_warmup_kl(problem: Problem, scores, target, loss, dscores, stream=None) -> None:
    """KL(target || softmax(scores)) per row and its score gradient
    (include/dsa.h: dsa_warmup_kl); dscores may be scores itself."""
    _check(lib.dsa_warmup_kl(ctypes.byref(problem.c()), _ptr(scores), _ptr(target), _ptr(loss),
                             _ptr(dscores), _stream(stream)))


def dsa_index_scores_bwd(problem: Problem, q_idx, k_idx, w, dscores, dq_idx, dw, dk_idx, stream=None) -> None:
    """Gradients of the indexer scores with respect to q_I, w (written) and k_I
    (accumulated into) for a score gradient dscores
    (include/dsa.h: dsa_index_scores_bwd)."""
    _check(lib.dsa_index_scores_bwd(ctypes.byref(problem.c()), _ptr(q_idx), _ptr(k_idx), _ptr(w), _ptr(dscores),
                                    _ptr(dq_idx), _ptr(dw), _ptr(dk_idx), _stream(stream)))


def dsa_masked_mha_attn(problem: Problem, q, kv, indices, out, lse=None, stream=None) -> None:
    """The same attention computed densely over each query's causal range with the
    non-selected tokens masked (include/dsa.h: dsa_masked_mha_attn)."""
    _check(lib.dsa_masked_mha_attn(ctypes.byref(problem.c()), _ptr(q), _ptr(kv), _ptr(indices),
                                   _ptr(out), _ptr(lse), _stream(stream)))


def dsa_forward(problem: Problem, q_idx, k_idx, w, q, kv, out, lse=None, indices=None,
                workspace=None, workspace_bytes: int = 0, stream=None) -> None:
    """Indexer -> top-k -> sparse attention on one stream (include/dsa.h: dsa_forward)."""
    if workspace is not None and not isinstance(workspace, int) and workspace_bytes == 0:
        workspace_bytes = workspace.numel() * workspace.element_size()
    _check(lib.dsa_forward(ctypes.byref(problem.c()), _ptr(q_idx), _ptr(k_idx), _ptr(w), _ptr(q),
                           _ptr(kv), _ptr(out), _ptr(lse), _ptr(indices), _ptr(workspace),
                           workspace_bytes, _stream(stream)))


def dsa_forward_noalloc(problem: Problem, q_idx, k_idx, w, q, kv, out, lse=None, indices=None,
                        stream=None) -> None:
    """dsa_forward on the library's static scratch, for callers that cannot
    allocate (include/dsa.h: dsa_forward_noalloc)."""
    _check(lib.dsa_forward_noalloc(ctypes.byref(problem.c()), _ptr(q_idx), _ptr(k_idx), _ptr(w), _ptr(q),
                                   _ptr(kv), _ptr(out), _ptr(lse), _ptr(indices), _stream(stream)))


def dsa_workspace_size(problem: Problem, op: int) -> int:
    return workspace_size(problem, op)


def dsa_last_error() -> str:
    return lib.dsa_last_error().decode()


def dsa_status_string(status: int) -> str:
    return lib.dsa_status_string(status).decode()
