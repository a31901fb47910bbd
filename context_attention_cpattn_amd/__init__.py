"""Python binding of libcpattn: context-parallel causal attention on MI355X (gfx950).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in ``include/cpattn.h``; torch supplies device
memory and the stream.  Importing this package fails loudly (ImportError) if
the library has not been built -- there is no fallback path.

Tensors use the [B, S, H, D] layout with a contiguous last axis; LSE tensors
are [B, S, H].  Calls are asynchronous on ``stream`` (default: torch's current
stream of the input's device).
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "CpattnError", "LIB_PATH", "version", "partial", "merge", "ring_prefill", "ring_prefill_workspace_size",
    "ring_step", "ring_merge",
    "splitkv_decode", "splitkv_decode_workspace_size", "PASS_KV", "PASS_Q", "MAX_MERGE",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libcpattn.so")

OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP = 0, 1, 2, 3, 4
DT_BF16, DT_F32 = 0, 1
PASS_KV, PASS_Q = 0, 1
MAX_MERGE = 64
_ORDERS = {"pass_kv": PASS_KV, "pass_q": PASS_Q, PASS_KV: PASS_KV, PASS_Q: PASS_Q}


class CpattnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"cpattn status {status}: {message}")
        self.status = status
        self.message = message


class Tensor(ctypes.Structure):
    """Mirror of ``cpattn_tensor``."""

    _fields_ = [
        ("data", ctypes.c_void_p), ("dtype", ctypes.c_int32), ("reserved", ctypes.c_int32),
        ("B", ctypes.c_int64), ("S", ctypes.c_int64), ("H", ctypes.c_int64), ("D", ctypes.c_int64),
        ("stride_b", ctypes.c_int64), ("stride_s", ctypes.c_int64), ("stride_h", ctypes.c_int64),
    ]


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                          "(python context_attention_cpattn_amd/_build.py)")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER(Tensor)
    i64, i32, vp, sz = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t
    sigs = {
        "cpattn_partial": ([P, P, P, i64, i64, i32, P, P, vp], i32),
        "cpattn_merge": ([P, P, i32, P, P, vp], i32),
        "cpattn_ring_prefill_workspace_size": ([P, i32, i32, i32], sz),
        "cpattn_ring_prefill": ([P, P, P, i32, i32, i32, P, P, vp, sz, vp], i32),
        "cpattn_ring_step": ([P, P, P, i32, i32, i32, i32, vp, sz, vp], i32),
        "cpattn_ring_merge": ([i32, i32, i32, vp, sz, P, P, vp], i32),
        "cpattn_ring_prefill_fused": ([P, P, P, i32, i32, P, P, vp], i32),
        "cpattn_ring_step_accumulate": ([P, P, P, i32, i32, i32, i32, P, P, vp], i32),
        "cpattn_splitkv_decode_workspace_size": ([P, P, i32], sz),
        "cpattn_splitkv_decode": ([P, P, P, i32, P, P, vp, sz, vp], i32),
        "cpattn_last_error": ([], ctypes.c_char_p),
        "cpattn_version": ([], ctypes.c_char_p),
    }
    for name, (args, res) in sigs.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    return lib


lib = _load()


def version() -> str:
    return lib.cpattn_version().decode()


def _check(status: int) -> None:
    if status != OK:
        raise CpattnError(status, lib.cpattn_last_error().decode())


def describe(t: torch.Tensor | None, lse: bool = False):
    """Build a cpattn_tensor for a [B,S,H,D] tensor (or [B,S,H] when ``lse``)."""
    if t is None:
        return None
    if t.dtype == torch.bfloat16:
        dt = DT_BF16
    elif t.dtype == torch.float32:
        dt = DT_F32
    else:
        raise TypeError(f"unsupported dtype {t.dtype}")
    if lse:
        if t.dim() != 3:
            raise ValueError("LSE tensors are [B, S, H]")
        B, S, H = t.shape
        D = 1
        sb, ss, sh = t.stride()
    else:
        if t.dim() != 4:
            raise ValueError("tensors are [B, S, H, D]")
        B, S, H, D = t.shape
        if D > 1 and t.stride(3) != 1:
            raise ValueError("the last (D) axis must be contiguous")
        sb, ss, sh = t.stride()[:3]
    return Tensor(t.data_ptr() if t.numel() else None, dt, 0, B, S, H, D, sb, ss, sh)


def _ref(x):
    return ctypes.byref(x) if x is not None else None


def _stream(t: torch.Tensor, stream) -> int | None:
    if stream is None:
        return torch.cuda.current_stream(t.device).cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def partial(q, k, v, q_offset: int = 0, kv_offset: int = 0, causal: bool = True, out=None, lse=None, stream=None):
    """Attention of q against one K/V block at global offsets -> (O fp32, LSE fp32)."""
    B, S, H, D = q.shape
    if out is None:
        out = torch.empty(B, S, H, D, dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty(B, S, H, dtype=torch.float32, device=q.device)
    dq, dk, dv, do, dl = describe(q), describe(k), describe(v), describe(out), describe(lse, True)
    _check(lib.cpattn_partial(_ref(dq), _ref(dk), _ref(dv), int(q_offset), int(kv_offset), int(bool(causal)),
                              _ref(do), _ref(dl), _stream(q, stream)))
    return out, lse


def merge(partials, lses, out=None, out_lse=None, out_dtype=torch.float32, want_lse: bool = True, stream=None):
    """Log-sum-exp merge of partial (O, LSE) pairs, in the order given."""
    n = len(partials)
    if n != len(lses):
        raise ValueError("partials and lses differ in length")
    p0 = partials[0]
    if out is None:
        out = torch.empty(p0.shape, dtype=out_dtype, device=p0.device)
    if out_lse is None and want_lse:
        out_lse = torch.empty(p0.shape[:3], dtype=torch.float32, device=p0.device)
    arr_p = (Tensor * n)(*[describe(p) for p in partials])
    arr_l = (Tensor * n)(*[describe(x, True) for x in lses])
    do, dl = describe(out), describe(out_lse, True)
    _check(lib.cpattn_merge(arr_p, arr_l, n, _ref(do), _ref(dl), _stream(p0, stream)))
    return out, out_lse


def ring_prefill_workspace_size(q, n_chunks: int, order="pass_kv", causal: bool = True) -> int:
    n = lib.cpattn_ring_prefill_workspace_size(_ref(describe(q)), int(n_chunks), _ORDERS[order], int(bool(causal)))
    if n == 0 and q.numel():
        raise CpattnError(ERR_INVALID_ARG, lib.cpattn_last_error().decode())
    return n


def ring_prefill(q, k, v, n_chunks: int, order="pass_kv", causal: bool = True, out=None, lse=None,
                 workspace=None, out_dtype=torch.float32, want_lse: bool = True, stream=None):
    """Full causal attention of a sequence split into ``n_chunks`` CP chunks, by ring order."""
    B, S, H, D = q.shape
    if out is None:
        out = torch.empty(B, S, H, D, dtype=out_dtype, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty(B, S, H, dtype=torch.float32, device=q.device)
    need = ring_prefill_workspace_size(q, n_chunks, order, causal)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    dq, dk, dv, do, dl = describe(q), describe(k), describe(v), describe(out), describe(lse, True)
    _check(lib.cpattn_ring_prefill(_ref(dq), _ref(dk), _ref(dv), int(n_chunks), _ORDERS[order], int(bool(causal)),
                                   _ref(do), _ref(dl), workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                                   _stream(q, stream)))
    return out, lse


def ring_prefill_fused(q, k, v, n_chunks: int, causal: bool = True, out=None, lse=None, want_lse: bool = True,
                       stream=None):
    """The ring prefill with the merge done online: one launch, no workspace, fp32 output."""
    B, S, H, D = q.shape
    if out is None:
        out = torch.empty(B, S, H, D, dtype=torch.float32, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty(B, S, H, dtype=torch.float32, device=q.device)
    dq, dk, dv, do, dl = describe(q), describe(k), describe(v), describe(out), describe(lse, True)
    _check(lib.cpattn_ring_prefill_fused(_ref(dq), _ref(dk), _ref(dv), int(n_chunks), int(bool(causal)),
                                         _ref(do), _ref(dl), _stream(q, stream)))
    return out, lse


def ring_step(q, k, v, n_chunks: int, step: int, workspace, order="pass_kv", causal: bool = True, stream=None):
    """Partial attention of every rank's pair at ring step ``step`` into ``workspace``."""
    dq, dk, dv = describe(q), describe(k), describe(v)
    _check(lib.cpattn_ring_step(_ref(dq), _ref(dk), _ref(dv), int(n_chunks), _ORDERS[order], int(bool(causal)),
                                int(step), workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                                _stream(q, stream)))


def ring_step_accumulate(q, k, v, n_chunks: int, step: int, out, lse, order="pass_kv", causal: bool = True,
                         stream=None):
    """Ring step ``step`` with each pair's partial merged into the running ``out``/``lse`` (fp32):
    step 0 writes, later steps merge; after steps 0..n_chunks-1 they hold the full result."""
    dq, dk, dv, do, dl = describe(q), describe(k), describe(v), describe(out), describe(lse, True)
    _check(lib.cpattn_ring_step_accumulate(_ref(dq), _ref(dk), _ref(dv), int(n_chunks), _ORDERS[order],
                                           int(bool(causal)), int(step), _ref(do), _ref(dl), _stream(q, stream)))
    return out, lse


def ring_merge(n_chunks: int, workspace, out, lse=None, order="pass_kv", causal: bool = True, stream=None):
    """Merge each Q chunk's partials (filled by ``ring_step`` over all steps) into ``out``/``lse``."""
    do, dl = describe(out), describe(lse, True)
    _check(lib.cpattn_ring_merge(int(n_chunks), _ORDERS[order], int(bool(causal)), workspace.data_ptr(),
                                 workspace.numel() * workspace.element_size(), _ref(do), _ref(dl),
                                 _stream(out, stream)))
    return out, lse


def splitkv_decode_workspace_size(q, k, n_chunks: int) -> int:
    n = lib.cpattn_splitkv_decode_workspace_size(_ref(describe(q)), _ref(describe(k)), int(n_chunks))
    if n == 0 and q.numel():
        raise CpattnError(ERR_INVALID_ARG, lib.cpattn_last_error().decode())
    return n


def splitkv_decode(q, k, v, n_chunks: int, out=None, lse=None, workspace=None, out_dtype=torch.float32,
                   want_lse: bool = True, stream=None):
    """One new token per sequence against a cached K/V split into ``n_chunks`` chunks."""
    B, S, H, D = q.shape
    if out is None:
        out = torch.empty(B, S, H, D, dtype=out_dtype, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty(B, S, H, dtype=torch.float32, device=q.device)
    need = splitkv_decode_workspace_size(q, k, n_chunks)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    dq, dk, dv, do, dl = describe(q), describe(k), describe(v), describe(out), describe(lse, True)
    _check(lib.cpattn_splitkv_decode(_ref(dq), _ref(dk), _ref(dv), int(n_chunks), _ref(do), _ref(dl),
                                     workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                                     _stream(q, stream)))
    return out, lse
