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
    "CpattnError", "Tensor", "LIB_PATH", "version", "describe", "partial", "merge",
    "ring_prefill", "ring_prefill_workspace_size", "ring_prefill_fused", "ring_select_order",
    "ring_step", "ring_step_accumulate", "ring_merge",
    "splitkv_decode", "splitkv_decode_workspace_size", "splitkv_decode_noalloc",
    "kv_cache_write", "kv_cache_append", "cp_decode", "cp_decode_workspace_size",
    "PASS_KV", "PASS_Q", "ORDER_AUTO", "MAX_MERGE",
]

# The in-tree library; CPATTN_LIB names another build of the same sources (the host-sanitizer build
# that the CPU ABI tests run against).
LIB_PATH = os.environ.get("CPATTN_LIB") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libcpattn.so")

OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP = 0, 1, 2, 3, 4
DT_BF16, DT_F32 = 0, 1
PASS_KV, PASS_Q, ORDER_AUTO = 0, 1, 2
MAX_MERGE = 64
_ORDERS = {"pass_kv": PASS_KV, "pass_q": PASS_Q, "auto": ORDER_AUTO, PASS_KV: PASS_KV, PASS_Q: PASS_Q,
           ORDER_AUTO: ORDER_AUTO}
_ORDER_NAMES = {PASS_KV: "pass_kv", PASS_Q: "pass_q"}


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
        "cpattn_ring_prefill_workspace_size": ([P, P, i32, i32], sz),
        "cpattn_ring_select_order": ([P, P, i32, i32, ctypes.POINTER(ctypes.c_int), ctypes.POINTER(ctypes.c_uint64),
                                      ctypes.POINTER(ctypes.c_uint64)], i32),
        "cpattn_ring_prefill": ([P, P, P, i32, i32, i32, P, P, vp, sz, vp], i32),
        "cpattn_ring_step": ([P, P, P, i32, i32, i32, i32, vp, sz, vp], i32),
        "cpattn_ring_merge": ([i32, i32, i32, i64, vp, sz, P, P, vp], i32),
        "cpattn_ring_prefill_fused": ([P, P, P, i32, i32, P, P, vp], i32),
        "cpattn_ring_step_accumulate": ([P, P, P, i32, i32, i32, i32, P, P, vp], i32),
        "cpattn_splitkv_decode_workspace_size": ([P, P, i32], sz),
        "cpattn_splitkv_decode": ([P, P, P, i32, P, P, vp, sz, vp], i32),
        "cpattn_splitkv_decode_noalloc": ([P, P, P, i32, P, P, vp], i32),
        "cpattn_kv_cache_write": ([P, P, i32, P, P, vp], i32),
        "cpattn_kv_cache_append": ([P, P, P, P, i64, vp], i32),
        "cpattn_cp_decode_workspace_size": ([P, P, i32], sz),
        "cpattn_cp_decode": ([P, P, P, ctypes.POINTER(ctypes.c_int64), i32, P, P, vp, sz, vp], i32),
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


def _stream(t: torch.Tensor, stream):
    """(raw hipStream_t handle, the torch stream object when it is not torch's current stream).

    ``stream`` may be None (torch's current stream of ``t``'s device), a torch
    stream, or a raw handle."""
    cur = torch.cuda.current_stream(t.device)
    if stream is None:
        return cur.cuda_stream, None
    if not isinstance(stream, torch.cuda.Stream):
        handle = int(stream)
        if handle == cur.cuda_stream:
            return handle, None
        stream = torch.cuda.ExternalStream(handle, device=t.device)
    if stream.cuda_stream == cur.cuda_stream:
        return stream.cuda_stream, None
    return stream.cuda_stream, stream


def _keep(side, *tensors) -> None:
    """Buffers this binding allocated on torch's current stream but handed to kernels on another
    stream: tell the caching allocator, so it does not reuse them while those kernels run."""
    if side is not None:
        for t in tensors:
            if t is not None and t.is_cuda:
                t.record_stream(side)


def _nbytes(t: torch.Tensor) -> int:
    return t.numel() * t.element_size()


def partial(q, k, v, q_offset: int = 0, kv_offset: int = 0, causal: bool = True, out=None, lse=None, stream=None):
    """Attention of q against one K/V block at global offsets -> (O fp32, LSE fp32)."""
    B, S, H, D = q.shape
    h, side = _stream(q, stream)
    if out is None:
        out = torch.empty(B, S, H, D, dtype=torch.float32, device=q.device)
        _keep(side, out)
    if lse is None:
        lse = torch.empty(B, S, H, dtype=torch.float32, device=q.device)
        _keep(side, lse)
    dq, dk, dv, do, dl = describe(q), describe(k), describe(v), describe(out), describe(lse, True)
    _check(lib.cpattn_partial(_ref(dq), _ref(dk), _ref(dv), int(q_offset), int(kv_offset), int(bool(causal)),
                              _ref(do), _ref(dl), h))
    return out, lse


def merge(partials, lses, out=None, out_lse=None, out_dtype=torch.float32, want_lse: bool = True, stream=None):
    """Log-sum-exp merge of partial (O, LSE) pairs, in the order given."""
    n = len(partials)
    if n != len(lses):
        raise ValueError("partials and lses differ in length")
    p0 = partials[0]
    h, side = _stream(p0, stream)
    if out is None:
        out = torch.empty(p0.shape, dtype=out_dtype, device=p0.device)
        _keep(side, out)
    if out_lse is None and want_lse:
        out_lse = torch.empty(p0.shape[:3], dtype=torch.float32, device=p0.device)
        _keep(side, out_lse)
    arr_p = (Tensor * n)(*[describe(p) for p in partials])
    arr_l = (Tensor * n)(*[describe(x, True) for x in lses])
    do, dl = describe(out), describe(out_lse, True)
    _check(lib.cpattn_merge(arr_p, arr_l, n, _ref(do), _ref(dl), h))
    return out, out_lse


def ring_prefill_workspace_size(q, n_chunks: int, causal: bool = True, k=None) -> int:
    """Workspace bytes of a ring over q and K/V of ``k``'s length (default: q's)."""
    n = lib.cpattn_ring_prefill_workspace_size(_ref(describe(q)), _ref(describe(k)), int(n_chunks),
                                               int(bool(causal)))
    if n == 0 and q.numel():
        raise CpattnError(ERR_INVALID_ARG, lib.cpattn_last_error().decode())
    return n


def ring_select_order(q, k, n_chunks: int, causal: bool = True):
    """The ring order moving fewer bytes between ranks: ("pass_kv" | "pass_q", bytes Pass-KV, bytes Pass-Q)."""
    order, bkv, bq = ctypes.c_int(), ctypes.c_uint64(), ctypes.c_uint64()
    _check(lib.cpattn_ring_select_order(_ref(describe(q)), _ref(describe(k)), int(n_chunks), int(bool(causal)),
                                        ctypes.byref(order), ctypes.byref(bkv), ctypes.byref(bq)))
    return _ORDER_NAMES[order.value], bkv.value, bq.value


def ring_prefill(q, k, v, n_chunks: int, order="pass_kv", causal: bool = True, out=None, lse=None,
                 workspace=None, out_dtype=torch.float32, want_lse: bool = True, stream=None):
    """Attention of q (the last q.S positions) over the whole K/V sequence, split into ``n_chunks``
    CP chunks, by ring order ("pass_kv", "pass_q" or "auto")."""
    B, S, H, D = q.shape
    h, side = _stream(q, stream)
    if out is None:
        out = torch.empty(B, S, H, D, dtype=out_dtype, device=q.device)
        _keep(side, out)
    if lse is None and want_lse:
        lse = torch.empty(B, S, H, dtype=torch.float32, device=q.device)
        _keep(side, lse)
    need = ring_prefill_workspace_size(q, n_chunks, causal, k)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
        _keep(side, workspace)
    dq, dk, dv, do, dl = describe(q), describe(k), describe(v), describe(out), describe(lse, True)
    _check(lib.cpattn_ring_prefill(_ref(dq), _ref(dk), _ref(dv), int(n_chunks), _ORDERS[order], int(bool(causal)),
                                   _ref(do), _ref(dl), workspace.data_ptr(), _nbytes(workspace), h))
    return out, lse


def ring_prefill_fused(q, k, v, n_chunks: int, causal: bool = True, out=None, lse=None, want_lse: bool = True,
                       stream=None):
    """The ring prefill with the merge done online: one launch, no workspace, fp32 output."""
    B, S, H, D = q.shape
    h, side = _stream(q, stream)
    if out is None:
        out = torch.empty(B, S, H, D, dtype=torch.float32, device=q.device)
        _keep(side, out)
    if lse is None and want_lse:
        lse = torch.empty(B, S, H, dtype=torch.float32, device=q.device)
        _keep(side, lse)
    dq, dk, dv, do, dl = describe(q), describe(k), describe(v), describe(out), describe(lse, True)
    _check(lib.cpattn_ring_prefill_fused(_ref(dq), _ref(dk), _ref(dv), int(n_chunks), int(bool(causal)),
                                         _ref(do), _ref(dl), h))
    return out, lse


def ring_step(q, k, v, n_chunks: int, step: int, workspace, order="pass_kv", causal: bool = True, stream=None):
    """Partial attention of every rank's pair at ring step ``step`` into ``workspace``."""
    dq, dk, dv = describe(q), describe(k), describe(v)
    h, _ = _stream(q, stream)
    _check(lib.cpattn_ring_step(_ref(dq), _ref(dk), _ref(dv), int(n_chunks), _ORDERS[order], int(bool(causal)),
                                int(step), workspace.data_ptr(), _nbytes(workspace), h))


def ring_step_accumulate(q, k, v, n_chunks: int, step: int, out, lse, order="pass_kv", causal: bool = True,
                         stream=None):
    """Ring step ``step`` with each pair's partial merged into the running ``out``/``lse`` (fp32):
    step 0 writes, later steps merge; after steps 0..n_chunks-1 they hold the full result."""
    dq, dk, dv, do, dl = describe(q), describe(k), describe(v), describe(out), describe(lse, True)
    h, _ = _stream(q, stream)
    _check(lib.cpattn_ring_step_accumulate(_ref(dq), _ref(dk), _ref(dv), int(n_chunks), _ORDERS[order],
                                           int(bool(causal)), int(step), _ref(do), _ref(dl), h))
    return out, lse


def ring_merge(n_chunks: int, workspace, out, lse=None, order="pass_kv", causal: bool = True, kv_len=None,
               stream=None):
    """Merge each Q chunk's partials (filled by ``ring_step`` over all steps) into ``out``/``lse``;
    ``kv_len`` is the K/V length the steps ran with (default: the output's length)."""
    do, dl = describe(out), describe(lse, True)
    h, _ = _stream(out, stream)
    kv_len = out.shape[1] if kv_len is None else int(kv_len)
    _check(lib.cpattn_ring_merge(int(n_chunks), _ORDERS[order], int(bool(causal)), kv_len, workspace.data_ptr(),
                                 _nbytes(workspace), _ref(do), _ref(dl), h))
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
    h, side = _stream(q, stream)
    if out is None:
        out = torch.empty(B, S, H, D, dtype=out_dtype, device=q.device)
        _keep(side, out)
    if lse is None and want_lse:
        lse = torch.empty(B, S, H, dtype=torch.float32, device=q.device)
        _keep(side, lse)
    need = splitkv_decode_workspace_size(q, k, n_chunks)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
        _keep(side, workspace)
    dq, dk, dv, do, dl = describe(q), describe(k), describe(v), describe(out), describe(lse, True)
    _check(lib.cpattn_splitkv_decode(_ref(dq), _ref(dk), _ref(dv), int(n_chunks), _ref(do), _ref(dl),
                                     workspace.data_ptr(), _nbytes(workspace), h))
    return out, lse


def splitkv_decode_noalloc(q, k, v, n_chunks: int, out, lse=None, stream=None):
    """``splitkv_decode`` with the partials in the library's fixed 64 MiB scratch: the C call
    allocates nothing (``out``/``lse`` are the caller's).  Calls that overlap on one GPU race."""
    h, _ = _stream(q, stream)
    _check(lib.cpattn_splitkv_decode_noalloc(_ref(describe(q)), _ref(describe(k)), _ref(describe(v)), int(n_chunks),
                                             _ref(describe(out)), _ref(describe(lse, True)), h))
    return out, lse


def _shard_array(shards):
    return (Tensor * len(shards))(*[describe(x) for x in shards])


def kv_cache_write(k, v, n_chunks: int, k_shards, v_shards, stream=None) -> None:
    """Rows [rC, (r+1)C) of k/v into rows [0, C) of shard r (C = S / n_chunks)."""
    if len(k_shards) != n_chunks or len(v_shards) != n_chunks:
        raise ValueError("need one K and one V shard per chunk")
    h, _ = _stream(k, stream)
    _check(lib.cpattn_kv_cache_write(_ref(describe(k)), _ref(describe(v)), int(n_chunks), _shard_array(k_shards),
                                     _shard_array(v_shards), h))


def kv_cache_append(k_new, v_new, k_shard, v_shard, row: int, stream=None) -> None:
    """New tokens' K/V [B, T, Hkv, D] into rows [row, row + T) of one shard."""
    h, _ = _stream(k_new, stream)
    _check(lib.cpattn_kv_cache_append(_ref(describe(k_new)), _ref(describe(v_new)), _ref(describe(k_shard)),
                                      _ref(describe(v_shard)), int(row), h))


def cp_decode_workspace_size(q, k_shards) -> int:
    n = lib.cpattn_cp_decode_workspace_size(_ref(describe(q)), _shard_array(k_shards), len(k_shards))
    if n == 0 and q.numel():
        raise CpattnError(ERR_INVALID_ARG, lib.cpattn_last_error().decode())
    return n


def cp_decode(q, k_shards, v_shards, lengths, out=None, lse=None, workspace=None, out_dtype=torch.float32,
              want_lse: bool = True, stream=None):
    """One new token per sequence against a KV cache sharded over CP ranks: shard r contributes
    its first ``lengths[r]`` rows; the per-shard partials are merged."""
    n = len(k_shards)
    if len(v_shards) != n or len(lengths) != n:
        raise ValueError("k_shards, v_shards and lengths differ in length")
    B, S, H, D = q.shape
    h, side = _stream(q, stream)
    if out is None:
        out = torch.empty(B, S, H, D, dtype=out_dtype, device=q.device)
        _keep(side, out)
    if lse is None and want_lse:
        lse = torch.empty(B, S, H, dtype=torch.float32, device=q.device)
        _keep(side, lse)
    need = cp_decode_workspace_size(q, k_shards)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
        _keep(side, workspace)
    lens = (ctypes.c_int64 * n)(*[int(x) for x in lengths])
    _check(lib.cpattn_cp_decode(_ref(describe(q)), _shard_array(k_shards), _shard_array(v_shards), lens, n,
                                _ref(describe(out)), _ref(describe(lse, True)), workspace.data_ptr(),
                                _nbytes(workspace), h))
    return out, lse
