"""C ABI checks that need no GPU: the library loads, exports what the header
declares, and every argument check fails before any HIP call.

Only invalid calls are made here (plus zero-size no-ops), so no kernel is
ever launched; the fake device pointers are never dereferenced.  On a machine
with a visible GPU these tests are skipped, since a validation bug there could
turn a fake pointer into a real launch.
"""
import ctypes
import os
import re

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "cpattn.h")

cp = pytest.importorskip("context_attention_cpattn_amd")
T = cp.Tensor
lib = cp.lib

no_gpu = pytest.mark.skipif(torch.cuda.is_available(), reason="validation probes use fake device pointers")

FAKE = 0x100000  # 16-byte aligned, never dereferenced


def header_symbols():
    txt = open(HEADER).read()
    return sorted(set(re.findall(r"^\w[\w\s\*]*?\b(cpattn_\w+)\s*\(", txt, flags=re.M)))


def test_exports_every_declared_symbol():
    syms = header_symbols()
    assert {"cpattn_partial", "cpattn_merge", "cpattn_ring_prefill", "cpattn_ring_prefill_workspace_size",
            "cpattn_splitkv_decode", "cpattn_splitkv_decode_workspace_size", "cpattn_last_error",
            "cpattn_version", "cpattn_ring_select_order", "cpattn_kv_cache_write", "cpattn_kv_cache_append",
            "cpattn_cp_decode", "cpattn_cp_decode_workspace_size"} <= set(syms)
    raw = ctypes.CDLL(cp.LIB_PATH)
    for s in syms:
        assert hasattr(raw, s), f"{s} declared in cpattn.h but not exported"
    # and nothing else: every exported cpattn_ symbol is declared
    import subprocess
    nm = subprocess.run(["nm", "-D", "--defined-only", cp.LIB_PATH], capture_output=True, text=True)
    if nm.returncode == 0:
        exported = set(re.findall(r"\bT (cpattn_\w+)", nm.stdout))
        assert exported == set(syms), exported ^ set(syms)


def test_version():
    v = cp.version()
    assert v.startswith("cpattn ") and "gfx950" in v


def bshd(B, S, H, D, dt=cp.DT_BF16, ptr=FAKE):
    return T(ptr, dt, 0, B, S, H, D, S * H * D, H * D, D)


def lse_of(B, S, H, ptr=FAKE):
    return T(ptr, cp.DT_F32, 0, B, S, H, 1, S * H, H, 1)


def call_partial(q, k, v, out, lse, qo=0, ko=0, causal=1):
    r = ctypes.byref
    return lib.cpattn_partial(r(q) if q else None, r(k), r(v), qo, ko, causal, r(out), r(lse) if lse else None, None)


def err():
    return lib.cpattn_last_error().decode()


@no_gpu
def test_partial_validation():
    q, k, v = bshd(1, 64, 4, 128), bshd(1, 64, 2, 128), bshd(1, 64, 2, 128)
    out, lse = bshd(1, 64, 4, 128, cp.DT_F32), lse_of(1, 64, 4)
    assert call_partial(None, k, v, out, lse) == cp.ERR_INVALID_ARG and "NULL" in err()
    assert call_partial(q, k, v, out, None) == cp.ERR_INVALID_ARG
    # dtype mismatch
    assert call_partial(q, bshd(1, 64, 2, 128, cp.DT_F32), v, out, lse) == cp.ERR_INVALID_ARG
    # unsupported head dim
    assert call_partial(bshd(1, 64, 4, 96), bshd(1, 64, 2, 96), bshd(1, 64, 2, 96),
                        bshd(1, 64, 4, 96, cp.DT_F32), lse) == cp.ERR_UNSUPPORTED
    # Hq not a multiple of Hkv
    assert call_partial(bshd(1, 64, 3, 128), k, v, bshd(1, 64, 3, 128, cp.DT_F32),
                        lse_of(1, 64, 3)) == cp.ERR_INVALID_ARG and "multiple" in err()
    # misaligned pointer and stride
    assert call_partial(bshd(1, 64, 4, 128, ptr=FAKE + 8), k, v, out, lse) == cp.ERR_INVALID_ARG
    bad = bshd(1, 64, 4, 128)
    bad.stride_s = 4 * 128 + 4
    assert call_partial(bad, k, v, out, lse) == cp.ERR_INVALID_ARG and "multiples" in err()
    # partial output must be F32, lse must be [B,S,H] with D == 1
    assert call_partial(q, k, v, bshd(1, 64, 4, 128, cp.DT_BF16), lse) == cp.ERR_INVALID_ARG
    bad_lse = lse_of(1, 64, 4)
    bad_lse.D = 2
    assert call_partial(q, k, v, out, bad_lse) == cp.ERR_INVALID_ARG
    assert call_partial(q, k, v, out, lse_of(1, 63, 4)) == cp.ERR_INVALID_ARG
    # offsets, mask flag, reserved field, unknown dtype, negative size
    assert call_partial(q, k, v, out, lse, qo=-1) == cp.ERR_INVALID_ARG
    assert call_partial(q, k, v, out, lse, causal=2) == cp.ERR_INVALID_ARG
    r = bshd(1, 64, 4, 128)
    r.reserved = 1
    assert call_partial(r, k, v, out, lse) == cp.ERR_INVALID_ARG
    assert call_partial(bshd(1, 64, 4, 128, dt=7), k, v, out, lse) == cp.ERR_INVALID_ARG
    assert call_partial(bshd(1, -1, 4, 128), k, v, out, lse) == cp.ERR_INVALID_ARG
    # batch mismatch, k/v mismatch
    assert call_partial(q, bshd(2, 64, 2, 128), v, out, lse) == cp.ERR_INVALID_ARG
    assert call_partial(q, k, bshd(1, 65, 2, 128), out, lse) == cp.ERR_INVALID_ARG
    # K/V token strides beyond 2^24 elements
    wide_k, wide_v = bshd(1, 64, 2, 128), bshd(1, 64, 2, 128)
    wide_k.stride_s = wide_v.stride_s = (1 << 24) + 8
    assert call_partial(q, wide_k, wide_v, out, lse) == cp.ERR_UNSUPPORTED and "2^24" in err()


@no_gpu
def test_partial_empty_is_a_noop():
    q = bshd(1, 0, 4, 128, ptr=None)
    out = bshd(1, 0, 4, 128, cp.DT_F32, ptr=None)
    lse = lse_of(1, 0, 4, ptr=None)
    assert call_partial(q, bshd(1, 64, 2, 128), bshd(1, 64, 2, 128), out, lse) == cp.OK


@no_gpu
def test_merge_validation():
    r = ctypes.byref
    P = (T * 2)(bshd(1, 8, 2, 64, cp.DT_F32), bshd(1, 8, 2, 64, cp.DT_F32))
    L = (T * 2)(lse_of(1, 8, 2), lse_of(1, 8, 2))
    out = bshd(1, 8, 2, 64, cp.DT_F32)
    assert lib.cpattn_merge(P, L, 0, r(out), None, None) == cp.ERR_INVALID_ARG
    assert lib.cpattn_merge(P, L, cp.MAX_MERGE + 1, r(out), None, None) == cp.ERR_INVALID_ARG
    assert lib.cpattn_merge(None, L, 2, r(out), None, None) == cp.ERR_INVALID_ARG
    P2 = (T * 2)(bshd(1, 8, 2, 64, cp.DT_F32), bshd(1, 9, 2, 64, cp.DT_F32))
    assert lib.cpattn_merge(P2, L, 2, r(out), None, None) == cp.ERR_INVALID_ARG and "partial 1" in err()
    P3 = (T * 2)(bshd(1, 8, 2, 64, cp.DT_F32), bshd(1, 8, 2, 64, cp.DT_BF16))
    assert lib.cpattn_merge(P3, L, 2, r(out), None, None) == cp.ERR_INVALID_ARG
    assert lib.cpattn_merge(P, L, 2, r(bshd(1, 8, 2, 128, cp.DT_F32)), None, None) == cp.ERR_INVALID_ARG
    P4 = (T * 1)(bshd(1, 8, 2, 32, cp.DT_F32))
    assert lib.cpattn_merge(P4, L, 1, r(bshd(1, 8, 2, 32, cp.DT_F32)), None, None) == cp.ERR_UNSUPPORTED


def ring_ws(q, n, causal=1, k=None):
    return lib.cpattn_ring_prefill_workspace_size(ctypes.byref(q), ctypes.byref(k) if k is not None else None, n,
                                                  causal)


def test_ring_workspace_size_formula():
    # 128K-token shape, 16 chunks: 136 causal items, each fp32 O [1, 8192, 16, 128] and LSE [1, 8192, 16]
    q = bshd(1, 131072, 16, 128)
    n_items = 16 * 17 // 2
    o = n_items * 8192 * 16 * 128 * 4
    l = n_items * 8192 * 16 * 4
    up = lambda x: (x + 255) // 256 * 256
    assert ring_ws(q, 16) == up(o) + up(l)
    assert ring_ws(q, 16, k=bshd(1, 131072, 1, 128)) == up(o) + up(l)
    assert ring_ws(q, 16, causal=0) == up(256 * 8192 * 16 * 128 * 4) + up(256 * 8192 * 16 * 4)
    assert ring_ws(q, 3) == 0 and "divide" in err()
    assert ring_ws(q, 0) == 0
    assert ring_ws(q, 16, causal=5) == 0
    # K/V shorter than Q is refused; longer K/V must also divide into the chunks
    assert ring_ws(q, 16, k=bshd(1, 65536, 1, 128)) == 0 and "at least as long" in err()
    assert ring_ws(q, 16, k=bshd(1, 131080, 1, 128)) == 0


@pytest.mark.parametrize("Sq,Skv,P", [(2048, 133120, 16), (2048, 4096, 4), (96, 960, 3), (512, 512, 8),
                                      (64, 64 * 40, 64), (256, 1024, 1)])
def test_ring_workspace_slots_are_the_oracles_visible_pairs(Sq, Skv, P):
    """Queries shorter than K/V: one slot per pair the oracle's schedule visits (its visibility is
    decided from positions)."""
    import oracle
    q, k = bshd(1, Sq, 2, 64), bshd(1, Skv, 1, 64)
    up = lambda x: (x + 255) // 256 * 256
    for causal in (1, 0):
        n = sum(len(st) for st in oracle.schedule(P, oracle.PASS_KV, bool(causal), Sq, Skv))
        C = Sq // P
        assert ring_ws(q, P, causal, k) == up(n * C * 2 * 64 * 4) + up(n * C * 2 * 4)


def select(q, k, n, causal=1):
    order, bkv, bq = ctypes.c_int(-1), ctypes.c_uint64(), ctypes.c_uint64()
    st = lib.cpattn_ring_select_order(ctypes.byref(q), ctypes.byref(k), n, causal, ctypes.byref(order),
                                      ctypes.byref(bkv), ctypes.byref(bq))
    return st, order.value, bkv.value, bq.value


@pytest.mark.parametrize("shape", [(1, 131072, 131072, 16, 1, 128, 16), (1, 2048, 133120, 16, 1, 128, 16),
                                   (2, 512, 512, 8, 8, 64, 8), (3, 96, 960, 4, 2, 64, 3), (1, 64, 8192, 32, 8, 128, 4),
                                   (4, 1024, 4096, 16, 4, 128, 2), (1, 8, 8, 2, 1, 64, 1), (1, 4, 64, 64, 1, 128, 4)])
@pytest.mark.parametrize("dt", [cp.DT_BF16, cp.DT_F32])
def test_select_order_matches_the_oracle_walk(shape, dt):
    """The library's closed-form byte counts and choice equal the oracle's step-by-step walk of the
    ring (no device call is made)."""
    import oracle
    B, Sq, Skv, Hq, Hkv, D, P = shape
    e = 2 if dt == cp.DT_BF16 else 4
    for causal in (1, 0):
        st, order, bkv, bq = select(bshd(B, Sq, Hq, D, dt), bshd(B, Skv, Hkv, D, dt), P, causal)
        assert st == cp.OK
        assert bkv == oracle.exchange_bytes(P, oracle.PASS_KV, bool(causal), B, Sq, Skv, Hq, Hkv, D, e)
        assert bq == oracle.exchange_bytes(P, oracle.PASS_Q, bool(causal), B, Sq, Skv, Hq, Hkv, D, e)
        want = oracle.select_order(P, bool(causal), B, Sq, Skv, Hq, Hkv, D, e)
        assert order == (cp.PASS_Q if want == oracle.PASS_Q else cp.PASS_KV)


def test_select_order_validation():
    q, k = bshd(1, 512, 4, 64), bshd(1, 1024, 1, 64)
    assert select(q, k, 4)[0] == cp.OK
    assert select(q, k, 3)[0] == cp.ERR_INVALID_ARG
    assert select(q, bshd(1, 256, 1, 64), 4)[0] == cp.ERR_INVALID_ARG
    assert select(q, bshd(1, 1024, 3, 64), 4)[0] == cp.ERR_INVALID_ARG
    assert select(q, bshd(1, 1024, 1, 64, cp.DT_F32), 4)[0] == cp.ERR_INVALID_ARG
    assert lib.cpattn_ring_select_order(ctypes.byref(q), ctypes.byref(k), 4, 1, None, None, None) == cp.ERR_INVALID_ARG


def test_decode_workspace_size():
    """Partials per call: n_chunks x sub-splits, the sub-splits doubling while the grid has fewer
    than 1024 units, each sub-split keeps >= 256 keys, and the merge takes <= 64 partials."""
    def ws(B, Skv, Hq, Hkv, D, n):
        q, k = bshd(B, 1, Hq, D), bshd(B, Skv, Hkv, D)
        return lib.cpattn_splitkv_decode_workspace_size(ctypes.byref(q), ctypes.byref(k), n)
    up = lambda x: (x + 255) // 256 * 256
    size = lambda n_part, B, Hq, D: up(n_part * B * Hq * D * 4) + up(n_part * B * Hq * 4)
    assert ws(128, 32768, 16, 1, 128, 8) == size(8, 128, 16, 128)    # 1024 units already: no sub-split
    assert ws(1, 32768, 16, 1, 128, 8) == size(64, 1, 16, 128)       # 8 sub-splits: 8 x 8 = 64 partials, the limit
    assert ws(4, 2048, 16, 1, 128, 4) == size(8, 4, 16, 128)         # 512-key chunks: 2 sub-splits of 256
    assert ws(2, 96, 8, 2, 64, 3) == size(3, 2, 8, 64)               # chunks too short to split
    assert ws(2, 100, 8, 2, 64, 3) == 0 and "divide" in err()


@no_gpu
def test_ring_validation():
    r = ctypes.byref
    q, k, v = bshd(1, 512, 4, 64), bshd(1, 512, 1, 64), bshd(1, 512, 1, 64)
    out, lse = bshd(1, 512, 4, 64, cp.DT_F32), lse_of(1, 512, 4)
    need = ring_ws(q, 4)
    assert need > 0

    def call(n=4, order=0, causal=1, ws=FAKE, nbytes=None, k_=k, out_=out):
        v_ = bshd(k_.B, k_.S, k_.H, k_.D, k_.dtype)  # v shaped like k
        return lib.cpattn_ring_prefill(r(q), r(k_), r(v_), n, order, causal, r(out_), r(lse), ws,
                                       need if nbytes is None else nbytes, None)

    assert call(n=3) == cp.ERR_INVALID_ARG
    assert call(n=0) == cp.ERR_INVALID_ARG
    assert call(n=128) == cp.ERR_UNSUPPORTED
    assert call(order=9) == cp.ERR_INVALID_ARG
    assert call(causal=-1) == cp.ERR_INVALID_ARG
    assert call(ws=None) == cp.ERR_WORKSPACE
    assert call(nbytes=need - 1) == cp.ERR_WORKSPACE and "needed" in err()
    assert call(ws=FAKE + 4) == cp.ERR_WORKSPACE
    assert call(k_=bshd(1, 256, 1, 64)) == cp.ERR_INVALID_ARG and "at least as long" in err()
    assert call(k_=bshd(1, 514, 1, 64)) == cp.ERR_INVALID_ARG and "divisible" in err()
    assert call(out_=bshd(1, 512, 4, 64, dt=7)) == cp.ERR_INVALID_ARG
    assert call(order=3) == cp.ERR_INVALID_ARG

    def merge(n=4, order=0, causal=1, kv_len=512, nbytes=None, out_=out):
        return lib.cpattn_ring_merge(n, order, causal, kv_len, FAKE, need if nbytes is None else nbytes, r(out_),
                                     r(lse), None)

    assert merge(order=cp.ORDER_AUTO) == cp.ERR_INVALID_ARG  # the merge needs the order the steps ran in
    assert merge(kv_len=256) == cp.ERR_INVALID_ARG
    assert merge(kv_len=514) == cp.ERR_INVALID_ARG
    assert merge(nbytes=need - 1) == cp.ERR_WORKSPACE
    assert merge(kv_len=1024) == cp.ERR_WORKSPACE  # a longer K/V has more visible pairs than `need` holds


@no_gpu
def test_ring_online_merge_validation():
    """The accumulating ring step and the fused prefill check their arguments before any launch."""
    r = ctypes.byref
    q, k, v = bshd(1, 512, 4, 64), bshd(1, 512, 1, 64), bshd(1, 512, 1, 64)
    out, lse = bshd(1, 512, 4, 64, cp.DT_F32), lse_of(1, 512, 4)

    def acc(n=4, step=1, order=0, causal=1, lse_=lse, out_=out):
        return lib.cpattn_ring_step_accumulate(r(q), r(k), r(v), n, order, causal, step, r(out_),
                                               r(lse_) if lse_ else None, None)

    assert acc(lse_=None) == cp.ERR_INVALID_ARG and "lse" in err()  # the running LSE is required
    assert acc(step=4) == cp.ERR_INVALID_ARG and "step" in err()
    assert acc(step=-1) == cp.ERR_INVALID_ARG
    assert acc(n=3) == cp.ERR_INVALID_ARG
    assert acc(n=128) == cp.ERR_UNSUPPORTED
    assert acc(order=5) == cp.ERR_INVALID_ARG
    assert acc(out_=bshd(1, 512, 4, 64)) == cp.ERR_INVALID_ARG  # a bf16 running output is refused
    assert acc(out_=bshd(1, 256, 4, 64, cp.DT_F32)) == cp.ERR_INVALID_ARG

    def fused(n=4, causal=1, lse_=lse, out_=out):
        return lib.cpattn_ring_prefill_fused(r(q), r(k), r(v), n, causal, r(out_), r(lse_) if lse_ else None, None)

    assert fused(n=3) == cp.ERR_INVALID_ARG
    assert fused(n=0) == cp.ERR_INVALID_ARG
    assert fused(causal=2) == cp.ERR_INVALID_ARG
    assert fused(out_=bshd(1, 512, 4, 64)) == cp.ERR_INVALID_ARG
    assert fused(lse_=lse_of(1, 512, 3)) == cp.ERR_INVALID_ARG


@no_gpu
def test_decode_validation():
    r = ctypes.byref
    q, k, v = bshd(4, 1, 16, 128), bshd(4, 4096, 1, 128), bshd(4, 4096, 1, 128)
    out = bshd(4, 1, 16, 128, cp.DT_F32)
    need = lib.cpattn_splitkv_decode_workspace_size(r(q), r(k), 8)
    assert need > 0

    def call(q_=q, k_=k, v_=v, n=8, nbytes=need, ws=FAKE):
        return lib.cpattn_splitkv_decode(r(q_), r(k_), r(v_), n, r(out), None, ws, nbytes, None)

    assert call(q_=bshd(4, 2, 16, 128)) == cp.ERR_INVALID_ARG
    f32 = lambda t: T(t.data, cp.DT_F32, 0, t.B, t.S, t.H, t.D, t.stride_b, t.stride_s, t.stride_h)
    assert call(q_=f32(q), k_=f32(k), v_=f32(v)) == cp.ERR_UNSUPPORTED
    assert call(n=3) == cp.ERR_INVALID_ARG
    assert call(nbytes=need - 16) == cp.ERR_WORKSPACE
    assert call(q_=bshd(4, 1, 128, 128)) in (cp.ERR_INVALID_ARG, cp.ERR_UNSUPPORTED)
    assert lib.cpattn_splitkv_decode_workspace_size(r(q), r(k), 3) == 0


def shards(n, B, cap, H, D, dt=cp.DT_BF16, step=1 << 20):
    return (T * n)(*[bshd(B, cap, H, D, dt, ptr=FAKE + r * step) for r in range(n)])


@no_gpu
def test_kv_cache_validation():
    r = ctypes.byref
    k, v = bshd(2, 1024, 1, 128), bshd(2, 1024, 1, 128)
    ks, vs = shards(4, 2, 300, 1, 128), shards(4, 2, 300, 1, 128)
    w = lambda k_=k, v_=v, n=4, ks_=ks, vs_=vs: lib.cpattn_kv_cache_write(r(k_), r(v_), n, ks_, vs_, None)
    assert w(n=3) == cp.ERR_INVALID_ARG and "divisible" in err()
    assert w(n=0) == cp.ERR_INVALID_ARG
    assert w(n=65) == cp.ERR_UNSUPPORTED
    assert w(ks_=shards(4, 2, 200, 1, 128), vs_=shards(4, 2, 200, 1, 128)) == cp.ERR_INVALID_ARG and "chunk" in err()
    assert w(ks_=shards(4, 2, 300, 2, 128), vs_=shards(4, 2, 300, 2, 128)) == cp.ERR_INVALID_ARG
    assert w(ks_=shards(4, 2, 300, 1, 128, cp.DT_F32), vs_=shards(4, 2, 300, 1, 128, cp.DT_F32)) == cp.ERR_INVALID_ARG
    mixed = shards(4, 2, 300, 1, 128)
    mixed[2].S = 301
    assert w(ks_=mixed) == cp.ERR_INVALID_ARG and "shard 2" in err()
    assert lib.cpattn_kv_cache_write(r(k), r(v), 4, None, vs, None) == cp.ERR_INVALID_ARG
    kn, vn = bshd(2, 3, 1, 128), bshd(2, 3, 1, 128)
    a = lambda row, kn_=kn: lib.cpattn_kv_cache_append(r(kn_), r(vn), r(ks[0]), r(vs[0]), row, None)
    assert a(298) == cp.ERR_INVALID_ARG and "fit" in err()
    assert a(-1) == cp.ERR_INVALID_ARG
    assert a(0, kn_=bshd(2, 3, 2, 128)) == cp.ERR_INVALID_ARG


@no_gpu
def test_cp_decode_validation():
    r = ctypes.byref
    q = bshd(3, 1, 16, 128)
    ks, vs = shards(4, 3, 2048, 1, 128), shards(4, 3, 2048, 1, 128)
    need = lib.cpattn_cp_decode_workspace_size(r(q), ks, 4)
    assert need > 0
    out = bshd(3, 1, 16, 128, cp.DT_F32)

    def call(lens=(2048, 10, 0, 7), q_=q, n=4, nbytes=need, ks_=ks, vs_=vs):
        arr = (ctypes.c_int64 * len(lens))(*lens)
        return lib.cpattn_cp_decode(r(q_), ks_, vs_, arr, n, r(out), None, FAKE, nbytes, None)

    assert call(lens=(2049, 10, 0, 7)) == cp.ERR_INVALID_ARG and "shard 0" in err()
    assert call(lens=(5, -1, 0, 7)) == cp.ERR_INVALID_ARG
    assert call(nbytes=need - 16) == cp.ERR_WORKSPACE
    assert call(q_=bshd(3, 2, 16, 128)) == cp.ERR_INVALID_ARG
    assert call(n=0) == cp.ERR_INVALID_ARG
    assert call(ks_=shards(4, 3, 2048, 1, 64), vs_=shards(4, 3, 2048, 1, 64)) == cp.ERR_INVALID_ARG
    assert lib.cpattn_cp_decode(r(q), ks, vs, None, 4, r(out), None, FAKE, need, None) == cp.ERR_INVALID_ARG
    # the workspace is sized by capacity, so filling the shards never changes it
    assert lib.cpattn_cp_decode_workspace_size(r(q), shards(4, 3, 4096, 1, 128), 4) >= need


def test_last_error_cleared_by_success():
    q = bshd(1, 512, 4, 64)
    assert ring_ws(q, 3) == 0 and err() != ""
    assert ring_ws(q, 4) > 0 and err() == ""
