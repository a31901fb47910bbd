"""Seeded input generator: determinism, stream definition and workload table."""
import numpy as np
import torch

import seeded_inputs as si


def test_stream_definition_and_prefix():
    # the first chunk of a tensor is the head of its own PCG64 stream
    t = si.draw_tensor(7, si.TENSOR_K, (1, 100, 1, 4), torch.float32)
    gen = np.random.Generator(np.random.PCG64(np.random.SeedSequence(entropy=7, spawn_key=(1, 0))))
    ref = gen.standard_normal(400, dtype=np.float32)
    assert np.array_equal(t.flatten().numpy(), ref)
    # shorter draws are prefixes of longer ones
    t2 = si.draw_tensor(7, si.TENSOR_K, (1, 10, 1, 4), torch.float32)
    assert torch.equal(t2.flatten(), t.flatten()[:40])


def test_chunks_are_independent_streams(monkeypatch):
    monkeypatch.setattr(si, "CHUNK_ELEMS", 64)
    t = si.draw_tensor(3, si.TENSOR_Q, (1, 50, 1, 4), torch.float32).flatten()  # 200 elems, 4 chunks
    for c in range(4):
        gen = np.random.Generator(np.random.PCG64(np.random.SeedSequence(entropy=3, spawn_key=(0, c))))
        n = min(64, 200 - 64 * c)
        assert np.array_equal(t[64 * c:64 * c + n].numpy(), gen.standard_normal(n, dtype=np.float32))
    assert not torch.equal(t[:64], t[64:128])


def test_bf16_is_round_to_nearest_of_f32():
    f = si.draw_tensor(11, si.TENSOR_V, (2, 64, 2, 8), torch.float32)
    b = si.draw_tensor(11, si.TENSOR_V, (2, 64, 2, 8), torch.bfloat16)
    assert torch.equal(f.to(torch.bfloat16), b)


def test_distribution_is_standard_normal():
    x = si.draw_tensor(1, si.TENSOR_Q, (1, 1 << 14, 1, 64), torch.float32).double()
    assert abs(x.mean().item()) < 5e-3 and abs(x.std().item() - 1.0) < 5e-3


def test_q_k_v_differ_and_seeds_differ():
    w = si.WORKLOADS["tiny_f32_s512_p4"]
    q, k, v = si.make_qkv(w)
    assert q.shape == (1, 512, 1, 64) and q.dtype == torch.float32
    assert not torch.equal(q, k) and not torch.equal(k, v)
    q0 = si.draw_tensor(0, si.TENSOR_Q, (1, 512, 1, 64), torch.float32)
    q1 = si.draw_tensor(1, si.TENSOR_Q, (1, 512, 1, 64), torch.float32)
    assert torch.equal(q, q0) and not torch.equal(q0, q1)


def test_workload_table():
    w = si.WORKLOADS
    assert [x.seed for x in w.values()] == [0, 1, 2, 3, 4]
    c4 = w["prefill_bf16_s128k_p16"]
    assert c4.chunk == 8192 and c4.orders == ("pass_kv", "pass_q")
    assert abs(c4.flops() - 4 * 128 * 16 * 131072 * 131073 / 2) < 1
    c3 = w["decode_b128_kv32k_p8"]
    assert c3.chunk == 4096 and c3.q_shape() == (128, 1, 16, 128) and c3.kv_shape() == (128, 32768, 1, 128)
    assert w["tiny_f32_s512_p4"].dtype == "f32" and w["gqa16_bf16_s8k_p8"].Hq == 16


def test_sampled_rows():
    w = si.WORKLOADS["prefill_bf16_s1m_p8"]
    rows = si.sampled_rows(w, 64)
    assert len(rows) == 64 and len(set(rows.tolist())) == 64
    assert rows[0] == 0 and rows[-1] == w.Sq - 1
    for c in range(1, 8):
        assert c * w.chunk - 1 in rows and c * w.chunk in rows
    assert np.array_equal(rows, si.sampled_rows(w, 64))
