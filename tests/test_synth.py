"""The seeded input generator (CPU only): determinism, independence of
tensors, shapes and element types, and the distributions each named workload
asks for."""
import numpy as np
import pytest
import torch

import synth


def test_deterministic_and_tag_independent():
    a = synth.normal(0, "x", (64, 64))
    b = synth.normal(0, "x", (64, 64))
    c = synth.normal(0, "r", (64, 64))
    d = synth.normal(1, "x", (64, 64))
    assert np.array_equal(a, b)
    assert not np.array_equal(a, c) and not np.array_equal(a, d)
    assert abs(np.corrcoef(a.ravel(), c.ravel())[0, 1]) < 0.05


def test_moments_of_named_workload():
    inp = synth.workload_inputs("add_rmsnorm_fwd_bf16_16384x7168", M=512)
    x, r, w = inp["x"].float(), inp["r"].float(), inp["w"].float()
    assert inp["x"].dtype == torch.bfloat16 and inp["x"].shape == (512, 7168)
    assert abs(x.mean().item()) < 0.01 and abs(x.std().item() - 1.0) < 0.01
    assert abs(r.std().item() - 0.5) < 0.005
    assert abs(w.mean().item() - 1.0) < 0.01 and abs(w.std().item() - 0.1) < 0.01


def test_decode_outlier_columns():
    cols = synth.outlier_columns(0, 8192)
    assert cols.size == 82 and np.unique(cols).size == 82
    inp = synth.workload_inputs("add_rmsnorm_fwd_bf16_decode_n8192", M=32)
    x = inp["x"].float()
    assert inp["w"].dtype == torch.float32
    big = x[:, cols].abs().mean().item()
    rest = np.delete(x.numpy(), cols, axis=1)
    assert 200 < big < 300 and np.abs(rest).mean() < 1.0


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16, torch.float64])
def test_store_types(dtype):
    t = synth.store(synth.normal(0, "x", (3, 5)), dtype)
    assert t.dtype == dtype and t.is_contiguous()


def test_rope_inputs():
    inp = synth.workload_inputs("rmsnorm_rope_bf16_t16384_q32_k8_d128", M=8192)
    assert inp["qkv"].shape == (8192, 48 * 128) and inp["qkv"].dtype == torch.bfloat16
    assert inp["cos"].shape == (32768, 64) and inp["cos"].dtype == torch.float32
    # a prefill batch of sequences of 4096 tokens
    assert torch.equal(inp["pos"][:4096], torch.arange(4096))
    assert torch.equal(inp["pos"][4096:8192], torch.arange(4096))
    assert not torch.equal(inp["wq"], inp["wk"])
    # the table holds cos and sin of p * 10000^(-2i/D), rounded once to float32
    p, i = 1234, 5
    ang = p * 10000.0 ** (-2.0 * i / 128)
    assert inp["cos"][p, i].item() == np.float32(np.cos(ang))
    assert inp["sin"][p, i].item() == np.float32(np.sin(ang))
    u = synth.positions(3, 1000, 77)
    assert u.dtype == torch.int64 and int(u.min()) >= 0 and int(u.max()) < 77
    assert torch.equal(u, synth.positions(3, 1000, 77))
