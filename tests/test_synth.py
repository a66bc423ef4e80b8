"""Seeded generators: determinism, the varlen length draw, the bf16 encoding."""
import numpy as np
import torch

from gated_delta_rule_09_amd import synth


def test_bf16_bits_matches_torch_cast():
    x = np.random.default_rng(0).standard_normal(50000).astype(np.float32) * 100
    ties = (np.arange(1, 5000, dtype=np.uint32) << 16 | 0x8000).view(np.float32)
    x = np.concatenate([x, ties])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(synth.bf16_bits(x), ref)
    back = synth.bf16_value(ref)
    np.testing.assert_array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_generators_are_deterministic():
    a = synth.chunk_inputs(1000, 130, Hk=2, Hv=6, d=16, h0_std=0.02)
    b = synth.chunk_inputs(1000, 130, Hk=2, Hv=6, d=16, h0_std=0.02)
    for name in ("q", "k", "v", "g", "beta", "h0"):
        assert synth.sha256(getattr(a, name)) == synth.sha256(getattr(b, name))
    c = synth.chunk_inputs(1001, 130, Hk=2, Hv=6, d=16, h0_std=0.02)
    assert synth.sha256(a.q) != synth.sha256(c.q)


def test_distributions():
    a = synth.chunk_inputs(7, 256, Hk=4, Hv=12, d=128)
    qn = np.linalg.norm(synth.bf16_value(a.q).astype(np.float64), axis=-1)
    assert np.all(np.abs(qn - 1) < 1e-2)
    assert a.g.min() >= -0.1 and a.g.max() < 0.0
    assert 0 < a.beta.min() and a.beta.max() < 1
    v = synth.bf16_value(a.v)
    assert abs(v.std() - 1) < 0.05


def test_varlen_lengths():
    lens = synth.varlen_lengths(1004)
    assert len(lens) == 24
    assert int(lens.sum()) == 262144
    assert lens.min() >= 256 and lens.max() <= 65536
    np.testing.assert_array_equal(lens, synth.varlen_lengths(1004))
    cu = synth.cu_from_lengths(lens)
    assert cu[0] == 0 and cu[-1] == 262144 and np.all(np.diff(cu) >= 0)
