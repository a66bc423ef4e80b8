"""Seeded synthetic inputs for the gated-delta-rule mixer.

This module only draws random tensors and encodes/decodes the bfloat16 storage
format; it holds none of the mixer's arithmetic.  The same bytes are handed to
the HIP library and to the CPU oracle.

Distributions follow the layer shape on the "Agnes-3.0-Flash" model card
(Architecture table, row "Delta-rule layers": 16 key heads, 48 value heads,
head dim 128, causal conv kernel 4, fp32 recurrent state) and the workload
recipe of the mixer:
  q, k  ~ N(0, 1), L2-normalised per head in fp32, stored bf16
  v     ~ N(0, 1), stored bf16
  g     ~ U(-0.1, 0)  (log-decay, alpha = exp(g)), fp32
  beta  = sigmoid(N(0, 1)), fp32
  S0    ~ N(0, 0.02^2), fp32, layout [N, Hv, dv, dk]
  x     ~ N(0, 1) bf16 (projected q|k|v channels before the conv)
  conv w ~ N(0, 0.5^2) bf16, layout [C, 4]
  z     ~ N(0, 1) bf16;  norm weight = 1 + N(0, 0.02^2) fp32
  gate projections a, b ~ N(0, 1) bf16 [T, Hv]; per head A_log = log U(1, 16),
  dt_bias ~ U(-7, -2.3) fp32 (a step of about 0.001 .. 0.1 at a = 0)
All draws use numpy's PCG64 from one seed, in the order documented per function.
"""
from __future__ import annotations

import hashlib
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

HK, HV, HEAD_DIM, CONV_K = 16, 48, 128, 4
QKV_CHANNELS = (HK + HK + HV) * HEAD_DIM  # 10240: [q h0..15 | k h0..15 | v h0..47]


def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def bf16_bits(x) -> np.ndarray:
    """fp32 -> bfloat16 bit patterns (uint16), round to nearest, ties to even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_value(bits) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> exact fp32 values."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _unit_rows(r: np.random.Generator, shape) -> np.ndarray:
    a = r.standard_normal(shape, dtype=np.float32)
    n = np.sqrt(np.sum(a * a, axis=-1, keepdims=True, dtype=np.float32))
    return a / n


def _sigmoid_f32(a: np.ndarray) -> np.ndarray:
    return (1.0 / (1.0 + np.exp(-a.astype(np.float64)))).astype(np.float32)


def varlen_lengths(seed: int, n_seqs: int = 24, total: int = 262144, lo: int = 256,
                   hi: int = 65536) -> np.ndarray:
    """Sequence lengths log-uniform in [lo, hi], the last one set to fill `total`.

    Drawing n_seqs-1 lengths and giving the remainder to the last can leave a
    remainder outside [lo, hi]; the draw is repeated (same stream) until the
    remainder is a valid length.  Draw order is kept.
    """
    r = rng(seed)
    for _ in range(100000):
        u = r.uniform(np.log(lo), np.log(hi), size=n_seqs - 1)
        lens = np.floor(np.exp(u)).astype(np.int64)
        rem = total - int(lens.sum())
        if lo <= rem <= hi:
            return np.concatenate([lens, [rem]]).astype(np.int32)
    raise RuntimeError("could not draw lengths")


def cu_from_lengths(lengths) -> np.ndarray:
    return np.concatenate([[0], np.cumsum(np.asarray(lengths, dtype=np.int64))]).astype(np.int32)


@dataclass
class ChunkInputs:
    q: np.ndarray            # uint16 [T, Hk, d]
    k: np.ndarray            # uint16 [T, Hk, d]
    v: np.ndarray            # uint16 [T, Hv, d]
    g: np.ndarray            # f32 [T, Hv]
    beta: np.ndarray         # f32 [T, Hv]
    h0: Optional[np.ndarray]  # f32 [N, Hv, d, d] or None
    cu_seqlens: Optional[np.ndarray]  # int32 [N+1] or None
    n_seqs: int
    meta: dict = field(default_factory=dict)


def chunk_inputs(seed: int, T: int, Hk: int = HK, Hv: int = HV, d: int = HEAD_DIM,
                 lengths=None, h0_std: Optional[float] = None) -> ChunkInputs:
    """Inputs of the core recurrence. Draw order: q, k, v, g, beta, S0."""
    r = rng(seed)
    q = bf16_bits(_unit_rows(r, (T, Hk, d)))
    k = bf16_bits(_unit_rows(r, (T, Hk, d)))
    v = bf16_bits(r.standard_normal((T, Hv, d), dtype=np.float32))
    g = r.uniform(-0.1, 0.0, size=(T, Hv)).astype(np.float32)
    beta = _sigmoid_f32(r.standard_normal((T, Hv), dtype=np.float32))
    if lengths is not None:
        cu = cu_from_lengths(lengths)
        assert int(cu[-1]) == T
        n = len(lengths)
    else:
        cu, n = None, 1
    h0 = None
    if h0_std is not None:
        h0 = (r.standard_normal((n, Hv, d, d), dtype=np.float32) * np.float32(h0_std))
    return ChunkInputs(q, k, v, g, beta, h0, cu, n, {"seed": seed, "T": T})


@dataclass
class BackwardSeeds:
    d_o: np.ndarray             # f32 [T, Hv, d]: gradient of the outputs
    dhT: Optional[np.ndarray]   # f32 [N, Hv, d, d]: gradient of the final states, or None


def backward_seeds(seed: int, T: int, n_seqs: int, Hv: int = HV, d: int = HEAD_DIM,
                   dhT_std: Optional[float] = 0.05) -> BackwardSeeds:
    """Upstream gradients for the backward. Draw order: d_o, dhT."""
    r = rng(seed)
    d_o = r.standard_normal((T, Hv, d), dtype=np.float32)
    dhT = None
    if dhT_std is not None:
        dhT = r.standard_normal((n_seqs, Hv, d, d), dtype=np.float32) * np.float32(dhT_std)
    return BackwardSeeds(d_o, dhT)


@dataclass
class GateInputs:
    a: np.ndarray        # uint16 [T, Hv] (bf16 projection of the decay step)
    b: np.ndarray        # uint16 [T, Hv] (bf16 projection of the write strength)
    A_log: np.ndarray    # f32 [Hv]
    dt_bias: np.ndarray  # f32 [Hv]


def gate_inputs(seed: int, T: int, Hv: int = HV) -> GateInputs:
    """Per-head gate projections and parameters. Draw order: a, b, A, dt_bias."""
    r = rng(seed)
    a = bf16_bits(r.standard_normal((T, Hv), dtype=np.float32))
    b = bf16_bits(r.standard_normal((T, Hv), dtype=np.float32))
    A_log = np.log(r.uniform(1.0, 16.0, size=Hv)).astype(np.float32)
    dt_bias = r.uniform(-7.0, -2.3, size=Hv).astype(np.float32)
    return GateInputs(a, b, A_log, dt_bias)


@dataclass
class MixerInputs:
    x: np.ndarray        # uint16 [T, C]
    conv_w: np.ndarray   # uint16 [C, 4]
    g: np.ndarray        # f32 [T, Hv]
    beta: np.ndarray     # f32 [T, Hv]
    z: np.ndarray        # uint16 [T, Hv, d]
    norm_w: np.ndarray   # f32 [d]
    conv_state: Optional[np.ndarray]  # uint16 [N, C, 3] or None


def mixer_inputs(seed: int, T: int, Hk: int = HK, Hv: int = HV, d: int = HEAD_DIM,
                 conv_state_seqs: int = 0) -> MixerInputs:
    """Inputs of the full mixer. Draw order: g, beta, x, conv w, z, norm w, conv state."""
    r = rng(seed)
    C = (2 * Hk + Hv) * d
    g = r.uniform(-0.1, 0.0, size=(T, Hv)).astype(np.float32)
    beta = _sigmoid_f32(r.standard_normal((T, Hv), dtype=np.float32))
    x = bf16_bits(r.standard_normal((T, C), dtype=np.float32))
    w = bf16_bits(r.standard_normal((C, CONV_K), dtype=np.float32) * np.float32(0.5))
    z = bf16_bits(r.standard_normal((T, Hv, d), dtype=np.float32))
    nw = (1.0 + 0.02 * r.standard_normal(d, dtype=np.float32)).astype(np.float32)
    cs = None
    if conv_state_seqs:
        cs = bf16_bits(r.standard_normal((conv_state_seqs, C, CONV_K - 1), dtype=np.float32))
    return MixerInputs(x, w, g, beta, z, nw, cs)


@dataclass
class DecodeInputs:
    q: np.ndarray       # uint16 [N, Hk, d]
    k: np.ndarray       # uint16 [N, Hk, d]
    v: np.ndarray       # uint16 [N, Hv, d]
    g: np.ndarray       # f32 [N, Hv]
    beta: np.ndarray    # f32 [N, Hv]
    state: np.ndarray   # f32 [N, Hv, d, d]
    x: np.ndarray       # uint16 [N, C]  (conv input for the step)
    conv_w: np.ndarray  # uint16 [C, 4]
    conv_state: np.ndarray  # uint16 [N, C, 3]


def decode_inputs(seed: int, N: int, Hk: int = HK, Hv: int = HV, d: int = HEAD_DIM,
                  state_std: float = 0.02, with_conv: bool = True) -> DecodeInputs:
    """Inputs of one decode step. Draw order: q, k, v, g, beta, state, x, conv w, conv state."""
    r = rng(seed)
    q = bf16_bits(_unit_rows(r, (N, Hk, d)))
    k = bf16_bits(_unit_rows(r, (N, Hk, d)))
    v = bf16_bits(r.standard_normal((N, Hv, d), dtype=np.float32))
    g = r.uniform(-0.1, 0.0, size=(N, Hv)).astype(np.float32)
    beta = _sigmoid_f32(r.standard_normal((N, Hv), dtype=np.float32))
    state = r.standard_normal((N, Hv, d, d), dtype=np.float32) * np.float32(state_std)
    C = (2 * Hk + Hv) * d
    if with_conv:
        x = bf16_bits(r.standard_normal((N, C), dtype=np.float32))
        w = bf16_bits(r.standard_normal((C, CONV_K), dtype=np.float32) * np.float32(0.5))
        cs = bf16_bits(r.standard_normal((N, C, CONV_K - 1), dtype=np.float32))
    else:
        x = w = cs = None
    return DecodeInputs(q, k, v, g, beta, state, x, w, cs)


def sha256(a: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


# ---------------------------------------------------------------- on-device draws
#
# Same distributions as above, drawn with torch's seeded generator directly on
# the GPU (a different random stream from numpy's PCG64).  Used for benchmark
# inputs that are too large to draw on the host quickly; parity tests use the
# numpy generators so the oracle sees the identical bytes.

def _tgen(seed: int, device):
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    return gen


def chunk_inputs_torch(seed: int, T: int, Hk: int = HK, Hv: int = HV, d: int = HEAD_DIM,
                       lengths=None, h0_std: Optional[float] = None, device="cuda"):
    """dict of device tensors: q, k, v (bf16), g, beta (fp32), h0, cu_seqlens."""
    import torch
    gen = _tgen(seed, device)

    def unit(shape):
        a = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
        return (a / a.norm(dim=-1, keepdim=True)).to(torch.bfloat16)

    q = unit((T, Hk, d))
    k = unit((T, Hk, d))
    v = torch.randn((T, Hv, d), generator=gen, device=device, dtype=torch.float32).to(torch.bfloat16)
    g = torch.rand((T, Hv), generator=gen, device=device, dtype=torch.float32) * -0.1
    beta = torch.sigmoid(torch.randn((T, Hv), generator=gen, device=device, dtype=torch.float32))
    n = 1 if lengths is None else len(lengths)
    cu = None
    if lengths is not None:
        cu = torch.from_numpy(cu_from_lengths(lengths)).to(device)
    h0 = None
    if h0_std is not None:
        h0 = torch.randn((n, Hv, d, d), generator=gen, device=device, dtype=torch.float32) * h0_std
    return dict(q=q, k=k, v=v, g=g, beta=beta, h0=h0, cu_seqlens=cu, n_seqs=n)


def backward_seeds_torch(seed: int, T: int, n_seqs: int, Hv: int = HV, d: int = HEAD_DIM,
                         dhT_std: float = 0.05, device="cuda"):
    """dict of device tensors d_o [T, Hv, d], dhT [n_seqs, Hv, d, d] (fp32), the
    distributions of backward_seeds."""
    import torch
    gen = _tgen(seed, device)
    d_o = torch.randn((T, Hv, d), generator=gen, device=device, dtype=torch.float32)
    dhT = torch.randn((n_seqs, Hv, d, d), generator=gen, device=device, dtype=torch.float32) * dhT_std
    return dict(d_o=d_o, dhT=dhT)


def mixer_inputs_torch(seed: int, T: int, Hk: int = HK, Hv: int = HV, d: int = HEAD_DIM,
                       device="cuda"):
    import torch
    gen = _tgen(seed, device)
    C = (2 * Hk + Hv) * d
    g = torch.rand((T, Hv), generator=gen, device=device) * -0.1
    beta = torch.sigmoid(torch.randn((T, Hv), generator=gen, device=device))
    x = torch.randn((T, C), generator=gen, device=device).to(torch.bfloat16)
    w = (torch.randn((C, CONV_K), generator=gen, device=device) * 0.5).to(torch.bfloat16)
    z = torch.randn((T, Hv, d), generator=gen, device=device).to(torch.bfloat16)
    nw = 1.0 + 0.02 * torch.randn((d,), generator=gen, device=device)
    return dict(x=x, conv_w=w, g=g, beta=beta, z=z, norm_w=nw)


def decode_inputs_torch(seed: int, N: int, Hk: int = HK, Hv: int = HV, d: int = HEAD_DIM,
                        state_std: float = 0.02, device="cuda"):
    import torch
    gen = _tgen(seed, device)

    def unit(shape):
        a = torch.randn(shape, generator=gen, device=device)
        return (a / a.norm(dim=-1, keepdim=True)).to(torch.bfloat16)

    C = (2 * Hk + Hv) * d
    return dict(
        q=unit((N, Hk, d)), k=unit((N, Hk, d)),
        v=torch.randn((N, Hv, d), generator=gen, device=device).to(torch.bfloat16),
        g=torch.rand((N, Hv), generator=gen, device=device) * -0.1,
        beta=torch.sigmoid(torch.randn((N, Hv), generator=gen, device=device)),
        state=torch.randn((N, Hv, d, d), generator=gen, device=device) * state_std,
        x=torch.randn((N, C), generator=gen, device=device).to(torch.bfloat16),
        conv_w=(torch.randn((C, CONV_K), generator=gen, device=device) * 0.5).to(torch.bfloat16),
        conv_state=torch.randn((N, C, CONV_K - 1), generator=gen, device=device).to(torch.bfloat16),
    )
