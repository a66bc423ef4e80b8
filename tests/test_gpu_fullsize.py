"""Parity at the full workload sizes.

The GPU runs each workload whole, in the launch configuration the benchmark
times (one call over every head and token, preallocated workspace); the fp64
oracle then recomputes outputs it can finish in seconds:
  core recurrence  B=1, T=512, 16/48 heads, S0 = 0          every head
  full mixer       B=1, T=8192 (conv -> rule -> gated norm)  all conv channels,
                                                             sampled value heads
  long prefill     B=1, T=65536, S0 ~ N(0, 0.02)             sampled value heads
  long prefill,    bf16 o (= fp32 o rounded) and gates from  bit-exact /
  other forms      projections (oracle)                       sampled heads
  decode step      256 sequences x 1 token, state in place   every head
  multi-token      256 sequences x 4 tokens, one pass        every head
  fused decode     the same batch through the whole mixer    every head
                   step in one launch (conv window, state)
  fused mixer      T=8192 in one gdn_mixer_fwd call          bit-identical to
                                                             the four launches
  varlen prefill   262,144 tokens in 24 sequences            sampled (sequence,
                                                             value head) pairs
A sampled value head h is recomputed on its own, with its key/query head
h // (Hv / Hk), so the check covers the head mapping too.
"""
import numpy as np
import pytest
import torch

import oracle
from gated_delta_rule_09_amd import ops, synth
from tests.gpu_util import assert_bf16_within_1ulp, assert_close, dev_bf16, dev_f32, host, log

pytestmark = pytest.mark.gpu

HK, HV, D = 16, 48, 128
GROUP = HV // HK


def bits(t: torch.Tensor) -> np.ndarray:
    """bf16 device tensor -> uint16 host array of its bits."""
    torch.cuda.synchronize()
    return t.contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def f32(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    return t.contiguous().cpu().numpy()


def key_heads(heads):
    """Key/query head of each value head."""
    return [h // GROUP for h in heads]


def test_full_core_T512_every_head():
    T = 512
    log(f"full core recurrence T={T} Hk={HK} Hv={HV}, S0 = 0")
    ci = synth.chunk_inputs(1000, T)
    o, hT = ops.gdn_chunk_fwd(dev_bf16(ci.q), dev_bf16(ci.k), dev_bf16(ci.v), dev_f32(ci.g),
                              dev_f32(ci.beta))
    ro, rT = oracle.recurrence(ci.q, ci.k, ci.v, ci.g, ci.beta)
    assert_close(host(o), ro, "o")
    assert_close(host(hT), rT, "final_state")


def test_full_mixer_T8192_sampled_heads():
    T = 8192
    heads = [0, 19, 38, 47]
    log(f"full mixer T={T}: conv all channels, rule + norm on value heads {heads}")
    mi = synth.mixer_inputs(1001, T)
    y = ops.gdn_conv1d_fwd(dev_bf16(mi.x), dev_bf16(mi.conv_w), n_l2_heads=2 * HK)
    yv = y.view(T, 2 * HK + HV, D)
    o, hT = ops.gdn_chunk_fwd(yv[:, :HK], yv[:, HK:2 * HK], yv[:, 2 * HK:], dev_f32(mi.g),
                              dev_f32(mi.beta))
    out = ops.gdn_gated_rmsnorm(o, dev_bf16(mi.z), dev_f32(mi.norm_w))
    log("  oracle conv")
    ry, _ = oracle.conv1d(mi.x, mi.conv_w, n_l2_heads=2 * HK, head_dim=D, stage_bf16=True)
    assert_bf16_within_1ulp(host(y), ry, "conv y")
    # the rule and the norm take the GPU's conv output, so they are checked on
    # their own inputs (the conv output was just checked against the oracle)
    ybits = bits(y).reshape(T, 2 * HK + HV, D)
    log("  oracle rule")
    kh = key_heads(heads)
    # one key head per value head: the oracle runs the chosen heads only
    ro, rT = oracle.recurrence(ybits[:, kh], ybits[:, HK + np.array(kh)],
                               ybits[:, 2 * HK + np.array(heads)], mi.g[:, heads],
                               mi.beta[:, heads])
    rout = oracle.gated_rmsnorm(ro, mi.z[:, heads], mi.norm_w)
    assert_close(host(o)[:, heads], ro, "o")
    assert_close(host(hT)[:, heads], rT, "final_state")
    assert_close(host(out)[:, heads], rout, "norm out")


def test_full_prefill_T65536_sampled_heads():
    T = 65536
    heads = [2, 24, 46]
    log(f"full prefill T={T} (benchmark inputs, seed 1002), oracle on value heads {heads}")
    ci = synth.chunk_inputs_torch(1002, T, h0_std=0.02)
    o = torch.empty((T, HV, D), dtype=torch.float32, device="cuda")
    fs = torch.empty((1, HV, D, D), dtype=torch.float32, device="cuda")
    ws = torch.empty(ops.gdn_chunk_fwd_workspace_bytes(1, T, HK, HV), dtype=torch.uint8,
                     device="cuda")
    ops.gdn_chunk_fwd(ci["q"], ci["k"], ci["v"], ci["g"], ci["beta"], initial_state=ci["h0"],
                      final_state=fs, o=o, n_seqs=1, workspace=ws)
    kh = key_heads(heads)
    log("  oracle")
    ro, rT = oracle.recurrence(bits(ci["q"][:, kh]), bits(ci["k"][:, kh]),
                               bits(ci["v"][:, heads]), f32(ci["g"][:, heads]),
                               f32(ci["beta"][:, heads]), f32(ci["h0"][:, heads]))
    assert_close(host(o[:, heads]), ro, "o")
    assert_close(host(fs[:, heads]), rT, "final_state")


def test_full_prefill_T65536_bf16_o_and_gated():
    """The two other prefill launch forms the benchmark times, at T=65536: o in
    bf16 is the fp32 o rounded (nearest even) bit for bit with identical final
    states; the gates formed from projections against the oracle's gate
    preparation and recurrence on sampled value heads."""
    T = 65536
    heads = [5, 29]
    log(f"full prefill T={T}: bf16 o, and gates from projections (oracle on heads {heads})")
    ci = synth.chunk_inputs_torch(1002, T, h0_std=0.02)
    args = (ci["q"], ci["k"], ci["v"], ci["g"], ci["beta"])
    o32, s32 = ops.gdn_chunk_fwd(*args, initial_state=ci["h0"], n_seqs=1)
    o16, s16 = ops.gdn_chunk_fwd(*args, initial_state=ci["h0"], n_seqs=1, o_bf16=True)
    torch.cuda.synchronize()
    assert torch.equal(s16, s32), "final states differ"
    assert torch.equal(o16, o32.to(torch.bfloat16)), "bf16 o is not the fp32 o rounded"
    del o16, s16
    gi = synth.gate_inputs(1007, T)
    og, sg = ops.gdn_chunk_fwd_gated(ci["q"], ci["k"], ci["v"], dev_bf16(gi.a), dev_bf16(gi.b),
                                     dev_f32(gi.A_log), dev_f32(gi.dt_bias),
                                     initial_state=ci["h0"], n_seqs=1)
    g, beta = oracle.gate_prep(gi.a[:, heads], gi.b[:, heads], gi.A_log[heads], gi.dt_bias[heads])
    kh = key_heads(heads)
    log("  oracle")
    ro, rT = oracle.recurrence(bits(ci["q"][:, kh]), bits(ci["k"][:, kh]), bits(ci["v"][:, heads]),
                               g, beta, f32(ci["h0"][:, heads]))
    assert_close(host(og[:, heads]), ro, "o (gated)")
    assert_close(host(sg[:, heads]), rT, "final_state (gated)")


def test_full_decode_N256_every_head():
    N = 256
    log(f"full decode step N={N}, state in place")
    di = synth.decode_inputs(1003, N, with_conv=False)
    state = dev_f32(di.state)
    o = ops.gdn_decode_step(dev_bf16(di.q), dev_bf16(di.k), dev_bf16(di.v), dev_f32(di.g),
                            dev_f32(di.beta), state)
    ro, rS = oracle.decode(di.q, di.k, di.v, di.g, di.beta, di.state)
    assert_close(host(o), ro, "o")
    assert_close(host(state), rS, "state")


def test_full_decode_tokens4_N256_every_head():
    """256 sequences x 4 tokens in one pass over the states (the multi-token
    decode the benchmark times): o of every token and the states, every head."""
    N, nt = 256, 4
    log(f"full multi-token decode N={N} x {nt} tokens, every head")
    ci = synth.chunk_inputs(1008, N * nt, lengths=[nt] * N, h0_std=0.02)
    state = dev_f32(ci.h0)
    o = ops.gdn_decode_tokens(dev_bf16(ci.q), dev_bf16(ci.k), dev_bf16(ci.v), dev_f32(ci.g),
                              dev_f32(ci.beta), state, nt)
    ro, rT = oracle.recurrence(ci.q, ci.k, ci.v, ci.g, ci.beta, ci.h0, cu_seqlens=ci.cu_seqlens,
                               n_seqs=N)
    assert_close(host(o), ro, "o")
    assert_close(host(state), rT, "state")


def test_full_decode_mixer_step_N256_every_head():
    N = 256
    log(f"full fused decode step N={N}: conv window and state in place, every head")
    mi = synth.mixer_inputs(1005, N, conv_state_seqs=N)
    state0 = synth.decode_inputs(1006, N, with_conv=False).state
    cs, state = dev_bf16(mi.conv_state), dev_f32(state0)
    out = ops.gdn_decode_mixer_step(dev_bf16(mi.x), dev_bf16(mi.conv_w), cs, dev_f32(mi.g),
                                    dev_f32(mi.beta), dev_bf16(mi.z), dev_f32(mi.norm_w), state,
                                    Hk=HK)
    log("  oracle conv -> decode -> norm")
    ry, rcs = oracle.conv1d(mi.x, mi.conv_w, conv_state=mi.conv_state, n_seqs=N,
                            n_l2_heads=2 * HK, head_dim=D, stage_bf16=True)
    ry = ry.reshape(N, 2 * HK + HV, D)
    ro, rS = oracle.decode(ry[:, :HK], ry[:, HK:2 * HK], ry[:, 2 * HK:], mi.g, mi.beta, state0)
    rout = oracle.gated_rmsnorm(ro, mi.z, mi.norm_w)
    assert_close(host(out), rout, "out")
    assert_close(host(state), rS, "state")
    np.testing.assert_array_equal(host(cs), rcs)


def test_full_mixer_fwd_T8192_equals_four_launches():
    T = 8192
    log(f"full fused mixer T={T}: one gdn_mixer_fwd call against conv, prefill and norm")
    mi = synth.mixer_inputs(1001, T)
    x, w, z, nw = dev_bf16(mi.x), dev_bf16(mi.conv_w), dev_bf16(mi.z), dev_f32(mi.norm_w)
    g, b = dev_f32(mi.g), dev_f32(mi.beta)
    out1, h1 = ops.gdn_mixer_fwd(x, w, g, b, z, nw, Hk=HK, n_seqs=1)
    y = ops.gdn_conv1d_fwd(x, w, n_l2_heads=2 * HK).view(T, 2 * HK + HV, D)
    o, h2 = ops.gdn_chunk_fwd(y[:, :HK], y[:, HK:2 * HK], y[:, 2 * HK:], g, b)
    out2 = ops.gdn_gated_rmsnorm(o, z, nw)
    torch.cuda.synchronize()
    assert torch.equal(out1, out2), "out"
    assert torch.equal(h1, h2), "final_state"


def test_full_varlen_262144_sampled_pairs():
    lens = synth.varlen_lengths(1004)
    T = int(lens.sum())
    log(f"full varlen prefill T={T} N={len(lens)} (benchmark inputs, seed 1004)")
    ci = synth.chunk_inputs_torch(1004, T, lengths=lens, h0_std=0.02)
    o = torch.empty((T, HV, D), dtype=torch.float32, device="cuda")
    fs = torch.empty((len(lens), HV, D, D), dtype=torch.float32, device="cuda")
    ws = torch.empty(ops.gdn_chunk_fwd_workspace_bytes(len(lens), T, HK, HV), dtype=torch.uint8,
                     device="cuda")
    ops.gdn_chunk_fwd(ci["q"], ci["k"], ci["v"], ci["g"], ci["beta"], initial_state=ci["h0"],
                      final_state=fs, o=o, cu_seqlens=ci["cu_seqlens"], workspace=ws)
    cu = synth.cu_from_lengths(lens)
    order = np.argsort(lens)
    picks = [(int(order[0]), 5), (int(order[len(lens) // 2]), 30), (int(order[-1]), 47)]
    g_all, beta_all = f32(ci["g"]), f32(ci["beta"])
    h0_all = f32(ci["h0"])
    for n, h in picks:
        a, b = int(cu[n]), int(cu[n + 1])
        kh = h // GROUP
        log(f"  sequence {n} (length {b - a}), value head {h}")
        q = bits(ci["q"][a:b, kh:kh + 1])
        k = bits(ci["k"][a:b, kh:kh + 1])
        v = bits(ci["v"][a:b, h:h + 1])
        ro, rT = oracle.recurrence(q, k, v, g_all[a:b, h:h + 1], beta_all[a:b, h:h + 1],
                                   h0_all[n:n + 1, h:h + 1])
        assert_close(host(o[a:b, h:h + 1]), ro, "o")
        assert_close(host(fs[n:n + 1, h:h + 1]), rT, "final_state")


def test_full_backward_8x1024_sampled_groups():
    """gdn_backward on the benchmark's backward batch (8 sequences x 1024
    tokens, all 48 value heads, h0 and dS_T given): for sampled (sequence, key
    head) pairs, dq, dk of the key head and dv, dg, dbeta, dh0 of its three
    value heads against the oracle run on that slice alone."""
    N, L = 8, 1024
    T = N * L
    log(f"full backward {N} x {L} tokens (benchmark inputs, seeds 1008/1009)")
    ci = synth.chunk_inputs_torch(1008, T, lengths=[L] * N, h0_std=0.02)
    bs = synth.backward_seeds_torch(1009, T, N)
    got = ops.gdn_backward(ci["q"], ci["k"], ci["v"], ci["g"], ci["beta"], bs["d_o"],
                           initial_state=ci["h0"], grad_final_state=bs["dhT"],
                           cu_seqlens=ci["cu_seqlens"])
    torch.cuda.synchronize()
    for n, kh in ((0, 3), (5, 14)):
        t0, t1 = n * L, (n + 1) * L
        hs = slice(kh * GROUP, (kh + 1) * GROUP)
        log(f"  oracle: sequence {n}, key head {kh}")
        ref = oracle.backward(bits(ci["q"][t0:t1, kh:kh + 1]), bits(ci["k"][t0:t1, kh:kh + 1]),
                              bits(ci["v"][t0:t1, hs]), f32(ci["g"][t0:t1, hs]),
                              f32(ci["beta"][t0:t1, hs]), f32(bs["d_o"][t0:t1, hs]),
                              h0=f32(ci["h0"][n:n + 1, hs]), dhT=f32(bs["dhT"][n:n + 1, hs]))
        tag = f"seq {n} kh {kh}"
        assert_close(host(got["dq"][t0:t1, kh:kh + 1]), ref["dq"], f"{tag} dq")
        assert_close(host(got["dk"][t0:t1, kh:kh + 1]), ref["dk"], f"{tag} dk")
        assert_close(host(got["dv"][t0:t1, hs]), ref["dv"], f"{tag} dv")
        assert_close(host(got["dg"][t0:t1, hs]), ref["dg"], f"{tag} dg")
        assert_close(host(got["dbeta"][t0:t1, hs]), ref["dbeta"], f"{tag} dbeta")
        assert_close(host(got["dh0"][n:n + 1, hs]), ref["dh0"], f"{tag} dh0")
