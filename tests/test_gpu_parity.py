"""GPU parity of every entry point against the fp64 oracle, at sizes the oracle
finishes in seconds, spanning several chunks and ragged tails, plus edge cases
(empty sequences, T = 1, partial chunks, slot maps)."""
import numpy as np
import pytest
import torch

import oracle
from gated_delta_rule_09_amd import ops, synth
from tests.gpu_util import (assert_bf16_rounded_close, assert_bf16_within_1ulp, assert_close,
                            dev_bf16, dev_f32, dev_i32, host, log)

pytestmark = pytest.mark.gpu


def run_chunk(ci: synth.ChunkInputs, scale=1.0, varlen=True):
    cu = dev_i32(ci.cu_seqlens) if (varlen and ci.cu_seqlens is not None) else None
    h0 = dev_f32(ci.h0) if ci.h0 is not None else None
    o, hT = ops.gdn_chunk_fwd(dev_bf16(ci.q), dev_bf16(ci.k), dev_bf16(ci.v), dev_f32(ci.g),
                              dev_f32(ci.beta), initial_state=h0, cu_seqlens=cu,
                              n_seqs=ci.n_seqs, scale=scale)
    return host(o), host(hT)


def oracle_chunk(ci: synth.ChunkInputs, scale=1.0):
    return oracle.recurrence(ci.q, ci.k, ci.v, ci.g, ci.beta, ci.h0, cu_seqlens=ci.cu_seqlens,
                             n_seqs=ci.n_seqs, scale=scale)


# ----------------------------------------------------------------- prefill

@pytest.mark.parametrize("T", [1, 2, 3, 63, 64, 65, 127, 200])
def test_chunk_single_sequence_lengths(T):
    log(f"chunk_fwd T={T} Hk=16 Hv=48 h0")
    ci = synth.chunk_inputs(2000 + T, T, h0_std=0.02)
    o, hT = run_chunk(ci)
    ro, rT = oracle_chunk(ci)
    assert_close(o, ro, "o")
    assert_close(hT, rT, "final_state")


@pytest.mark.parametrize("Hk,Hv", [(1, 1), (2, 6), (4, 8), (3, 12)])
def test_chunk_head_groupings(Hk, Hv):
    log(f"chunk_fwd T=150 Hk={Hk} Hv={Hv}")
    ci = synth.chunk_inputs(2100 + Hv, 150, Hk=Hk, Hv=Hv, h0_std=0.1)
    o, hT = run_chunk(ci)
    ro, rT = oracle_chunk(ci)
    assert_close(o, ro, "o")
    assert_close(hT, rT, "final_state")


@pytest.mark.parametrize("lens", [[150], [70, 0, 1, 64, 129, 5, 0, 200, 33]])
def test_chunk_bf16_output(lens):
    """gdn_chunk_fwd_bf16o: o is the fp32 result of gdn_chunk_fwd rounded to
    bf16 (nearest, ties to even) bit for bit, and the final states agree
    exactly; both paths against the oracle."""
    log(f"chunk_fwd bf16 o lens={lens}")
    ci = synth.chunk_inputs(2150 + len(lens), int(sum(lens)), Hk=4, Hv=12, lengths=lens, h0_std=0.05)
    args = (dev_bf16(ci.q), dev_bf16(ci.k), dev_bf16(ci.v), dev_f32(ci.g), dev_f32(ci.beta))
    kw = dict(initial_state=dev_f32(ci.h0), cu_seqlens=dev_i32(ci.cu_seqlens))
    o32, hT32 = ops.gdn_chunk_fwd(*args, **kw)
    o16, hT16 = ops.gdn_chunk_fwd(*args, o_bf16=True, **kw)
    assert o16.dtype == torch.bfloat16
    np.testing.assert_array_equal(host(hT16), host(hT32))
    want = oracle.round_bf16(host(o32))                 # fp64 values on the bf16 grid
    got = o16.float().cpu().numpy().astype(np.float64)   # exact widening
    np.testing.assert_array_equal(got, want)
    # against the oracle: the fp32 bar, plus the bf16 rounding itself.  The
    # fp32 o carries the fp16-operand error (rel-L2 a few 1e-4, more than half
    # a bf16 ulp on small elements), so no one-ulp check: by the triangle
    # inequality the rounded o is within 1e-3 + 2^-9 (the rounding's largest
    # relative step) in rel-L2
    ro, _ = oracle_chunk(ci)
    assert_close(host(o32), ro, "o (fp32)")
    assert_bf16_rounded_close(got, ro, "o (bf16)")


@pytest.mark.parametrize("out_bf16", [False, True])
def test_chunk_pooled_mixed_batch(out_bf16):
    """A batch mixing prefills with one- and two-token sequences (and an empty
    one), each continuing from its slot of a state pool and leaving its final
    state there; unnamed slots untouched bit for bit."""
    lens = [1, 300, 0, 1, 2, 65, 1, 129]
    n_slots = 12
    log(f"chunk_fwd_pooled lens={lens} bf16_o={out_bf16}")
    ci = synth.chunk_inputs(3500, sum(lens), Hk=4, Hv=12, lengths=lens)
    pool = np.random.default_rng(35).standard_normal((n_slots, 12, 128, 128)).astype(np.float32) * 0.05
    slots = np.array([9, 2, 11, 0, 5, 7, 3, 10], dtype=np.int32)
    st = dev_f32(pool)
    o = ops.gdn_chunk_fwd_pooled(dev_bf16(ci.q), dev_bf16(ci.k), dev_bf16(ci.v), dev_f32(ci.g),
                                 dev_f32(ci.beta), st, dev_i32(slots),
                                 cu_seqlens=dev_i32(ci.cu_seqlens), scale=0.9, o_bf16=out_bf16)
    ro, rT = oracle.recurrence(ci.q, ci.k, ci.v, ci.g, ci.beta, pool[slots],
                               cu_seqlens=ci.cu_seqlens, n_seqs=len(lens), scale=0.9)
    got = host(o)
    if out_bf16:
        assert_bf16_rounded_close(got, ro, "o (bf16)")
    else:
        assert_close(got, ro, "o")
    got_st = host(st)
    assert_close(got_st[slots], rT, "states (slots used)")
    np.testing.assert_array_equal(got_st[slots[2]], pool[slots[2]])   # the empty sequence
    others = [i for i in range(n_slots) if i not in slots]
    np.testing.assert_array_equal(got_st[others], pool[others])


def test_chunk_pooled_equals_gather_scatter():
    """The pooled call computes exactly what gdn_chunk_fwd computes on the
    gathered states (same kernels, same arithmetic): bit-identical o and
    states."""
    lens = [70, 1, 3, 200]
    log(f"chunk_fwd_pooled vs gathered gdn_chunk_fwd lens={lens}")
    ci = synth.chunk_inputs(3510, sum(lens), Hk=2, Hv=6, lengths=lens)
    pool = np.random.default_rng(36).standard_normal((6, 6, 128, 128)).astype(np.float32) * 0.05
    slots = np.array([4, 1, 5, 0], dtype=np.int32)
    args = (dev_bf16(ci.q), dev_bf16(ci.k), dev_bf16(ci.v), dev_f32(ci.g), dev_f32(ci.beta))
    cu = dev_i32(ci.cu_seqlens)
    st = dev_f32(pool)
    o1 = ops.gdn_chunk_fwd_pooled(*args, st, dev_i32(slots), cu_seqlens=cu)
    o2, hT = ops.gdn_chunk_fwd(*args, initial_state=dev_f32(pool[slots]), cu_seqlens=cu)
    assert torch.equal(o1, o2)
    np.testing.assert_array_equal(host(st)[slots], host(hT))


@pytest.mark.parametrize("strided", [False, True])
def test_chunk_gated_against_oracle(strided):
    """Gates formed in the prep kernel from bf16 projections: against the
    oracle's gate preparation followed by the recurrence.  With `strided`,
    a and b are columns of a wider projection output."""
    lens = [129, 0, 64, 7]
    T, Hv = sum(lens), 12
    log(f"chunk_fwd_gated lens={lens} strided={strided}")
    ci = synth.chunk_inputs(3520, T, Hk=4, Hv=Hv, lengths=lens, h0_std=0.05)
    gi = synth.gate_inputs(3521, T, Hv=Hv)
    if strided:
        wide = torch.zeros((T, 3 * Hv + 8), dtype=torch.bfloat16, device="cuda")
        wide[:, 8:8 + Hv] = dev_bf16(gi.a)
        wide[:, 8 + 2 * Hv:8 + 3 * Hv] = dev_bf16(gi.b)
        a_d, b_d = wide[:, 8:8 + Hv], wide[:, 8 + 2 * Hv:8 + 3 * Hv]
    else:
        a_d, b_d = dev_bf16(gi.a), dev_bf16(gi.b)
    o, hT = ops.gdn_chunk_fwd_gated(dev_bf16(ci.q), dev_bf16(ci.k), dev_bf16(ci.v), a_d, b_d,
                                    dev_f32(gi.A_log), dev_f32(gi.dt_bias),
                                    initial_state=dev_f32(ci.h0), cu_seqlens=dev_i32(ci.cu_seqlens))
    g, beta = oracle.gate_prep(gi.a, gi.b, gi.A_log, gi.dt_bias)
    log(f"  g in [{g.min():.3f}, {g.max():.4f}], beta in [{beta.min():.3f}, {beta.max():.3f}]")
    ro, rT = oracle.recurrence(ci.q, ci.k, ci.v, g, beta, ci.h0, cu_seqlens=ci.cu_seqlens,
                               n_seqs=len(lens))
    assert_close(host(o), ro, "o")
    assert_close(host(hT), rT, "final_state")


def test_chunk_gated_equals_given_gates():
    """The in-kernel gates against torch's fp32 softplus and sigmoid fed to
    gdn_chunk_fwd: the same up to the fp32 rounding of the two gate
    computations."""
    T, Hv = 200, 12
    log("chunk_fwd_gated vs gdn_chunk_fwd with torch-computed gates")
    ci = synth.chunk_inputs(3530, T, Hk=4, Hv=Hv)
    gi = synth.gate_inputs(3531, T, Hv=Hv)
    a, b = dev_bf16(gi.a), dev_bf16(gi.b)
    A_log, dt = dev_f32(gi.A_log), dev_f32(gi.dt_bias)
    q, k, v = dev_bf16(ci.q), dev_bf16(ci.k), dev_bf16(ci.v)
    o1, h1 = ops.gdn_chunk_fwd_gated(q, k, v, a, b, A_log, dt)
    g = (-torch.exp(A_log) * torch.nn.functional.softplus(a.float() + dt)).contiguous()
    beta = torch.sigmoid(b.float()).contiguous()
    o2, h2 = ops.gdn_chunk_fwd(q, k, v, g, beta)
    for name, x1, x2 in (("o", o1, o2), ("state", h1, h2)):
        x1, x2 = x1.double(), x2.double()
        rel = ((x1 - x2).norm() / x2.norm()).item()
        log(f"  {name}: rel_l2 in-kernel vs torch gates = {rel:.3e}")
        assert rel <= 1e-5, name


def test_chunk_zero_initial_state_and_scale():
    log("chunk_fwd T=300 no h0 scale=128^-0.5")
    ci = synth.chunk_inputs(2200, 300)
    s = 128 ** -0.5
    o, hT = run_chunk(ci, scale=s)
    ro, rT = oracle_chunk(ci, scale=s)
    assert_close(o, ro, "o")
    assert_close(hT, rT, "final_state")


def test_chunk_equal_split_without_cu_seqlens():
    log("chunk_fwd 3 equal sequences of 100, no cu_seqlens")
    ci = synth.chunk_inputs(2300, 300, Hk=4, Hv=12, lengths=[100, 100, 100], h0_std=0.05)
    o, hT = run_chunk(ci, varlen=False)
    ro, rT = oracle_chunk(ci)
    assert_close(o, ro, "o")
    assert_close(hT, rT, "final_state")


def test_chunk_varlen_with_empty_sequences():
    lens = [70, 0, 1, 64, 0, 129, 5]
    log(f"chunk_fwd varlen {lens}")
    ci = synth.chunk_inputs(2400, sum(lens), Hk=4, Hv=12, lengths=lens, h0_std=0.05)
    o, hT = run_chunk(ci)
    ro, rT = oracle_chunk(ci)
    assert_close(o, ro, "o")
    for n in range(len(lens)):
        assert_close(hT[n], rT[n], f"final_state[{n}]")
    # empty sequences hand back their initial state exactly
    np.testing.assert_array_equal(hT[1], ci.h0[1])
    np.testing.assert_array_equal(hT[4], ci.h0[4])


def test_chunk_strong_decay_and_beta_extremes():
    log("chunk_fwd strong decay, beta in {0, 1}")
    ci = synth.chunk_inputs(2500, 200, Hk=2, Hv=6, h0_std=0.05)
    ci.g = (ci.g * 30.0).astype(np.float32)           # alpha down to exp(-3)
    ci.beta[::3] = 1.0
    ci.beta[1::3] = 0.0
    o, hT = run_chunk(ci)
    ro, rT = oracle_chunk(ci)
    assert_close(o, ro, "o")
    assert_close(hT, rT, "final_state")


# ----------------------------------------------------------------- chunk map

def scaled(ci: synth.ChunkInputs, e: int) -> synth.ChunkInputs:
    """v and S0 times 2^e (exact: bf16 and fp32 keep every bit under a power
    of two within their exponent range).  The rule is linear in (S0, v), so
    o and the final state scale by 2^e too and the relative bar is the same."""
    v = synth.bf16_bits(synth.bf16_value(ci.v) * np.float32(2.0 ** e))
    assert np.array_equal(synth.bf16_value(v), synth.bf16_value(ci.v) * np.float32(2.0 ** e))
    return synth.ChunkInputs(ci.q, ci.k, v, ci.g, ci.beta,
                             None if ci.h0 is None else (ci.h0 * np.float32(2.0 ** e)),
                             ci.cu_seqlens, ci.n_seqs)


@pytest.mark.parametrize("T", [200, 1024])
@pytest.mark.parametrize("e", [-12, -10, 6, 8])
def test_chunk_value_and_state_scale(T, e):
    """The prefill's matrix-unit operands S0, U (and the V tile) are fp16: the
    relative bar must hold with v and S0 scaled by 2^e, from fp16's subnormal
    end (2^-12: S0 ~ 5e-6) to 2^8 (|v| up to ~1500)."""
    log(f"chunk_fwd T={T}, v and S0 times 2^{e}")
    ci = scaled(synth.chunk_inputs(2300 + T, T, h0_std=0.02), e)
    o, hT = run_chunk(ci)
    ro, rT = oracle_chunk(ci)
    assert_close(o, ro, "o")
    assert_close(hT, rT, "final_state")


@pytest.mark.parametrize("T", [200, 1024])
def test_chunk_value_outliers(T):
    """One value head carries a dozen |v| ~ 200 entries among N(0, 1) values."""
    log(f"chunk_fwd T={T}, |v| ~ 200 outliers on value head 7")
    ci = synth.chunk_inputs(2400 + T, T, h0_std=0.02)
    r = synth.rng(2401)
    v = synth.bf16_value(ci.v).copy()
    t = r.integers(0, T, 12)
    c = r.integers(0, ci.v.shape[2], 12)
    v[t, 7, c] = np.where(r.random(12) < 0.5, -1.0, 1.0) * r.uniform(150.0, 250.0, 12)
    ci = synth.ChunkInputs(ci.q, ci.k, synth.bf16_bits(v), ci.g, ci.beta, ci.h0, ci.cu_seqlens,
                           ci.n_seqs)
    o, hT = run_chunk(ci)
    ro, rT = oracle_chunk(ci)
    assert_close(o, ro, "o")
    assert_close(hT, rT, "final_state")
    assert_close(o[:, 7], ro[:, 7], "o head 7")
    assert_close(hT[:, 7], rT[:, 7], "final_state head 7")


@pytest.mark.parametrize("lens", [[5], [64, 64], [0, 0, 3], [100, 0, 65, 1, 64, 300, 0, 2],
                                  list(np.random.default_rng(3).integers(0, 400, 300))])
def test_chunk_map_bit_exact(lens):
    log(f"chunk_map N={len(lens)}")
    cu = synth.cu_from_lengths(lens)
    T = int(cu[-1])
    order, off, tab = ops.gdn_chunk_map(dev_i32(cu), T)
    r_off, r_tab = oracle.chunk_map(cu)
    torch.cuda.synchronize()
    # the schedule is the kernel's own choice (longest sequences first), not
    # part of the result: check it is a permutation with non-increasing lengths
    got_order = order.cpu().numpy()
    lens_arr = np.diff(np.asarray(cu, dtype=np.int64))
    assert sorted(got_order.tolist()) == list(range(len(lens)))
    assert np.all(np.diff(lens_arr[got_order]) <= 0)
    np.testing.assert_array_equal(off.cpu().numpy(), r_off)
    n = int(r_off[-1])
    np.testing.assert_array_equal(tab[:n].cpu().numpy(), r_tab)


# ----------------------------------------------------------------- decode

@pytest.mark.parametrize("N", [1, 5, 33])
def test_decode_step(N):
    log(f"decode_step N={N}")
    di = synth.decode_inputs(2600 + N, N, with_conv=False)
    st = dev_f32(di.state)
    o = ops.gdn_decode_step(dev_bf16(di.q), dev_bf16(di.k), dev_bf16(di.v), dev_f32(di.g),
                            dev_f32(di.beta), st)
    ro, rst = oracle.decode(di.q, di.k, di.v, di.g, di.beta, di.state)
    assert_close(host(o), ro, "o")
    assert_close(host(st), rst, "state")


def test_decode_step_slot_map_and_scale():
    N, slots_n = 6, 10
    log("decode_step with slot map")
    di = synth.decode_inputs(2700, N, with_conv=False)
    pool = np.random.default_rng(5).standard_normal((slots_n, 48, 128, 128)).astype(np.float32) * 0.02
    slots = np.array([7, 0, 3, 9, 4, 1], dtype=np.int32)
    pool[slots] = di.state
    st = dev_f32(pool)
    o = ops.gdn_decode_step(dev_bf16(di.q), dev_bf16(di.k), dev_bf16(di.v), dev_f32(di.g),
                            dev_f32(di.beta), st, state_slot=dev_i32(slots), scale=0.5)
    ro, rst = oracle.decode(di.q, di.k, di.v, di.g, di.beta, pool, state_slot=slots, scale=0.5)
    got = host(st)
    assert_close(host(o), ro, "o")
    assert_close(got[slots], rst[slots], "state (slots used)")
    others = [i for i in range(slots_n) if i not in slots]
    np.testing.assert_array_equal(got[others], pool[others])


@pytest.mark.parametrize("N,nt", [(1, 1), (3, 2), (6, 3), (4, 4), (5, 5), (4, 6), (2, 7), (17, 8)])
def test_decode_tokens_against_oracle(N, nt):
    """n_tokens tokens per sequence in one pass: the recurrence from each
    sequence's state, o of every token and the final state."""
    log(f"decode_tokens N={N} n_tokens={nt}")
    ci = synth.chunk_inputs(2800 + 10 * N + nt, N * nt, lengths=[nt] * N, h0_std=0.02)
    st = dev_f32(ci.h0)
    o = ops.gdn_decode_tokens(dev_bf16(ci.q), dev_bf16(ci.k), dev_bf16(ci.v), dev_f32(ci.g),
                              dev_f32(ci.beta), st, nt)
    ro, rT = oracle.recurrence(ci.q, ci.k, ci.v, ci.g, ci.beta, ci.h0, cu_seqlens=ci.cu_seqlens,
                               n_seqs=N)
    assert_close(host(o), ro, "o")
    assert_close(host(st), rT, "state")


@pytest.mark.parametrize("nt", [1, 3, 8])
def test_decode_tokens_equals_successive_steps(nt):
    """The same per-token arithmetic as gdn_decode_step: n_tokens tokens in one
    call agree with n_tokens successive one-token calls (slot map and scale
    included)."""
    N, slots_n = 6, 9
    log(f"decode_tokens vs {nt} decode_step calls")
    ci = synth.chunk_inputs(2900 + nt, N * nt, lengths=[nt] * N, h0_std=0.02)
    pool = np.random.default_rng(6).standard_normal((slots_n, 48, 128, 128)).astype(np.float32) * 0.02
    slots = np.array([8, 2, 0, 5, 3, 6], dtype=np.int32)
    pool[slots] = ci.h0
    q, k, v = dev_bf16(ci.q), dev_bf16(ci.k), dev_bf16(ci.v)
    g, b = dev_f32(ci.g), dev_f32(ci.beta)
    st1 = dev_f32(pool)
    o1 = ops.gdn_decode_tokens(q, k, v, g, b, st1, nt, state_slot=dev_i32(slots), scale=0.7)
    st2 = dev_f32(pool)
    o2 = torch.empty_like(o1)
    qv, kv, vv = q.view(N, nt, 16, 128), k.view(N, nt, 16, 128), v.view(N, nt, 48, 128)
    gv, bv, o2v = g.view(N, nt, 48), b.view(N, nt, 48), o2.view(N, nt, 48, 128)
    for t in range(nt):
        o2v[:, t] = ops.gdn_decode_step(qv[:, t], kv[:, t], vv[:, t], gv[:, t].contiguous(),
                                        bv[:, t].contiguous(), st2, state_slot=dev_i32(slots),
                                        scale=0.7)
    for name, a1, a2 in (("o", host(o1), host(o2)), ("state", host(st1), host(st2))):
        err = np.abs(a1.astype(np.float64) - a2).max() / np.abs(a2).max()
        log(f"  {name}: max|one call - successive calls| / max = {err:.3e}")
        assert err <= 1e-6, name
    others = [i for i in range(slots_n) if i not in slots]
    np.testing.assert_array_equal(host(st1)[others], pool[others])


# ----------------------------------------------------------------- conv

@pytest.mark.parametrize("lens", [[37], [1, 1, 1, 1], [10, 0, 2, 25, 1]])
def test_conv1d_varlen_with_state(lens):
    log(f"conv1d lens={lens}")
    mi = synth.mixer_inputs(2800 + len(lens), sum(lens), conv_state_seqs=len(lens))
    cu = synth.cu_from_lengths(lens)
    cs = dev_bf16(mi.conv_state)
    y = ops.gdn_conv1d_fwd(dev_bf16(mi.x), dev_bf16(mi.conv_w), conv_state=cs,
                           cu_seqlens=dev_i32(cu), n_l2_heads=32)
    ry, rcs = oracle.conv1d(mi.x, mi.conv_w, conv_state=mi.conv_state, cu_seqlens=cu,
                            n_l2_heads=32, head_dim=128, l2_eps=1e-6, stage_bf16=True)
    assert_bf16_within_1ulp(host(y), ry, "y")
    np.testing.assert_array_equal(host(cs), rcs)


def test_conv1d_no_state_equal_split_and_bias():
    T, N = 96, 3
    log("conv1d no state, equal split, bias")
    mi = synth.mixer_inputs(2900, T)
    bias = np.random.default_rng(9).standard_normal(mi.x.shape[1]).astype(np.float32) * 0.1
    y = ops.gdn_conv1d_fwd(dev_bf16(mi.x), dev_bf16(mi.conv_w), bias=dev_f32(bias), n_seqs=N,
                           n_l2_heads=32)
    ry, _ = oracle.conv1d(mi.x, mi.conv_w, bias=bias, n_seqs=N, n_l2_heads=32, head_dim=128,
                          l2_eps=1e-6, stage_bf16=True)
    assert_bf16_within_1ulp(host(y), ry, "y")


def test_conv1d_strided_rows():
    T = 20
    log("conv1d strided x and y rows")
    mi = synth.mixer_inputs(3000, T)
    C = mi.x.shape[1]
    xb = torch.zeros((T, C + 64), dtype=torch.bfloat16, device="cuda")
    xb[:, :C] = dev_bf16(mi.x)
    yb = torch.full((T, C + 32), 7.0, dtype=torch.bfloat16, device="cuda")
    ops.gdn_conv1d_fwd(xb[:, :C], dev_bf16(mi.conv_w), y=yb[:, :C], n_l2_heads=32)
    ry, _ = oracle.conv1d(mi.x, mi.conv_w, n_l2_heads=32, head_dim=128, stage_bf16=True)
    got = host(yb)
    assert_bf16_within_1ulp(got[:, :C], ry, "y")
    assert np.all(got[:, C:] == 7.0), "padding columns of y were written"


# ----------------------------------------------------------------- gated norm

@pytest.mark.parametrize("out_bf16", [False, True])
def test_gated_rmsnorm(out_bf16):
    rows, Hv = 77, 48
    log(f"gated_rmsnorm rows={rows} bf16_out={out_bf16}")
    r = np.random.default_rng(11)
    o = r.standard_normal((rows, Hv, 128)).astype(np.float32) * 0.3
    z = synth.bf16_bits(r.standard_normal((rows, Hv, 128)).astype(np.float32))
    w = (1 + 0.02 * r.standard_normal(128)).astype(np.float32)
    out = ops.gdn_gated_rmsnorm(dev_f32(o), dev_bf16(z), dev_f32(w), out_bf16=out_bf16)
    ref = oracle.gated_rmsnorm(o, z, w, eps=1e-6, stage_bf16=out_bf16)
    if out_bf16:
        assert_bf16_within_1ulp(host(out), ref, "out")
    else:
        assert_close(host(out), ref, "out")


def test_gated_rmsnorm_in_place():
    rows, Hv = 10, 4
    log("gated_rmsnorm in place")
    r = np.random.default_rng(12)
    o = r.standard_normal((rows, Hv, 128)).astype(np.float32)
    z = synth.bf16_bits(r.standard_normal((rows, Hv, 128)).astype(np.float32))
    w = np.ones(128, dtype=np.float32)
    od = dev_f32(o)
    ops.gdn_gated_rmsnorm(od, dev_bf16(z), dev_f32(w), out=od)
    assert_close(host(od), oracle.gated_rmsnorm(o, z, w), "out")


# ----------------------------------------------------------------- fused prefill mixer

def _unfused_mixer(x, w, bias, cs, g, beta, z, nw, h0, cu, n_seqs, Hk, Hv, out_bf16, scale=1.0):
    T = x.shape[0]
    y = ops.gdn_conv1d_fwd(x, w, bias=bias, conv_state=cs, cu_seqlens=cu, n_seqs=n_seqs,
                           n_l2_heads=2 * Hk).view(T, 2 * Hk + Hv, 128)
    o, hT = ops.gdn_chunk_fwd(y[:, :Hk], y[:, Hk:2 * Hk], y[:, 2 * Hk:], g, beta,
                              initial_state=h0, cu_seqlens=cu, n_seqs=n_seqs, scale=scale)
    return ops.gdn_gated_rmsnorm(o, z, nw, out_bf16=out_bf16), hT


@pytest.mark.parametrize("case", ["single", "varlen", "varlen_wide", "equal_split"])
def test_mixer_fwd_equals_unfused(case):
    """gdn_mixer_fwd (conv front for q, k inside the prep kernel, for v inside
    the scan kernel) against the separate conv, prefill and norm calls on the
    same inputs: out, final states and the conv window identical bit for bit.
    The cases take the scan's three forms: 32 channels per work-group
    (single, equal_split), 64 channels (varlen), and 64 channels without the
    L2 touch of the V rows (varlen_wide: 64 (sequence, key head) chains)."""
    if case == "single":
        lens, Hk, Hv, out_bf16, with_cs, with_bias = [200], 16, 48, False, False, False
    elif case == "varlen":
        lens, Hk, Hv, out_bf16, with_cs, with_bias = [70, 0, 1, 130, 3, 64], 4, 12, True, True, True
    elif case == "varlen_wide":
        lens, Hk, Hv, out_bf16, with_cs, with_bias = [150, 64, 2, 90], 16, 48, False, True, True
    else:
        lens, Hk, Hv, out_bf16, with_cs, with_bias = [64, 64, 64], 2, 6, False, True, False
    T, N = sum(lens), len(lens)
    log(f"mixer_fwd vs unfused: {case} lens={lens} Hk={Hk} Hv={Hv} bf16_out={out_bf16}")
    mi = synth.mixer_inputs(3600 + N, T, Hk=Hk, Hv=Hv, conv_state_seqs=N if with_cs else 0)
    r = np.random.default_rng(37)
    bias = dev_f32((0.1 * r.standard_normal(mi.x.shape[1])).astype(np.float32)) if with_bias else None
    h0 = dev_f32((0.05 * r.standard_normal((N, Hv, 128, 128))).astype(np.float32))
    cu = dev_i32(synth.cu_from_lengths(lens)) if case.startswith("varlen") else None
    x, w, z, nw = dev_bf16(mi.x), dev_bf16(mi.conv_w), dev_bf16(mi.z), dev_f32(mi.norm_w)
    g, b = dev_f32(mi.g), dev_f32(mi.beta)
    cs1 = dev_bf16(mi.conv_state) if with_cs else None
    cs2 = dev_bf16(mi.conv_state) if with_cs else None
    out1, h1 = ops.gdn_mixer_fwd(x, w, g, b, z, nw, Hk=Hk, conv_bias=bias, conv_state=cs1,
                                 initial_state=h0, cu_seqlens=cu, n_seqs=N, out_bf16=out_bf16)
    out2, h2 = _unfused_mixer(x, w, bias, cs2, g, b, z, nw, h0, cu, N, Hk, Hv, out_bf16)
    torch.cuda.synchronize()
    assert torch.equal(out1, out2), "out"
    assert torch.equal(h1, h2), "final_state"
    if with_cs:
        assert torch.equal(cs1, cs2), "conv_state"


def test_mixer_fwd_long_segmented():
    """B=1, T = 2 * 16384 + 100: gdn_mixer_fwd through the overlapped launch
    (the conv front inside the prep of every segment, the last segment short)
    against the four separate launches: out, final state bit for bit."""
    T = 2 * 16384 + 100
    log(f"mixer_fwd T={T} (segmented) against the four launches")
    mi = synth.mixer_inputs_torch(3900, T)
    x, w, z, nw, g, b = mi["x"], mi["conv_w"], mi["z"], mi["norm_w"], mi["g"], mi["beta"]
    out1, h1 = ops.gdn_mixer_fwd(x, w, g, b, z, nw, Hk=16, n_seqs=1)
    y = ops.gdn_conv1d_fwd(x, w, n_l2_heads=32).view(T, 80, 128)
    o, h2 = ops.gdn_chunk_fwd(y[:, :16], y[:, 16:32], y[:, 32:], g, b)
    out2 = ops.gdn_gated_rmsnorm(o, z, nw)
    torch.cuda.synchronize()
    assert torch.equal(out1, out2), "out"
    assert torch.equal(h1, h2), "final_state"


def test_mixer_fwd_gates_from_projections():
    """gdn_mixer_fwd with the gates formed from bf16 projections: bit-identical
    to conv -> gdn_chunk_fwd_gated -> norm, and against the oracle's gate
    preparation followed by conv -> recurrence -> gated norm."""
    lens, Hk, Hv = [100, 1, 70], 4, 12
    T, N = sum(lens), len(lens)
    log(f"mixer_fwd, gates from projections, lens={lens}")
    mi = synth.mixer_inputs(3750, T, Hk=Hk, Hv=Hv, conv_state_seqs=N)
    gi = synth.gate_inputs(3751, T, Hv=Hv)
    cu = synth.cu_from_lengths(lens)
    x, w, z, nw = dev_bf16(mi.x), dev_bf16(mi.conv_w), dev_bf16(mi.z), dev_f32(mi.norm_w)
    ga, gb, A_log, dt = dev_bf16(gi.a), dev_bf16(gi.b), dev_f32(gi.A_log), dev_f32(gi.dt_bias)
    cs1, cs2 = dev_bf16(mi.conv_state), dev_bf16(mi.conv_state)
    out1, h1 = ops.gdn_mixer_fwd(x, w, None, None, z, nw, Hk=Hk, a=ga, b=gb, A_log=A_log,
                                 dt_bias=dt, conv_state=cs1, cu_seqlens=dev_i32(cu))
    y = ops.gdn_conv1d_fwd(x, w, conv_state=cs2, cu_seqlens=dev_i32(cu),
                           n_l2_heads=2 * Hk).view(T, 2 * Hk + Hv, 128)
    o, h2 = ops.gdn_chunk_fwd_gated(y[:, :Hk], y[:, Hk:2 * Hk], y[:, 2 * Hk:], ga, gb, A_log, dt,
                                    cu_seqlens=dev_i32(cu))
    out2 = ops.gdn_gated_rmsnorm(o, z, nw)
    torch.cuda.synchronize()
    assert torch.equal(out1, out2) and torch.equal(h1, h2) and torch.equal(cs1, cs2)
    g, beta = oracle.gate_prep(gi.a, gi.b, gi.A_log, gi.dt_bias)
    ry, _ = oracle.conv1d(mi.x, mi.conv_w, conv_state=mi.conv_state, cu_seqlens=cu,
                          n_l2_heads=2 * Hk, head_dim=128, stage_bf16=True)
    ry = ry.reshape(T, 2 * Hk + Hv, 128)
    ro, rT = oracle.recurrence(ry[:, :Hk], ry[:, Hk:2 * Hk], ry[:, 2 * Hk:], g, beta,
                               cu_seqlens=cu, n_seqs=N)
    assert_close(host(out1), oracle.gated_rmsnorm(ro, mi.z, mi.norm_w), "out")
    assert_close(host(h1), rT, "final_state")


def test_mixer_fwd_with_state_pools():
    """gdn_mixer_fwd over pools of states and conv windows (slot map, in place)
    equals the call on the gathered rows, scattered back, bit for bit; pool
    rows no sequence names are untouched."""
    lens, Hk, Hv, n_slots = [90, 0, 1, 70], 2, 6, 7
    T, N = sum(lens), len(lens)
    log(f"mixer_fwd with state pools, lens={lens}")
    mi = synth.mixer_inputs(3800, T, Hk=Hk, Hv=Hv, conv_state_seqs=n_slots)
    pool = (0.05 * np.random.default_rng(39).standard_normal((n_slots, Hv, 128, 128))).astype(np.float32)
    slots = np.array([5, 0, 3, 6], dtype=np.int32)
    cu = dev_i32(synth.cu_from_lengths(lens))
    x, w, z, nw = dev_bf16(mi.x), dev_bf16(mi.conv_w), dev_bf16(mi.z), dev_f32(mi.norm_w)
    g, b = dev_f32(mi.g), dev_f32(mi.beta)
    cs_pool, st_pool = dev_bf16(mi.conv_state), dev_f32(pool)
    out1, _ = ops.gdn_mixer_fwd(x, w, g, b, z, nw, Hk=Hk, conv_state=cs_pool, initial_state=st_pool,
                                state_slot=dev_i32(slots), cu_seqlens=cu)
    cs_g, st_g = dev_bf16(mi.conv_state[slots]), dev_f32(pool[slots])
    out2, hT = ops.gdn_mixer_fwd(x, w, g, b, z, nw, Hk=Hk, conv_state=cs_g, initial_state=st_g,
                                 cu_seqlens=cu)
    torch.cuda.synchronize()
    assert torch.equal(out1, out2)
    idx = torch.from_numpy(slots.astype(np.int64)).cuda()
    assert torch.equal(st_pool[idx], hT) and torch.equal(cs_pool[idx], cs_g)
    others = [i for i in range(n_slots) if i not in slots]
    np.testing.assert_array_equal(host(st_pool)[others], pool[others])
    assert torch.equal(cs_pool[others], dev_bf16(mi.conv_state)[others])


def test_mixer_fwd_padding_slot():
    """gdn_mixer_fwd over pools with a padding sequence (slot -1): the real
    sequences' out rows, states and conv windows equal those of the call on
    the real sequences alone (bit for bit), and no other pool row changes."""
    lens, Hk, Hv, n_slots = [40, 70, 1, 129], 2, 6, 7
    T, N = sum(lens), len(lens)
    log(f"mixer_fwd with a padding slot, lens={lens}")
    mi = synth.mixer_inputs(3850, T, Hk=Hk, Hv=Hv, conv_state_seqs=n_slots)
    pool = (0.05 * np.random.default_rng(43).standard_normal((n_slots, Hv, 128, 128))).astype(np.float32)
    slots = np.array([2, -1, 6, 4], dtype=np.int32)
    keep = [0, 2, 3]
    cu = synth.cu_from_lengths(lens)
    x, w, z, nw = dev_bf16(mi.x), dev_bf16(mi.conv_w), dev_bf16(mi.z), dev_f32(mi.norm_w)
    g, b = dev_f32(mi.g), dev_f32(mi.beta)
    cs_pool, st_pool = dev_bf16(mi.conv_state), dev_f32(pool)
    out1, _ = ops.gdn_mixer_fwd(x, w, g, b, z, nw, Hk=Hk, conv_state=cs_pool, initial_state=st_pool,
                                state_slot=dev_i32(slots), cu_seqlens=dev_i32(cu))
    rows = np.concatenate([np.arange(cu[n], cu[n + 1]) for n in keep])
    ridx = torch.from_numpy(rows.astype(np.int64)).cuda()
    cu2 = np.concatenate([[0], np.cumsum([lens[n] for n in keep])]).astype(np.int32)
    cs_g, st_g = dev_bf16(mi.conv_state[slots[keep]]), dev_f32(pool[slots[keep]])
    out2, hT = ops.gdn_mixer_fwd(x[ridx].contiguous(), w, g[ridx].contiguous(), b[ridx].contiguous(),
                                 z[ridx].contiguous(), nw, Hk=Hk, conv_state=cs_g, initial_state=st_g,
                                 cu_seqlens=dev_i32(cu2))
    torch.cuda.synchronize()
    assert torch.equal(out1[ridx], out2), "out (real sequences)"
    idx = torch.from_numpy(slots[keep].astype(np.int64)).cuda()
    assert torch.equal(st_pool[idx], hT) and torch.equal(cs_pool[idx], cs_g)
    others = [i for i in range(n_slots) if i not in slots[keep]]
    np.testing.assert_array_equal(host(st_pool)[others], pool[others])
    assert torch.equal(cs_pool[others], dev_bf16(mi.conv_state)[others])


def test_mixer_fwd_against_oracle():
    """The fused mixer against the oracle's conv -> recurrence -> gated norm,
    varlen with conv states, initial states and an empty sequence."""
    lens, Hk, Hv = [90, 0, 5, 140], 4, 12
    T, N = sum(lens), len(lens)
    log(f"mixer_fwd vs oracle lens={lens}")
    mi = synth.mixer_inputs(3650, T, Hk=Hk, Hv=Hv, conv_state_seqs=N)
    h0 = (0.05 * np.random.default_rng(38).standard_normal((N, Hv, 128, 128))).astype(np.float32)
    cu = synth.cu_from_lengths(lens)
    cs = dev_bf16(mi.conv_state)
    out, hT = ops.gdn_mixer_fwd(dev_bf16(mi.x), dev_bf16(mi.conv_w), dev_f32(mi.g), dev_f32(mi.beta),
                                dev_bf16(mi.z), dev_f32(mi.norm_w), Hk=Hk, conv_state=cs,
                                initial_state=dev_f32(h0), cu_seqlens=dev_i32(cu))
    ry, rcs = oracle.conv1d(mi.x, mi.conv_w, conv_state=mi.conv_state, cu_seqlens=cu,
                            n_l2_heads=2 * Hk, head_dim=128, stage_bf16=True)
    ry = ry.reshape(T, 2 * Hk + Hv, 128)
    ro, rT = oracle.recurrence(ry[:, :Hk], ry[:, Hk:2 * Hk], ry[:, 2 * Hk:], mi.g, mi.beta, h0,
                               cu_seqlens=cu, n_seqs=N)
    rout = oracle.gated_rmsnorm(ro, mi.z, mi.norm_w)
    assert_close(host(out), rout, "out")
    assert_close(host(hT), rT, "final_state")
    np.testing.assert_array_equal(host(cs), rcs)


# ----------------------------------------------------------------- fused decode step

def _mixer_step_case(seed, N, Hk, Hv, n_slots):
    mi = synth.mixer_inputs(seed, N, Hk=Hk, Hv=Hv, conv_state_seqs=n_slots)
    pool = synth.decode_inputs(seed + 1, n_slots, Hk=Hk, Hv=Hv, with_conv=False).state
    return mi, pool


def oracle_mixer_step(mi, pool, Hk, Hv, slots, bias=None, scale=1.0, out_bf16=False):
    """conv (one token per sequence, history from its slot) -> L2 of q, k ->
    one step of the rule on the slot's state -> gated RMSNorm, all in the oracle."""
    N = mi.x.shape[0]
    ry, rcs = oracle.conv1d(mi.x, mi.conv_w, bias=bias, conv_state=mi.conv_state[slots], n_seqs=N,
                            n_l2_heads=2 * Hk, head_dim=128, l2_eps=1e-6, stage_bf16=True)
    ry = ry.reshape(N, 2 * Hk + Hv, 128)
    ro, rst = oracle.decode(ry[:, :Hk], ry[:, Hk:2 * Hk], ry[:, 2 * Hk:], mi.g, mi.beta, pool,
                            state_slot=slots, scale=scale)
    rout = oracle.gated_rmsnorm(ro, mi.z, mi.norm_w, eps=1e-6, stage_bf16=out_bf16)
    return rout, rcs, rst


@pytest.mark.parametrize("N,Hk,Hv,slotted,out_bf16", [
    (1, 16, 48, False, False), (5, 16, 48, True, False), (3, 2, 2, False, True),
    (4, 4, 8, True, True), (2, 2, 8, False, False), (7, 3, 9, True, False)])
def test_decode_mixer_step_against_oracle(N, Hk, Hv, slotted, out_bf16):
    """The fused step: normalised output, the conv window and the state of every
    slot it used, against the oracle's conv -> rule -> norm; slots it did not
    use are left as they were, bit for bit."""
    n_slots = N + 3 if slotted else N
    log(f"decode_mixer_step N={N} Hk={Hk} Hv={Hv} slotted={slotted} bf16_out={out_bf16}")
    mi, pool = _mixer_step_case(3300 + 7 * N + Hv, N, Hk, Hv, n_slots)
    r = np.random.default_rng(N + Hv)
    slots = (r.permutation(n_slots)[:N] if slotted else np.arange(N)).astype(np.int32)
    bias = (0.1 * r.standard_normal(mi.x.shape[1])).astype(np.float32) if slotted else None
    scale = 0.6 if slotted else 1.0
    cs, st = dev_bf16(mi.conv_state), dev_f32(pool)
    out = ops.gdn_decode_mixer_step(dev_bf16(mi.x), dev_bf16(mi.conv_w), cs, dev_f32(mi.g),
                                    dev_f32(mi.beta), dev_bf16(mi.z), dev_f32(mi.norm_w), st, Hk=Hk,
                                    conv_bias=None if bias is None else dev_f32(bias),
                                    state_slot=dev_i32(slots) if slotted else None, scale=scale,
                                    out_bf16=out_bf16)
    rout, rcs, rst = oracle_mixer_step(mi, pool, Hk, Hv, slots, bias=bias, scale=scale,
                                       out_bf16=out_bf16)
    if out_bf16:
        # both sides round once to bf16 (the oracle from fp64): one ulp apart at most
        assert out.dtype == torch.bfloat16
        assert_bf16_within_1ulp(host(out), rout, "out (bf16)")
    else:
        assert_close(host(out), rout, "out")
    got_cs, got_st = host(cs), host(st)
    np.testing.assert_array_equal(got_cs[slots], rcs)
    assert_close(got_st[slots], rst[slots], "state (slots used)")
    others = [i for i in range(n_slots) if i not in slots]
    cs_bits = cs.cpu().view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(cs_bits[others], mi.conv_state[others])
    np.testing.assert_array_equal(got_st[others], pool[others])


def test_decode_mixer_step_gates_from_projections():
    """The fused decode step with the gates formed from bf16 projections
    (a, b as columns of a wider buffer) against the oracle's gate preparation
    followed by conv -> rule -> norm, with a slot map."""
    N, Hk, Hv, n_slots = 5, 4, 12, 8
    log("decode_mixer_step, gates from projections")
    mi, pool = _mixer_step_case(3700, N, Hk, Hv, n_slots)
    gi = synth.gate_inputs(3701, N, Hv=Hv)
    slots = np.array([6, 1, 3, 0, 7], dtype=np.int32)
    wide = torch.zeros((N, 2 * Hv + 16), dtype=torch.bfloat16, device="cuda")
    wide[:, 16:16 + Hv] = dev_bf16(gi.a)
    wide[:, 16 + Hv:] = dev_bf16(gi.b)
    cs, st = dev_bf16(mi.conv_state), dev_f32(pool)
    out = ops.gdn_decode_mixer_step(dev_bf16(mi.x), dev_bf16(mi.conv_w), cs, None, None,
                                    dev_bf16(mi.z), dev_f32(mi.norm_w), st, Hk=Hk,
                                    a=wide[:, 16:16 + Hv], b=wide[:, 16 + Hv:],
                                    A_log=dev_f32(gi.A_log), dt_bias=dev_f32(gi.dt_bias),
                                    state_slot=dev_i32(slots))
    g, beta = oracle.gate_prep(gi.a, gi.b, gi.A_log, gi.dt_bias)
    mg = synth.MixerInputs(mi.x, mi.conv_w, g, beta, mi.z, mi.norm_w, mi.conv_state)
    rout, rcs, rst = oracle_mixer_step(mg, pool, Hk, Hv, slots)
    assert_close(host(out), rout, "out")
    assert_close(host(st)[slots], rst[slots], "state (slots used)")
    np.testing.assert_array_equal(host(cs)[slots], rcs)


@pytest.mark.parametrize("out_bf16", [False, True])
def test_decode_mixer_step_matches_unfused(out_bf16):
    """One fused call against the three separate calls it replaces (batch conv
    with the conv window, gdn_decode_step, gdn_gated_rmsnorm) on the same
    device inputs: identical conv windows, states and outputs up to the
    reduction order of the two L2 norms."""
    N, Hk, Hv = 33, 16, 48
    log(f"decode_mixer_step vs conv + decode_step + gated_rmsnorm, N={N} bf16_out={out_bf16}")
    mi, pool = _mixer_step_case(3400, N, Hk, Hv, N)
    x, w, z, nw = dev_bf16(mi.x), dev_bf16(mi.conv_w), dev_bf16(mi.z), dev_f32(mi.norm_w)
    g, b = dev_f32(mi.g), dev_f32(mi.beta)
    cs1, st1 = dev_bf16(mi.conv_state), dev_f32(pool)
    out1 = ops.gdn_decode_mixer_step(x, w, cs1, g, b, z, nw, st1, Hk=Hk, scale=0.8,
                                     out_bf16=out_bf16)
    cs2, st2 = dev_bf16(mi.conv_state), dev_f32(pool)
    y = ops.gdn_conv1d_fwd(x, w, conv_state=cs2, n_seqs=N, n_l2_heads=2 * Hk).view(N, 2 * Hk + Hv, 128)
    o = ops.gdn_decode_step(y[:, :Hk], y[:, Hk:2 * Hk], y[:, 2 * Hk:], g, b, st2, scale=0.8)
    out2 = ops.gdn_gated_rmsnorm(o, z, nw, out_bf16=out_bf16)
    torch.cuda.synchronize()
    assert torch.equal(cs1, cs2)
    for name, a1, a2 in (("state", st1, st2), ("out", out1, out2)):
        if out_bf16 and name == "out":
            # each path rounds its fp32 result to bf16 once
            assert_bf16_within_1ulp(host(a1), host(a2), "out (bf16), fused vs unfused")
            continue
        a1, a2 = a1.double(), a2.double()
        err = ((a1 - a2).abs().max() / a2.abs().max()).item()
        rel = ((a1 - a2).norm() / a2.norm()).item()
        log(f"  {name}: max|fused - unfused| / max = {err:.3e}, rel_l2 = {rel:.3e}")
        assert rel <= 1e-4, name


# ----------------------------------------------------------------- full mixer

def test_mixer_conv_chunk_norm():
    """conv front -> chunked rule -> gated norm, as one layer's token mixer."""
    T = 200
    log(f"mixer T={T}")
    mi = synth.mixer_inputs(3100, T)
    y = ops.gdn_conv1d_fwd(dev_bf16(mi.x), dev_bf16(mi.conv_w), n_l2_heads=32)
    yv = y.view(T, 80, 128)
    q, k, v = yv[:, :16], yv[:, 16:32], yv[:, 32:]
    o, hT = ops.gdn_chunk_fwd(q, k, v, dev_f32(mi.g), dev_f32(mi.beta))
    out = ops.gdn_gated_rmsnorm(o, dev_bf16(mi.z), dev_f32(mi.norm_w))
    ry, _ = oracle.conv1d(mi.x, mi.conv_w, n_l2_heads=32, head_dim=128, stage_bf16=True)
    ry = ry.reshape(T, 80, 128)
    ro, rT = oracle.recurrence(ry[:, :16], ry[:, 16:32], ry[:, 32:], mi.g, mi.beta)
    rout = oracle.gated_rmsnorm(ro, mi.z, mi.norm_w)
    assert_close(host(o), ro, "o")
    assert_close(host(hT), rT, "final_state")
    assert_close(host(out), rout, "norm out")


# ----------------------------------------------------------------- padding slots

def test_padding_slots_skip_their_sequences():
    """A slot outside [0, n_slots) (-1, or n_slots itself) marks a padding
    sequence: the decode step, the multi-token step, the fused decode mixer
    step and the pooled prefill leave every pool row and that sequence's
    output rows untouched, and the real sequences match the oracle."""
    rng = np.random.default_rng(41)
    N, n_slots, Hk, Hv = 5, 7, 2, 6
    slots = np.array([3, -1, 0, 7, 5], dtype=np.int32)     # sequences 1 and 3 are padding
    real = np.array([0, 2, 4])
    sentinel = 12345.0

    # one-token decode step
    log("padding slots: decode_step")
    di = synth.decode_inputs(4100, N, Hk=Hk, Hv=Hv, with_conv=False)
    pool = rng.standard_normal((n_slots, Hv, 128, 128)).astype(np.float32) * 0.02
    st = dev_f32(pool)
    o = torch.full((N, Hv, 128), sentinel, dtype=torch.float32, device="cuda")
    ops.gdn_decode_step(dev_bf16(di.q), dev_bf16(di.k), dev_bf16(di.v), dev_f32(di.g),
                        dev_f32(di.beta), st, state_slot=dev_i32(slots), o=o)
    ro, rst = oracle.decode(di.q[real], di.k[real], di.v[real], di.g[real], di.beta[real], pool,
                            state_slot=slots[real])
    got, got_st = host(o), host(st)
    assert_close(got[real], ro, "o (real sequences)")
    assert np.all(got[[1, 3]] == sentinel)
    assert_close(got_st[slots[real]], rst[slots[real]], "states (real slots)")
    others = [i for i in range(n_slots) if i not in slots[real]]
    np.testing.assert_array_equal(got_st[others], pool[others])

    # three tokens per sequence
    log("padding slots: decode_tokens")
    nt = 3
    ti = synth.decode_inputs(4101, N * nt, Hk=Hk, Hv=Hv, with_conv=False)
    st = dev_f32(pool)
    o = torch.full((N * nt, Hv, 128), sentinel, dtype=torch.float32, device="cuda")
    ops.gdn_decode_tokens(dev_bf16(ti.q), dev_bf16(ti.k), dev_bf16(ti.v), dev_f32(ti.g),
                          dev_f32(ti.beta), st, nt, state_slot=dev_i32(slots), o=o)
    got, got_st = host(o), host(st)
    rows = np.concatenate([np.arange(n * nt, n * nt + nt) for n in real])
    cu = np.arange(0, len(real) * nt + 1, nt, dtype=np.int32)
    ro, rT = oracle.recurrence(ti.q[rows], ti.k[rows], ti.v[rows], ti.g[rows], ti.beta[rows],
                               pool[slots[real]], cu_seqlens=cu, n_seqs=len(real))
    assert_close(got[rows], ro, "o (real sequences)")
    pad_rows = np.concatenate([np.arange(n * nt, n * nt + nt) for n in (1, 3)])
    assert np.all(got[pad_rows] == sentinel)
    assert_close(got_st[slots[real]], rT, "states (real slots)")
    np.testing.assert_array_equal(got_st[others], pool[others])

    # the whole mixer's decode step: conv window and state pools
    log("padding slots: decode_mixer_step")
    mi = synth.mixer_inputs(4102, N, Hk=Hk, Hv=Hv)
    C = (2 * Hk + Hv) * 128
    cst = dev_bf16(synth.bf16_bits(rng.standard_normal((n_slots, C, 3)).astype(np.float32)))
    cst0 = cst.clone()
    st = dev_f32(pool)
    out = torch.full((N, Hv, 128), sentinel, dtype=torch.float32, device="cuda")
    ops.gdn_decode_mixer_step(dev_bf16(mi.x), dev_bf16(mi.conv_w), cst, dev_f32(mi.g),
                              dev_f32(mi.beta), dev_bf16(mi.z), dev_f32(mi.norm_w), st, Hk=Hk,
                              state_slot=dev_i32(slots), out=out)
    got, got_st = host(out), host(st)
    assert np.all(got[[1, 3]] == sentinel)
    np.testing.assert_array_equal(got_st[others], pool[others])
    unnamed = [i for i in range(n_slots) if i not in slots[real]]
    assert torch.equal(cst[unnamed], cst0[unnamed])
    assert np.all(np.isfinite(got[real]))

    # pooled prefill with a padding sequence of 70 tokens
    log("padding slots: chunk_fwd_pooled")
    lens = [40, 70, 1, 129]
    pslots = np.array([2, -1, 6, 4], dtype=np.int32)
    ci = synth.chunk_inputs(4103, sum(lens), Hk=Hk, Hv=Hv, lengths=lens)
    st = dev_f32(pool)
    T = sum(lens)
    o = torch.full((T, Hv, 128), sentinel, dtype=torch.float32, device="cuda")
    ops.gdn_chunk_fwd_pooled(dev_bf16(ci.q), dev_bf16(ci.k), dev_bf16(ci.v), dev_f32(ci.g),
                             dev_f32(ci.beta), st, dev_i32(pslots),
                             cu_seqlens=dev_i32(ci.cu_seqlens), o=o)
    got, got_st = host(o), host(st)
    keep = [0, 2, 3]
    rows = np.concatenate([np.arange(ci.cu_seqlens[n], ci.cu_seqlens[n + 1]) for n in keep])
    cu2 = np.concatenate([[0], np.cumsum([lens[n] for n in keep])]).astype(np.int32)
    ro, rT = oracle.recurrence(ci.q[rows], ci.k[rows], ci.v[rows], ci.g[rows], ci.beta[rows],
                               pool[pslots[keep]], cu_seqlens=cu2, n_seqs=len(keep))
    assert_close(got[rows], ro, "o (real sequences)")
    assert np.all(got[ci.cu_seqlens[1]:ci.cu_seqlens[2]] == sentinel)
    assert_close(got_st[pslots[keep]], rT, "states (real slots)")
    untouched = [i for i in range(n_slots) if i not in pslots[keep]]
    np.testing.assert_array_equal(got_st[untouched], pool[untouched])
