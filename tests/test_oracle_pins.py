"""Pins of the fp64 oracle against facts that do not come from the oracle itself.

Every routine of the oracle is checked here against invariants of the rule,
closed forms, a brute-force unrolled form, an independent chunked (WY)
formulation, and library routines (torch conv1d / rms_norm / bf16 cast, in
fp64 on the CPU), with special cases chosen so that a dropped term, a wrong
sign, a transposed state or a wrong head/sequence index fails at least one.
"""
import numpy as np
import pytest
import torch

import oracle
from tests import forms

RNG = np.random.default_rng


def unit(a):
    return a / np.linalg.norm(a, axis=-1, keepdims=True)


def rand_inputs(seed, T, Hk, Hv, d, dv=None, h0=True, N=1):
    r = RNG(seed)
    dv = dv or d
    q = unit(r.standard_normal((T, Hk, d)))
    k = unit(r.standard_normal((T, Hk, d)))
    v = r.standard_normal((T, Hv, dv))
    g = r.uniform(-0.3, 0.0, (T, Hv))
    b = 1.0 / (1.0 + np.exp(-r.standard_normal((T, Hv))))
    S0 = r.standard_normal((N, Hv, dv, d)) * 0.3 if h0 else None
    return q, k, v, g, b, S0


# ---------------------------------------------------------------- recurrence

def test_pin_a_delta_invariant():
    """beta=1, alpha=1, |k|=1: S_t k_t = v_t for every t.  With q=k, o_t = v_t."""
    T, Hk, Hv, d = 200, 2, 6, 32
    q, k, v, g, b, S0 = rand_inputs(1, T, Hk, Hv, d)
    g[:] = 0.0
    b[:] = 1.0
    o, _ = oracle.recurrence(k, k, v, g, b, S0)
    assert np.max(np.abs(o - v)) <= 1e-12


def test_pin_b_decay_closed_form_asymmetric_state():
    """beta=0: S_t = exp(G_t) S0 and o_t = exp(G_t) S0 q_t.  S0 is asymmetric so
    the row = value-index orientation is pinned (S0^T q would fail)."""
    T, Hk, Hv, d, dv = 40, 2, 6, 16, 24   # dv != dk also pins the orientation
    q, k, v, g, b, S0 = rand_inputs(2, T, Hk, Hv, d, dv=dv)
    b[:] = 0.0
    scale = 0.37
    o, ST = oracle.recurrence(q, k, v, g, b, S0, scale=scale)
    G = np.cumsum(g, axis=0)   # [T, Hv]
    for h in range(Hv):
        kh = h // 3
        ref = scale * np.exp(G[:, h])[:, None] * (q[:, kh] @ S0[0, h].T)
        np.testing.assert_allclose(o[:, h], ref, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(ST[0, h], np.exp(G[-1, h]) * S0[0, h], rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("T", [1, 2, 7, 32])
def test_pin_c_bruteforce_unrolled(T):
    """Agreement with the unrolled product form on T <= 32."""
    Hk, Hv, d, dv = 2, 6, 12, 10
    q, k, v, g, b, S0 = rand_inputs(10 + T, T, Hk, Hv, d, dv=dv)
    scale = 0.8
    o, ST = oracle.recurrence(q, k, v, g, b, S0, scale=scale)
    for h in range(Hv):
        qq, kk, vv, gg, bb, s0 = forms.heads(q, k, v, g, b, S0, 0, h, 3)
        ro, rS = forms.unrolled(qq, kk, vv, gg, bb, s0, scale)
        assert np.linalg.norm(o[:, h] - ro) <= 1e-12 * max(1.0, np.linalg.norm(ro))
        assert np.linalg.norm(ST[0, h] - rS) <= 1e-12 * max(1.0, np.linalg.norm(rS))


def test_pin_d_identical_keys_overwrite():
    """Identical unit keys, beta=1, alpha=1, S0=0: the memory holds only the
    last value, so o_t = v_t (k . q_t)."""
    T, Hk, Hv, d = 20, 1, 3, 16
    q, k, v, g, b, _ = rand_inputs(3, T, Hk, Hv, d)
    k[:] = k[0:1]
    g[:] = 0.0
    b[:] = 1.0
    o, _ = oracle.recurrence(q, k, v, g, b, None)
    for h in range(Hv):
        ref = v[:, h] * (q[:, 0] @ k[0, 0])[:, None]
        np.testing.assert_allclose(o[:, h], ref, rtol=1e-12, atol=1e-13)


def test_pin_e_one_step_invariant():
    """|k|=1: S_t k_t = a_t (1 - b_t) S_{t-1} k_t + b_t v_t, for any a, b."""
    Hk, Hv, d = 2, 6, 16
    q, k, v, g, b, S0 = rand_inputs(4, 5, Hk, Hv, d)
    state = S0.copy()
    for t in range(5):
        # o of a decode step with q = k is S_t k_t
        o, new = oracle.decode(k[t:t + 1], k[t:t + 1], v[t:t + 1], g[t:t + 1], b[t:t + 1], state)
        for h in range(Hv):
            kh = h // 3
            pred = np.exp(g[t, h]) * (1 - b[t, h]) * (state[0, h] @ k[t, kh]) + b[t, h] * v[t, h]
            np.testing.assert_allclose(o[0, h], pred, rtol=1e-12, atol=1e-13)
        state = new


def test_pin_f_linearity_in_state_and_values():
    """o and S_T are jointly linear in (S0, V)."""
    T, Hk, Hv, d = 30, 2, 6, 8
    q, k, v, g, b, S0 = rand_inputs(5, T, Hk, Hv, d)
    _, _, v2, _, _, S02 = rand_inputs(6, T, Hk, Hv, d)
    a1, a2 = 0.7, -1.3
    o1, s1 = oracle.recurrence(q, k, v, g, b, S0)
    o2, s2 = oracle.recurrence(q, k, v2, g, b, S02)
    o3, s3 = oracle.recurrence(q, k, a1 * v + a2 * v2, g, b, a1 * S0 + a2 * S02)
    np.testing.assert_allclose(o3, a1 * o1 + a2 * o2, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(s3, a1 * s1 + a2 * s2, rtol=1e-11, atol=1e-12)


def test_pin_f_head_group_equivariance():
    """Permuting key heads together with their groups of value heads permutes
    the outputs the same way (pins the value-head -> key-head map h // 3)."""
    T, Hk, Hv, d = 25, 4, 12, 8
    q, k, v, g, b, S0 = rand_inputs(7, T, Hk, Hv, d)
    perm_k = np.array([2, 0, 3, 1])
    perm_v = np.concatenate([np.arange(3 * p, 3 * p + 3) for p in perm_k])
    o, s = oracle.recurrence(q, k, v, g, b, S0)
    op, sp = oracle.recurrence(q[:, perm_k], k[:, perm_k], v[:, perm_v], g[:, perm_v],
                               b[:, perm_v], S0[:, perm_v])
    np.testing.assert_array_equal(op, o[:, perm_v])
    np.testing.assert_array_equal(sp, s[:, perm_v])
    # a wrong (interleaved) head map would not be equivariant; make sure the
    # groups actually differ so the check has teeth
    assert np.max(np.abs(o[:, 0] - o[:, 3])) > 1e-3


@pytest.mark.parametrize("T,chunk", [(64, 64), (200, 64), (130, 16), (65, 64), (1, 64)])
def test_pin_g_chunked_wy_form(T, chunk):
    """The chunked WY/UT form (partial chunks, nonzero S0) equals the oracle."""
    Hk, Hv, d = 2, 6, 32
    q, k, v, g, b, S0 = rand_inputs(8 + T, T, Hk, Hv, d)
    o, ST = oracle.recurrence(q, k, v, g, b, S0, scale=0.5)
    for h in range(Hv):
        qq, kk, vv, gg, bb, s0 = forms.heads(q, k, v, g, b, S0, 0, h, 3)
        ro, rS = forms.chunked(qq, kk, vv, gg, bb, s0, chunk=chunk, scale=0.5)
        assert np.max(np.abs(o[:, h] - ro)) <= 1e-11 * max(1.0, np.max(np.abs(ro)))
        assert np.max(np.abs(ST[0, h] - rS)) <= 1e-11 * max(1.0, np.max(np.abs(rS)))


def test_pin_g_chunked_full_head_dim():
    """Same at the layer's head dim 128 with a strong decay."""
    T, Hk, Hv, d = 150, 1, 3, 128
    q, k, v, g, b, S0 = rand_inputs(9, T, Hk, Hv, d)
    g *= 5.0
    o, ST = oracle.recurrence(q, k, v, g, b, S0)
    for h in range(Hv):
        ro, rS = forms.chunked(*forms.heads(q, k, v, g, b, S0, 0, h, 3))
        assert np.max(np.abs(o[:, h] - ro)) <= 1e-11 * np.max(np.abs(ro))
        assert np.max(np.abs(ST[0, h] - rS)) <= 1e-11 * np.max(np.abs(rS))


def test_varlen_equals_separate_calls():
    """Packed sequences (including empty ones) restart the state at each start."""
    lens = [5, 0, 17, 1, 0, 9]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T = int(cu[-1])
    N = len(lens)
    q, k, v, g, b, S0 = rand_inputs(11, T, 2, 6, 8, N=N)
    o, ST = oracle.recurrence(q, k, v, g, b, S0, cu_seqlens=cu)
    for n in range(N):
        s, e = cu[n], cu[n + 1]
        on, sn = oracle.recurrence(q[s:e], k[s:e], v[s:e], g[s:e], b[s:e], S0[n:n + 1])
        np.testing.assert_array_equal(o[s:e], on)
        np.testing.assert_array_equal(ST[n], sn[0])
    # empty sequences return their initial state
    np.testing.assert_array_equal(ST[1], S0[1])
    np.testing.assert_array_equal(ST[4], S0[4])


def test_decode_equals_recurrence_T1_with_slots():
    """A decode step equals the recurrence with one token per sequence; the slot
    map routes each sequence to its own state."""
    N, Hk, Hv, d = 5, 2, 6, 16
    q, k, v, g, b, S0 = rand_inputs(12, N, Hk, Hv, d, N=N)
    cu = np.arange(N + 1, dtype=np.int32)
    o_r, s_r = oracle.recurrence(q, k, v, g, b, S0, cu_seqlens=cu)
    slots = np.array([3, 0, 6, 2, 5], dtype=np.int32)
    pool = np.random.default_rng(1).standard_normal((7, Hv, d, d))
    pool[slots] = S0
    o_d, new = oracle.decode(q, k, v, g, b, pool, state_slot=slots)
    np.testing.assert_array_equal(o_d, o_r)
    np.testing.assert_array_equal(new[slots], s_r)
    untouched = [i for i in range(7) if i not in slots]
    np.testing.assert_array_equal(new[untouched], pool[untouched])


# ---------------------------------------------------------------- conv front

def torch_conv_ref(x, w, cs=None):
    """fp64 torch conv1d (groups=C, kernel 4, left context) + SiLU."""
    T, C = x.shape
    xt = torch.from_numpy(x.T.copy())[None]          # [1, C, T]
    if cs is None:
        pad = torch.zeros(1, C, 3, dtype=torch.float64)
    else:
        pad = torch.from_numpy(cs.copy())[None]      # [1, C, 3] oldest first
    xt = torch.cat([pad, xt], dim=2)
    y = torch.nn.functional.conv1d(xt, torch.from_numpy(w.copy())[:, None, :], groups=C)
    y = torch.nn.functional.silu(y)
    return y[0].T.numpy()


def test_conv_matches_torch_conv1d_fp64():
    r = RNG(20)
    T, C, hd, nl2 = 37, 48, 8, 4
    x = r.standard_normal((T, C))
    w = r.standard_normal((C, 4)) * 0.5
    cs = r.standard_normal((1, C, 3))
    y, cso = oracle.conv1d(x, w, conv_state=cs, n_l2_heads=nl2, head_dim=hd, l2_eps=1e-6,
                           stage_bf16=False)
    ref = torch_conv_ref(x, w, cs[0])
    heads = ref[:, :nl2 * hd].reshape(T, nl2, hd)
    heads = heads / np.sqrt((heads ** 2).sum(-1, keepdims=True) + 1e-6)
    ref[:, :nl2 * hd] = heads.reshape(T, -1)
    np.testing.assert_allclose(y, ref, rtol=1e-13, atol=1e-14)
    np.testing.assert_array_equal(cso[0], x[-3:].T)


def test_conv_special_taps():
    r = RNG(21)
    T, C = 10, 16
    x = r.standard_normal((T, C))
    silu = lambda a: a / (1 + np.exp(-a))
    w = np.zeros((C, 4))
    w[:, 3] = 1.0      # current token only -> SiLU(x)
    y, _ = oracle.conv1d(x, w, stage_bf16=False)
    np.testing.assert_allclose(y, silu(x), rtol=1e-14)
    w = np.zeros((C, 4))
    w[:, 0] = 1.0      # oldest tap -> 3-token shift
    y, _ = oracle.conv1d(x, w, stage_bf16=False)
    ref = np.zeros_like(x)
    ref[3:] = silu(x[:-3])
    np.testing.assert_allclose(y, ref, rtol=1e-14)


def test_conv_l2_norm_closed_form():
    """|y_hat| = |y| / sqrt(|y|^2 + eps) for every q/k head; v channels untouched."""
    r = RNG(22)
    T, hd, nl2, C = 9, 16, 3, 64
    x = r.standard_normal((T, C)) * 0.05
    w = r.standard_normal((C, 4))
    eps = 1e-3
    y_raw, _ = oracle.conv1d(x, w, n_l2_heads=0, head_dim=hd, stage_bf16=False)
    y, _ = oracle.conv1d(x, w, n_l2_heads=nl2, head_dim=hd, l2_eps=eps, stage_bf16=False)
    for hh in range(nl2):
        raw = np.linalg.norm(y_raw[:, hh * hd:(hh + 1) * hd], axis=1)
        got = np.linalg.norm(y[:, hh * hd:(hh + 1) * hd], axis=1)
        np.testing.assert_allclose(got, raw / np.sqrt(raw ** 2 + eps), rtol=1e-13)
    np.testing.assert_array_equal(y[:, nl2 * hd:], y_raw[:, nl2 * hd:])


def test_conv_state_continuity():
    """prefill(T) followed by one batch-mode step equals prefill(T+1); a
    sequence shorter than 3 keeps part of the old history."""
    r = RNG(23)
    T, C = 12, 24
    x = r.standard_normal((T + 1, C))
    w = r.standard_normal((C, 4))
    cs0 = r.standard_normal((1, C, 3))
    y_full, cs_full = oracle.conv1d(x, w, conv_state=cs0, stage_bf16=False)
    y_a, cs_a = oracle.conv1d(x[:T], w, conv_state=cs0, stage_bf16=False)
    y_b, cs_b = oracle.conv1d(x[T:], w, conv_state=cs_a, stage_bf16=False)
    np.testing.assert_array_equal(np.concatenate([y_a, y_b]), y_full)
    np.testing.assert_array_equal(cs_b, cs_full)
    y1, cs1 = oracle.conv1d(x[:1], w, conv_state=cs0, stage_bf16=False)
    np.testing.assert_array_equal(cs1[0], np.concatenate([cs0[0][:, 1:], x[:1].T], axis=1))


def test_conv_varlen_packed_equals_separate():
    r = RNG(24)
    lens = [4, 0, 1, 9, 2]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    C = 16
    x = r.standard_normal((int(cu[-1]), C))
    w = r.standard_normal((C, 4))
    cs = r.standard_normal((len(lens), C, 3))
    y, cso = oracle.conv1d(x, w, conv_state=cs, cu_seqlens=cu, n_l2_heads=1, head_dim=8,
                           stage_bf16=True)
    for n in range(len(lens)):
        s, e = cu[n], cu[n + 1]
        yn, csn = oracle.conv1d(x[s:e], w, conv_state=cs[n:n + 1], n_l2_heads=1, head_dim=8,
                                stage_bf16=True)
        np.testing.assert_array_equal(y[s:e], yn)
        np.testing.assert_array_equal(cso[n], csn[0])
    np.testing.assert_array_equal(cso[1], cs[1])


# ---------------------------------------------------------------- gated norm

def test_gated_rmsnorm_matches_torch_fp64():
    r = RNG(30)
    rows, Hv, dv = 7, 5, 32
    o = r.standard_normal((rows, Hv, dv))
    z = r.standard_normal((rows, Hv, dv))
    w = 1 + 0.02 * r.standard_normal(dv)
    out = oracle.gated_rmsnorm(o, z, w, eps=1e-6)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(o), (dv,), torch.from_numpy(w), eps=1e-6)
    ref = (ref * torch.nn.functional.silu(torch.from_numpy(z))).numpy()
    np.testing.assert_allclose(out, ref, rtol=1e-13, atol=1e-15)


def test_gated_rmsnorm_constant_closed_form():
    rows, Hv, dv = 3, 2, 16
    c = -0.7
    o = np.full((rows, Hv, dv), c)
    z = np.random.default_rng(31).standard_normal((rows, Hv, dv))
    w = np.linspace(0.5, 1.5, dv)
    out = oracle.gated_rmsnorm(o, z, w, eps=1e-6)
    ref = w * c / np.sqrt(c * c + 1e-6) * z / (1 + np.exp(-z))
    np.testing.assert_allclose(out, ref, rtol=1e-13)


# ---------------------------------------------------------------- bf16 grid

def test_round_bf16_matches_torch_cast():
    """For fp32-representable inputs the fp64 -> bf16 rounding equals torch's
    fp32 -> bf16 cast (round to nearest, ties to even), including ties,
    subnormals and overflow."""
    r = RNG(40)
    x32 = (r.standard_normal(20000) * np.exp(r.uniform(-30, 30, 20000))).astype(np.float32)
    ties = (np.arange(1, 2000, dtype=np.uint32) << 16 | 0x8000).view(np.float32)
    sub = np.array([1e-39, -3e-40, 9.2e-41, 1.17e-38, 3.3e38, 3.5e38, -3.4e38], dtype=np.float32)
    x32 = np.concatenate([x32, ties, sub])
    got = oracle.round_bf16(x32.astype(np.float64))
    ref = torch.from_numpy(x32).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(got, ref)


# ----------------------------------------------------------------- chunk map

@pytest.mark.parametrize("lens", [[5], [0], [64, 64], [65, 0, 1, 128, 63, 0, 200], [7, 7, 3, 7],
                                  [300, 1, 64, 65, 129, 0, 0, 2]])
def test_chunk_map_brute_force(lens):
    """The varlen chunk map against a direct enumeration: every sequence cut into
    64-token pieces from its own start (the last one partial)."""
    lens = np.asarray(lens, dtype=np.int64)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    off, tab = oracle.chunk_map(cu)
    rows, offs = [], [0]
    for n, L in enumerate(lens):
        start = int(cu[n])
        for a in range(0, int(L), 64):
            rows.append([n, start + a, min(64, int(L) - a)])
        offs.append(len(rows))
    assert off.tolist() == offs
    assert tab.tolist() == rows
    # each token belongs to exactly one chunk
    covered = np.zeros(int(cu[-1]), dtype=np.int32)
    for _, t0, ln in rows:
        covered[t0:t0 + ln] += 1
    assert np.all(covered == 1)


# ----------------------------------------------------------------- gate prep

_A_LOG = np.log(np.array([0.5, 1.0, 2.0, 4.0, 8.0, 16.0]))
_DT = np.array([0.0, 0.5, -1.0, 2.0, -3.0, 1.0])


def test_gate_prep_closed_forms():
    """a + dt_bias = 0 makes the step softplus(0) = ln 2, so g = -A ln 2 per head;
    b = 0 gives beta = 1/2."""
    Hv = _A_LOG.size
    a = np.tile(-_DT, (3, 1))
    g, beta = oracle.gate_prep(a, np.zeros((3, Hv)), _A_LOG, _DT)
    np.testing.assert_allclose(g, np.tile(-np.exp(_A_LOG) * np.log(2.0), (3, 1)), rtol=1e-15)
    assert np.all(beta == 0.5)


def test_gate_prep_power_form_and_logit():
    """The decay exp(g) equals (1 + e^(a + dt_bias))^(-exp(A_log)) -- the same
    value written as a power -- head by head (a wrong head index, sign or
    exponent fails it); beta / (1 - beta) = e^b; g < 0 and 0 < beta < 1."""
    r = np.random.default_rng(41)
    Hv = _A_LOG.size
    a = r.normal(0.0, 2.0, (64, Hv))
    b = r.normal(0.0, 3.0, (64, Hv))
    g, beta = oracle.gate_prep(a, b, _A_LOG, _DT)
    alpha = (1.0 + np.exp(a + _DT)) ** (-np.exp(_A_LOG))
    np.testing.assert_allclose(np.exp(g), alpha, rtol=1e-12)
    np.testing.assert_allclose(beta / (1.0 - beta), np.exp(b), rtol=1e-12)
    assert np.all(g < 0) and np.all((beta > 0) & (beta < 1))


def test_gate_prep_softplus_reflection_and_tails():
    """softplus(x) - softplus(-x) = x; softplus(x) = x to rounding for large x
    (no overflow at x = 800) and e^x for very negative x."""
    x = np.array([[-800.0, -50.0, -3.0, 0.25, 7.0, 50.0, 800.0]])
    Hv = x.shape[1]
    zero = np.zeros(Hv)
    gp, _ = oracle.gate_prep(x, np.zeros_like(x), zero, zero)    # A = 1: g = -softplus(x)
    gm, _ = oracle.gate_prep(-x, np.zeros_like(x), zero, zero)
    np.testing.assert_allclose(gm - gp, x, rtol=1e-15, atol=1e-15)
    sp = -gp[0]
    assert sp[-1] == 800.0 and abs(sp[-2] - 50.0) <= 1e-14
    np.testing.assert_allclose(sp[1], np.exp(-50.0), rtol=1e-14)
    assert sp[0] == 0.0 or sp[0] < 1e-300


# ----------------------------------------------------------------- backward

def _bwd_case(seed, T, Hk, Hv, dk, dv, n_states):
    r = np.random.default_rng(seed)
    k = r.standard_normal((T, Hk, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    return dict(q=r.standard_normal((T, Hk, dk)), k=k, v=r.standard_normal((T, Hv, dv)),
                g=-r.uniform(0.0, 0.5, (T, Hv)), beta=r.uniform(0.1, 0.9, (T, Hv)),
                h0=0.3 * r.standard_normal((n_states, Hv, dv, dk))), \
        r.standard_normal((T, Hv, dv)), r.standard_normal((n_states, Hv, dv, dk))


def test_backward_central_differences():
    """Every element of every input: the oracle's gradient of
    L = sum(d_o * o) + sum(dhT * hT) against a central finite difference of L
    computed with the forward oracle (varlen, two value heads on one key
    head, scale != 1)."""
    cu = np.array([0, 4, 6], dtype=np.int32)
    x, d_o, dhT = _bwd_case(51, 6, 1, 2, 3, 2, 2)

    def loss(x):
        o, hT = oracle.recurrence(x["q"], x["k"], x["v"], x["g"], x["beta"], x["h0"],
                                  cu_seqlens=cu, n_seqs=2, scale=0.7)
        return float(np.sum(d_o * o) + np.sum(dhT * hT))

    grad = oracle.backward(x["q"], x["k"], x["v"], x["g"], x["beta"], d_o, h0=x["h0"], dhT=dhT,
                           cu_seqlens=cu, scale=0.7)
    names = dict(q="dq", k="dk", v="dv", g="dg", beta="dbeta", h0="dh0")
    eps = 1e-6
    for name, gname in names.items():
        fd = np.zeros_like(x[name])
        for idx in np.ndindex(x[name].shape):
            xp = {kk: vv.copy() for kk, vv in x.items()}
            xm = {kk: vv.copy() for kk, vv in x.items()}
            xp[name][idx] += eps
            xm[name][idx] -= eps
            fd[idx] = (loss(xp) - loss(xm)) / (2 * eps)
        np.testing.assert_allclose(grad[gname], fd, rtol=1e-6, atol=1e-7, err_msg=gname)


def test_backward_matches_torch_autograd_fp64():
    """The hand-derived reverse recurrence against torch autograd through the
    forward definition in fp64 (equal-length sequences, two value heads per
    key head, dv != dk)."""
    T, Hk, Hv, dk, dv, N = 12, 2, 4, 5, 3, 2
    x, d_o, dhT = _bwd_case(52, T, Hk, Hv, dk, dv, N)
    grad = oracle.backward(x["q"], x["k"], x["v"], x["g"], x["beta"], d_o, h0=x["h0"], dhT=dhT,
                           n_seqs=N, scale=1.3)
    tx = {kk: torch.tensor(vv, dtype=torch.float64, requires_grad=True) for kk, vv in x.items()}
    L = T // N
    loss = torch.zeros((), dtype=torch.float64)
    for n in range(N):
        for h in range(Hv):
            kh = h // (Hv // Hk)
            S = tx["h0"][n, h]
            for t in range(n * L, (n + 1) * L):
                kt, qt = tx["k"][t, kh], tx["q"][t, kh]
                a, b = torch.exp(tx["g"][t, h]), tx["beta"][t, h]
                S = a * S + torch.outer(b * (tx["v"][t, h] - a * (S @ kt)), kt)
                loss = loss + torch.dot(torch.as_tensor(d_o[t, h]), 1.3 * (S @ qt))
            loss = loss + torch.sum(torch.as_tensor(dhT[n, h]) * S)
    loss.backward()
    for name, gname in dict(q="dq", k="dk", v="dv", g="dg", beta="dbeta", h0="dh0").items():
        np.testing.assert_allclose(grad[gname], tx[name].grad.numpy(), rtol=1e-10, atol=1e-12,
                                   err_msg=gname)
