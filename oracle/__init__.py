"""fp64 CPU oracle for the gated-delta-rule token mixer.

TEST INFRASTRUCTURE ONLY: imported by tests/, by the smoke check and by the
benchmark's CPU-baseline leg, never by the product path.  It shares no code with
the HIP library: the arithmetic lives in ``gdn_oracle.c`` (plain C, fp64, libm),
and this module only marshals numpy arrays into it.

Inputs given as bf16 bit patterns (uint16) are widened exactly to fp64 here;
fp32 inputs are widened exactly.  All results come back as fp64 arrays.

Functions (each documented in gdn_oracle.c with its source):
  recurrence(...)     sequential rule over packed sequences
  decode(...)         one token per sequence, state in place
  conv1d(...)         causal depthwise conv k=4 + SiLU + per-head L2
  gated_rmsnorm(...)  (o / rms(o)) * w * silu(z)
  round_bf16(...)     round-to-nearest-even onto the bfloat16 grid
  chunk_map(...)      varlen chunk offsets / chunk table (integer bookkeeping)
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

_dp = ctypes.POINTER(ctypes.c_double)
_ip = ctypes.POINTER(ctypes.c_int32)


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _b
        _b.build()
    lib = ctypes.CDLL(_LIB_PATH)
    lib.oracle_gdn_recurrence.argtypes = [_dp, _dp, _dp, _dp, _dp, _dp, _dp, _dp, _ip,
                                          ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                          ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                          ctypes.c_double, ctypes.c_int32]
    lib.oracle_gdn_recurrence.restype = ctypes.c_int
    lib.oracle_gdn_decode.argtypes = [_dp, _dp, _dp, _dp, _dp, _dp, _ip, ctypes.c_int32, _dp,
                                      ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                      ctypes.c_int32, ctypes.c_int32, ctypes.c_double,
                                      ctypes.c_int32]
    lib.oracle_gdn_decode.restype = ctypes.c_int
    lib.oracle_conv1d.argtypes = [_dp, _dp, _dp, _dp, _dp, _dp, _ip, ctypes.c_int32,
                                  ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                  ctypes.c_int32, ctypes.c_double, ctypes.c_int32,
                                  ctypes.c_int32]
    lib.oracle_conv1d.restype = ctypes.c_int
    lib.oracle_gated_rmsnorm.argtypes = [_dp, _dp, _dp, _dp, ctypes.c_int64, ctypes.c_int32,
                                         ctypes.c_int32, ctypes.c_double, ctypes.c_int32,
                                         ctypes.c_int32]
    lib.oracle_gated_rmsnorm.restype = ctypes.c_int
    lib.oracle_chunk_map.argtypes = [_ip, ctypes.c_int32, ctypes.c_int32, _ip, _ip]
    lib.oracle_chunk_map.restype = ctypes.c_int
    lib.oracle_gate_prep.argtypes = [_dp, ctypes.c_int64, _dp, ctypes.c_int64, _dp, _dp, _dp, _dp,
                                     ctypes.c_int64, ctypes.c_int32]
    lib.oracle_gate_prep.restype = ctypes.c_int
    lib.oracle_gdn_backward.argtypes = [_dp, _dp, _dp, _dp, _dp, _dp, _dp, _dp, _ip,
                                        ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                        ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                        ctypes.c_double, _dp, _dp, _dp, _dp, _dp, _dp,
                                        ctypes.c_int32]
    lib.oracle_gdn_backward.restype = ctypes.c_int
    lib.oracle_round_bf16_array.argtypes = [_dp, _dp, ctypes.c_int64]
    lib.oracle_round_bf16_array.restype = None
    _lib = lib
    return lib


def _f64(a):
    """Exact widening to a C-contiguous fp64 array. uint16 is read as bf16 bits."""
    if a is None:
        return None
    a = np.asarray(a)
    if a.dtype == np.uint16:
        a = (a.astype(np.uint32) << 16).view(np.float32)
    return np.ascontiguousarray(a, dtype=np.float64)


def _ptr(a, ty=_dp):
    return None if a is None else a.ctypes.data_as(ty)


def _i32(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.int32)


def _threads(n):
    if n is not None:
        return int(n)
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def recurrence(q, k, v, g, beta, h0=None, cu_seqlens=None, n_seqs=1, scale=1.0,
               n_threads=None):
    """o, final_state of the rule over packed sequences.

    q, k [T, Hk, dk]; v [T, Hv, dv]; g, beta [T, Hv]; h0 [N, Hv, dv, dk] or None.
    Returns (o [T, Hv, dv], hT [N, Hv, dv, dk]) in fp64.
    """
    lib = _load()
    q, k, v, g, beta, h0 = map(_f64, (q, k, v, g, beta, h0))
    T, Hk, dk = q.shape
    Hv, dv = v.shape[1], v.shape[2]
    cu = _i32(cu_seqlens)
    if cu is not None:
        n_seqs = cu.shape[0] - 1
    o = np.zeros((T, Hv, dv))
    hT = np.zeros((n_seqs, Hv, dv, dk))
    rc = lib.oracle_gdn_recurrence(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(h0),
                                   _ptr(o), _ptr(hT), _ptr(cu, _ip), n_seqs, T, Hk, Hv, dk, dv,
                                   float(scale), _threads(n_threads))
    if rc:
        raise ValueError(f"oracle_gdn_recurrence failed ({rc})")
    return o, hT


def backward(q, k, v, g, beta, d_o, h0=None, dhT=None, cu_seqlens=None, n_seqs=1, scale=1.0,
             n_threads=None):
    """Gradients of L = sum(d_o * o) + sum(dhT * hT) of the recurrence.

    Shapes as recurrence(); d_o like o, dhT like the final state (or None).
    Returns dict(dq, dk, dv, dg, dbeta, dh0) in fp64.
    """
    lib = _load()
    q, k, v, g, beta, d_o, h0, dhT = map(_f64, (q, k, v, g, beta, d_o, h0, dhT))
    T, Hk, dk = q.shape
    Hv, dv = v.shape[1], v.shape[2]
    cu = _i32(cu_seqlens)
    if cu is not None:
        n_seqs = cu.shape[0] - 1
    out = dict(dq=np.zeros((T, Hk, dk)), dk=np.zeros((T, Hk, dk)), dv=np.zeros((T, Hv, dv)),
               dg=np.zeros((T, Hv)), dbeta=np.zeros((T, Hv)), dh0=np.zeros((n_seqs, Hv, dv, dk)))
    rc = lib.oracle_gdn_backward(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(h0),
                                 _ptr(d_o), _ptr(dhT), _ptr(cu, _ip), n_seqs, T, Hk, Hv, dk, dv,
                                 float(scale), _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]),
                                 _ptr(out["dg"]), _ptr(out["dbeta"]), _ptr(out["dh0"]),
                                 _threads(n_threads))
    if rc:
        raise ValueError(f"oracle_gdn_backward failed ({rc})")
    return out


def decode(q, k, v, g, beta, state, state_slot=None, scale=1.0, n_threads=None):
    """One decode step. Returns (o [N, Hv, dv], new_state) without touching `state`."""
    lib = _load()
    q, k, v, g, beta = map(_f64, (q, k, v, g, beta))
    st = _f64(state).copy()
    N, Hk, dk = q.shape
    Hv, dv = v.shape[1], v.shape[2]
    slots = _i32(state_slot)
    o = np.zeros((N, Hv, dv))
    rc = lib.oracle_gdn_decode(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(st),
                               _ptr(slots, _ip), st.shape[0], _ptr(o), N, Hk, Hv, dk, dv,
                               float(scale), _threads(n_threads))
    if rc:
        raise ValueError(f"oracle_gdn_decode failed ({rc})")
    return o, st


def conv1d(x, w, bias=None, conv_state=None, cu_seqlens=None, n_seqs=1, n_l2_heads=0,
           head_dim=128, l2_eps=1e-6, stage_bf16=True, n_threads=None):
    """Causal depthwise conv k=4 + SiLU + per-head L2 on the first n_l2_heads heads.

    x [T, C]; w [C, 4]; conv_state [N, C, 3] or None. Returns (y [T, C], new_state [N, C, 3]).
    """
    lib = _load()
    x, w, bias, cs = map(_f64, (x, w, bias, conv_state))
    T, C = x.shape
    cu = _i32(cu_seqlens)
    if cu is not None:
        n_seqs = cu.shape[0] - 1
    y = np.zeros((T, C))
    cs_out = np.zeros((n_seqs, C, 3))
    rc = lib.oracle_conv1d(_ptr(x), _ptr(w), _ptr(bias), _ptr(cs), _ptr(y), _ptr(cs_out),
                           _ptr(cu, _ip), n_seqs, T, C, n_l2_heads, head_dim, float(l2_eps),
                           1 if stage_bf16 else 0, _threads(n_threads))
    if rc:
        raise ValueError(f"oracle_conv1d failed ({rc})")
    return y, cs_out


def gated_rmsnorm(o, z, w, eps=1e-6, stage_bf16=False, n_threads=None):
    """(o / sqrt(mean(o^2) + eps)) * w * silu(z) per (row, head). o, z [rows, Hv, dv]."""
    lib = _load()
    o, z, w = map(_f64, (o, z, w))
    rows, Hv, dv = o.shape
    z = z.reshape(rows, Hv, dv)
    out = np.zeros_like(o)
    rc = lib.oracle_gated_rmsnorm(_ptr(o), _ptr(z), _ptr(w), _ptr(out), rows, Hv, dv,
                                  float(eps), 1 if stage_bf16 else 0, _threads(n_threads))
    if rc:
        raise ValueError(f"oracle_gated_rmsnorm failed ({rc})")
    return out


def gate_prep(a, b, A_log, dt_bias):
    """g = -exp(A_log) * softplus(a + dt_bias), beta = sigmoid(b) per (token, value head).

    a, b [T, Hv] (bf16 bits as uint16, or values); A_log, dt_bias [Hv]. Returns (g, beta) fp64.
    """
    lib = _load()
    a, b, A_log, dt_bias = map(_f64, (a, b, A_log, dt_bias))
    T, Hv = a.shape
    g = np.zeros((T, Hv))
    beta = np.zeros((T, Hv))
    rc = lib.oracle_gate_prep(_ptr(a), Hv, _ptr(b), Hv, _ptr(A_log), _ptr(dt_bias), _ptr(g),
                              _ptr(beta), T, Hv)
    if rc:
        raise ValueError(f"oracle_gate_prep failed ({rc})")
    return g, beta


def round_bf16(x):
    """Round fp64 values to the nearest bf16 value (ties to even); returns fp64."""
    lib = _load()
    x = np.ascontiguousarray(x, dtype=np.float64)
    y = np.empty_like(x)
    lib.oracle_round_bf16_array(_ptr(x), _ptr(y), x.size)
    return y


def chunk_map(cu_seqlens, chunk=64):
    """(chunk_off [N+1], tab [n_chunks, 3]) as int32 numpy arrays."""
    lib = _load()
    cu = _i32(cu_seqlens)
    N = cu.shape[0] - 1
    lens = np.diff(cu.astype(np.int64))
    n_chunks = int(np.sum((lens + chunk - 1) // chunk))
    off = np.zeros(N + 1, dtype=np.int32)
    tab = np.zeros((max(n_chunks, 1), 3), dtype=np.int32)
    rc = lib.oracle_chunk_map(_ptr(cu, _ip), N, chunk, _ptr(off, _ip), _ptr(tab, _ip))
    if rc:
        raise ValueError(f"oracle_chunk_map failed ({rc})")
    return off, tab[:n_chunks]
