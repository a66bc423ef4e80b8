"""Python binding of libgdn (include/gdn.h): argument marshalling only.

Each function takes torch tensors on the GPU, checks dtype, device and layout,
passes raw device pointers and the current HIP stream to the C ABI entry point
of the same name, and raises GdnError on a non-zero status.  Every step of the
computation runs in the HIP kernels; there is no CPU fallback, and a missing
libgdn.so raises at the first call.
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import Optional, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgdn.so")
HEADER = os.path.join(os.path.dirname(_HERE), "include", "gdn.h")

_c = ctypes
_vp, _i32, _i64, _f32, _sz = _c.c_void_p, _c.c_int32, _c.c_int64, _c.c_float, _c.c_size_t

_SIGS = {
    "gdn_status_string": (_c.c_char_p, [_i32]),
    "gdn_last_error": (_c.c_char_p, []),
    "gdn_abi_version": (_i32, []),
    "gdn_conv1d_fwd": (_i32, [_vp, _i64, _vp, _vp, _vp, _i64, _vp, _vp, _i32, _i32, _i32, _i32,
                              _i32, _f32, _vp]),
    "gdn_chunk_fwd_workspace_bytes": (_sz, [_i32, _i32, _i32, _i32, _i32]),
    "gdn_chunk_fwd": (_i32, [_vp, _i64, _vp, _i64, _vp, _i64, _vp, _vp, _vp, _vp, _vp, _vp,
                             _i32, _i32, _i32, _i32, _i32, _i32, _f32, _vp, _sz, _vp]),
    "gdn_chunk_fwd_noalloc": (_i32, [_vp, _i64, _vp, _i64, _vp, _i64, _vp, _vp, _vp, _vp, _vp,
                                     _vp, _i32, _i32, _i32, _i32, _i32, _i32, _f32, _vp]),
    "gdn_chunk_fwd_bf16o": (_i32, [_vp, _i64, _vp, _i64, _vp, _i64, _vp, _vp, _vp, _vp, _vp, _vp,
                                   _i32, _i32, _i32, _i32, _i32, _i32, _f32, _vp, _sz, _vp]),
    "gdn_chunk_fwd_pooled": (_i32, [_vp, _i64, _vp, _i64, _vp, _i64, _vp, _vp, _vp, _i32, _vp,
                                    _vp, _i32, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _f32,
                                    _vp, _sz, _vp]),
    "gdn_chunk_fwd_gated": (_i32, [_vp, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _vp,
                                   _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32,
                                   _f32, _vp, _sz, _vp]),
    "gdn_mixer_fwd_workspace_bytes": (_sz, [_i32, _i32, _i32, _i32, _i32, _i32]),
    "gdn_mixer_fwd": (_i32, [_vp, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _vp, _i64, _vp, _vp,
                             _vp, _i64, _vp, _vp, _i32, _vp, _vp, _vp, _i32, _vp, _i32, _i32,
                             _i32, _i32, _i32, _f32, _f32, _f32, _vp, _sz, _vp]),
    "gdn_chunk_map": (_i32, [_vp, _i32, _i32, _vp, _vp, _vp, _vp]),
    "gdn_decode_step": (_i32, [_vp, _i64, _vp, _i64, _vp, _i64, _vp, _vp, _vp, _vp, _i32, _vp,
                               _i32, _i32, _i32, _i32, _i32, _f32, _vp]),
    "gdn_decode_tokens": (_i32, [_vp, _i64, _vp, _i64, _vp, _i64, _vp, _vp, _vp, _vp, _i32, _vp,
                                 _i32, _i32, _i32, _i32, _i32, _i32, _f32, _vp]),
    "gdn_decode_mixer_step": (_i32, [_vp, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _vp, _i64, _vp,
                                     _vp, _vp, _i64, _vp, _vp, _vp, _i32, _vp, _i32, _i32, _i32,
                                     _i32, _i32, _f32, _f32, _f32, _vp]),
    "gdn_gated_rmsnorm": (_i32, [_vp, _vp, _i64, _vp, _vp, _i32, _i64, _i32, _i32, _f32, _vp]),
    "gdn_validate_cu_seqlens": (_i32, [_vp, _i32, _i32, _vp]),
    "gdn_calib_mfma_loop_flops": (_c.c_double, [_i32, _i32]),
    "gdn_calib_mfma_loop": (_i32, [_i32, _i32, _vp, _vp]),
    "gdn_calib_stream_inplace": (_i32, [_vp, _i64, _i32, _vp]),
    "gdn_backward_workspace_bytes": (_sz, [_i32, _i32, _i32]),
    "gdn_backward": (_i32, [_vp, _i64, _vp, _i64, _vp, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _i32,
                            _i32, _i32, _i32, _i32, _i32, _f32, _vp, _vp, _vp, _vp, _vp, _vp,
                            _vp, _sz, _vp]),
}

_lib_handle = None


class GdnError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        super().__init__(f"{where}: status {status} ({detail})")
        self.status = status


def lib() -> ctypes.CDLL:
    """The loaded libgdn.so with prototypes set (raises if it is not built)."""
    global _lib_handle
    if _lib_handle is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build() "
                               "(hipcc, gfx950) first")
        h = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(h, name)
            fn.restype = res
            fn.argtypes = args
        _lib_handle = h
    return _lib_handle


def header_functions() -> list:
    """Names of the functions declared in include/gdn.h."""
    txt = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[\w\s\*]+?\b(gdn_\w+)\s*\(", txt, re.M)))


def _check(status: int, where: str):
    if status != 0:
        h = lib()
        raise GdnError(status, where, f"{h.gdn_status_string(status).decode()}: "
                                      f"{h.gdn_last_error().decode()}")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _stream():
    return torch.cuda.current_stream().cuda_stream


def _need(t: torch.Tensor, name: str, dtype, dims: int):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != dims:
        raise ValueError(f"{name} must have {dims} dims, got {tuple(t.shape)}")


def _inner_contig(t: torch.Tensor, name: str):
    # all dims but the first contiguous (row stride free, multiple of 8)
    exp = 1
    for d in range(t.dim() - 1, 0, -1):
        if t.stride(d) != exp:
            raise ValueError(f"{name}: inner dims must be contiguous")
        exp *= t.shape[d]


def gdn_conv1d_fwd(x: torch.Tensor, w: torch.Tensor, *, y: Optional[torch.Tensor] = None,
                   bias: Optional[torch.Tensor] = None, conv_state: Optional[torch.Tensor] = None,
                   cu_seqlens: Optional[torch.Tensor] = None, n_seqs: Optional[int] = None,
                   n_l2_heads: int = 32, head_dim: int = 128, l2_eps: float = 1e-6) -> torch.Tensor:
    """x [T, C] bf16, w [C, 4] bf16 -> y [T, C] bf16; conv_state [N, C, 3] updated in place."""
    _need(x, "x", torch.bfloat16, 2)
    _need(w, "w", torch.bfloat16, 2)
    T, C = x.shape
    _inner_contig(x, "x")
    w = w.contiguous()
    if y is None:
        y = torch.empty((T, C), dtype=torch.bfloat16, device=x.device)
    _need(y, "y", torch.bfloat16, 2)
    _inner_contig(y, "y")
    if bias is not None:
        _need(bias, "bias", torch.float32, 1)
    if conv_state is not None:
        _need(conv_state, "conv_state", torch.bfloat16, 3)
        if not conv_state.is_contiguous():
            raise ValueError("conv_state must be contiguous")
    if cu_seqlens is not None:
        _need(cu_seqlens, "cu_seqlens", torch.int32, 1)
        n_seqs = cu_seqlens.shape[0] - 1
    elif n_seqs is None:
        n_seqs = conv_state.shape[0] if conv_state is not None else 1
    st = lib().gdn_conv1d_fwd(_ptr(x), x.stride(0), _ptr(w), _ptr(bias), _ptr(y), y.stride(0),
                              _ptr(conv_state), _ptr(cu_seqlens), n_seqs, T, C, n_l2_heads,
                              head_dim, l2_eps, _stream())
    _check(st, "gdn_conv1d_fwd")
    return y


def gdn_chunk_fwd_workspace_bytes(n_seqs: int, T_total: int, Hk: int, Hv: int, d: int = 128) -> int:
    return int(lib().gdn_chunk_fwd_workspace_bytes(n_seqs, T_total, Hk, Hv, d))


def gdn_chunk_map(cu_seqlens: torch.Tensor, T_total: int):
    """(order [N], chunk_off [N+1], chunk_tab [n_chunks_max, 3]) int32 on the GPU."""
    _need(cu_seqlens, "cu_seqlens", torch.int32, 1)
    N = cu_seqlens.shape[0] - 1
    dev = cu_seqlens.device
    order = torch.empty(max(N, 1), dtype=torch.int32, device=dev)
    off = torch.empty(N + 1, dtype=torch.int32, device=dev)
    tab = torch.empty((T_total // 64 + N, 3), dtype=torch.int32, device=dev)
    st = lib().gdn_chunk_map(_ptr(cu_seqlens), N, T_total, _ptr(order), _ptr(off), _ptr(tab),
                             _stream())
    _check(st, "gdn_chunk_map")
    return order[:N], off, tab


def gdn_chunk_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
                  beta: torch.Tensor, *, initial_state: Optional[torch.Tensor] = None,
                  final_state: Optional[torch.Tensor] = None, output_final_state: bool = True,
                  cu_seqlens: Optional[torch.Tensor] = None, n_seqs: Optional[int] = None,
                  scale: float = 1.0, o: Optional[torch.Tensor] = None,
                  workspace: Optional[torch.Tensor] = None,
                  o_bf16: bool = False) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Chunked prefill. q, k [T, Hk, 128], v [T, Hv, 128] bf16; g, beta [T, Hv] fp32.

    Returns (o [T, Hv, 128] fp32 -- bf16 with o_bf16 or a bf16 `o` --,
    final_state [N, Hv, 128, 128] fp32 or None).
    """
    for t, nm in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, nm, torch.bfloat16, 3)
        _inner_contig(t, nm)
    _need(g, "g", torch.float32, 2)
    _need(beta, "beta", torch.float32, 2)
    if not (g.is_contiguous() and beta.is_contiguous()):
        raise ValueError("g and beta must be contiguous")
    T, Hk, dk = q.shape
    Hv, dv = v.shape[1], v.shape[2]
    if cu_seqlens is not None:
        _need(cu_seqlens, "cu_seqlens", torch.int32, 1)
        n_seqs = cu_seqlens.shape[0] - 1
    elif n_seqs is None:
        n_seqs = initial_state.shape[0] if initial_state is not None else 1
    if o is not None and o.dtype == torch.bfloat16:
        o_bf16 = True
    odt = torch.bfloat16 if o_bf16 else torch.float32
    if o is None:
        o = torch.empty((T, Hv, dv), dtype=odt, device=q.device)
    _need(o, "o", odt, 3)
    if not o.is_contiguous():
        raise ValueError("o must be contiguous")
    if initial_state is not None:
        _need(initial_state, "initial_state", torch.float32, 4)
        if not initial_state.is_contiguous():
            raise ValueError("initial_state must be contiguous")
    if final_state is None and output_final_state:
        final_state = torch.empty((n_seqs, Hv, dv, dk), dtype=torch.float32, device=q.device)
    if final_state is not None:
        _need(final_state, "final_state", torch.float32, 4)
        if not final_state.is_contiguous():
            raise ValueError("final_state must be contiguous")
    ws_bytes = 0
    if n_seqs > 0:
        if workspace is None:
            workspace = torch.empty(gdn_chunk_fwd_workspace_bytes(n_seqs, T, Hk, Hv, dk),
                                    dtype=torch.uint8, device=q.device)
        ws_bytes = workspace.numel()
    fn = lib().gdn_chunk_fwd_bf16o if o_bf16 else lib().gdn_chunk_fwd
    st = fn(_ptr(q), q.stride(0), _ptr(k), k.stride(0), _ptr(v), v.stride(0),
            _ptr(g), _ptr(beta), _ptr(o), _ptr(initial_state), _ptr(final_state),
            _ptr(cu_seqlens), n_seqs, T, Hk, Hv, dk, dv, scale, _ptr(workspace),
            ws_bytes, _stream())
    _check(st, "gdn_chunk_fwd_bf16o" if o_bf16 else "gdn_chunk_fwd")
    return o, final_state


def gdn_chunk_fwd_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
                          beta: torch.Tensor, o: torch.Tensor, *,
                          initial_state: Optional[torch.Tensor] = None,
                          final_state: Optional[torch.Tensor] = None,
                          cu_seqlens: Optional[torch.Tensor] = None, n_seqs: Optional[int] = None,
                          scale: float = 1.0) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """gdn_chunk_fwd into caller-provided o (fp32) and final_state, with the
    library's static device workspace instead of a workspace argument (nothing
    is allocated, here or in the library).  Returns (o, final_state)."""
    for t, nm in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, nm, torch.bfloat16, 3)
        _inner_contig(t, nm)
    _need(g, "g", torch.float32, 2)
    _need(beta, "beta", torch.float32, 2)
    _need(o, "o", torch.float32, 3)
    if not (g.is_contiguous() and beta.is_contiguous() and o.is_contiguous()):
        raise ValueError("g, beta and o must be contiguous")
    T, Hk, dk = q.shape
    Hv, dv = v.shape[1], v.shape[2]
    if cu_seqlens is not None:
        _need(cu_seqlens, "cu_seqlens", torch.int32, 1)
        n_seqs = cu_seqlens.shape[0] - 1
    elif n_seqs is None:
        n_seqs = initial_state.shape[0] if initial_state is not None else 1
    for t, nm in ((initial_state, "initial_state"), (final_state, "final_state")):
        if t is not None:
            _need(t, nm, torch.float32, 4)
            if not t.is_contiguous():
                raise ValueError(f"{nm} must be contiguous")
    st = lib().gdn_chunk_fwd_noalloc(_ptr(q), q.stride(0), _ptr(k), k.stride(0), _ptr(v),
                                     v.stride(0), _ptr(g), _ptr(beta), _ptr(o),
                                     _ptr(initial_state), _ptr(final_state), _ptr(cu_seqlens),
                                     n_seqs, T, Hk, Hv, dk, dv, scale, _stream())
    _check(st, "gdn_chunk_fwd_noalloc")
    return o, final_state


def _qkv_checks(q, k, v):
    for t, nm in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, nm, torch.bfloat16, 3)
        _inner_contig(t, nm)


def _workspace(workspace, n_seqs, T, Hk, Hv, dk, device):
    if n_seqs <= 0:
        return None, 0
    if workspace is None:
        workspace = torch.empty(gdn_chunk_fwd_workspace_bytes(n_seqs, T, Hk, Hv, dk),
                                dtype=torch.uint8, device=device)
    return workspace, workspace.numel()


def gdn_chunk_fwd_pooled(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
                         beta: torch.Tensor, state: torch.Tensor, state_slot: torch.Tensor, *,
                         cu_seqlens: Optional[torch.Tensor] = None, n_seqs: Optional[int] = None,
                         scale: float = 1.0, o: Optional[torch.Tensor] = None,
                         o_bf16: bool = False,
                         workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Chunked prefill continuing from a state pool: sequence n starts from
    state[state_slot[n]] and leaves its final state there (in place).
    state [n_slots, Hv, 128, 128] fp32; returns o [T, Hv, 128]."""
    _qkv_checks(q, k, v)
    _need(g, "g", torch.float32, 2)
    _need(beta, "beta", torch.float32, 2)
    _need(state, "state", torch.float32, 4)
    _need(state_slot, "state_slot", torch.int32, 1)
    if not (g.is_contiguous() and beta.is_contiguous() and state.is_contiguous()):
        raise ValueError("g, beta and state must be contiguous")
    T, Hk, dk = q.shape
    Hv, dv = v.shape[1], v.shape[2]
    if cu_seqlens is not None:
        _need(cu_seqlens, "cu_seqlens", torch.int32, 1)
        n_seqs = cu_seqlens.shape[0] - 1
    elif n_seqs is None:
        n_seqs = state_slot.shape[0]
    if o is not None and o.dtype == torch.bfloat16:
        o_bf16 = True
    odt = torch.bfloat16 if o_bf16 else torch.float32
    if o is None:
        o = torch.empty((T, Hv, dv), dtype=odt, device=q.device)
    _need(o, "o", odt, 3)
    if not o.is_contiguous():
        raise ValueError("o must be contiguous")
    workspace, ws_bytes = _workspace(workspace, n_seqs, T, Hk, Hv, dk, q.device)
    st = lib().gdn_chunk_fwd_pooled(_ptr(q), q.stride(0), _ptr(k), k.stride(0), _ptr(v),
                                    v.stride(0), _ptr(g), _ptr(beta), _ptr(o),
                                    1 if o_bf16 else 0, _ptr(state), _ptr(state_slot),
                                    state.shape[0], _ptr(cu_seqlens), n_seqs, T, Hk, Hv, dk, dv,
                                    scale, _ptr(workspace), ws_bytes, _stream())
    _check(st, "gdn_chunk_fwd_pooled")
    return o


def gdn_chunk_fwd_gated(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, a: torch.Tensor,
                        b: torch.Tensor, A_log: torch.Tensor, dt_bias: torch.Tensor, *,
                        initial_state: Optional[torch.Tensor] = None,
                        final_state: Optional[torch.Tensor] = None,
                        output_final_state: bool = True,
                        cu_seqlens: Optional[torch.Tensor] = None, n_seqs: Optional[int] = None,
                        scale: float = 1.0, o: Optional[torch.Tensor] = None,
                        workspace: Optional[torch.Tensor] = None
                        ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Chunked prefill with the gates formed in the prep kernel from the bf16
    projections a, b [T, Hv] (token stride free, columns contiguous) and
    A_log, dt_bias [Hv] fp32: g = -exp(A_log) softplus(a + dt_bias),
    beta = sigmoid(b).  Returns (o fp32, final_state or None)."""
    _qkv_checks(q, k, v)
    for t, nm in ((a, "a"), (b, "b")):
        _need(t, nm, torch.bfloat16, 2)
        _inner_contig(t, nm)
    for t, nm in ((A_log, "A_log"), (dt_bias, "dt_bias")):
        _need(t, nm, torch.float32, 1)
    T, Hk, dk = q.shape
    Hv, dv = v.shape[1], v.shape[2]
    if cu_seqlens is not None:
        _need(cu_seqlens, "cu_seqlens", torch.int32, 1)
        n_seqs = cu_seqlens.shape[0] - 1
    elif n_seqs is None:
        n_seqs = initial_state.shape[0] if initial_state is not None else 1
    if o is None:
        o = torch.empty((T, Hv, dv), dtype=torch.float32, device=q.device)
    _need(o, "o", torch.float32, 3)
    if not o.is_contiguous():
        raise ValueError("o must be contiguous")
    if initial_state is not None:
        _need(initial_state, "initial_state", torch.float32, 4)
    if final_state is None and output_final_state:
        final_state = torch.empty((n_seqs, Hv, dv, dk), dtype=torch.float32, device=q.device)
    if final_state is not None:
        _need(final_state, "final_state", torch.float32, 4)
    for t, nm in ((initial_state, "initial_state"), (final_state, "final_state")):
        if t is not None and not t.is_contiguous():
            raise ValueError(f"{nm} must be contiguous")
    workspace, ws_bytes = _workspace(workspace, n_seqs, T, Hk, Hv, dk, q.device)
    st = lib().gdn_chunk_fwd_gated(_ptr(q), q.stride(0), _ptr(k), k.stride(0), _ptr(v),
                                   v.stride(0), _ptr(a), a.stride(0), _ptr(b), b.stride(0),
                                   _ptr(A_log), _ptr(dt_bias), _ptr(o), _ptr(initial_state),
                                   _ptr(final_state), _ptr(cu_seqlens), n_seqs, T, Hk, Hv, dk, dv,
                                   scale, _ptr(workspace), ws_bytes, _stream())
    _check(st, "gdn_chunk_fwd_gated")
    return o, final_state


def gdn_mixer_fwd_workspace_bytes(n_seqs: int, T_total: int, Hk: int, Hv: int, d: int = 128,
                                  out_bf16: bool = False) -> int:
    return int(lib().gdn_mixer_fwd_workspace_bytes(n_seqs, T_total, Hk, Hv, d, 1 if out_bf16 else 0))


def gdn_mixer_fwd(x: torch.Tensor, conv_w: torch.Tensor, g: Optional[torch.Tensor],
                  beta: Optional[torch.Tensor], z: torch.Tensor, norm_w: torch.Tensor, *,
                  Hk: int = 16, a: Optional[torch.Tensor] = None, b: Optional[torch.Tensor] = None,
                  A_log: Optional[torch.Tensor] = None, dt_bias: Optional[torch.Tensor] = None,
                  conv_bias: Optional[torch.Tensor] = None,
                  conv_state: Optional[torch.Tensor] = None,
                  initial_state: Optional[torch.Tensor] = None,
                  final_state: Optional[torch.Tensor] = None, output_final_state: bool = True,
                  state_slot: Optional[torch.Tensor] = None,
                  cu_seqlens: Optional[torch.Tensor] = None, n_seqs: Optional[int] = None,
                  scale: float = 1.0, l2_eps: float = 1e-6, norm_eps: float = 1e-6,
                  out_bf16: bool = False, out: Optional[torch.Tensor] = None,
                  workspace: Optional[torch.Tensor] = None
                  ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """The whole mixer over a prefill: x [T, (2 Hk + Hv) 128] bf16 pre-conv rows,
    conv_w [C, 4] bf16, g, beta [T, Hv] fp32, z [T, Hv, 128] bf16, norm_w [128]
    fp32 -> (out [T, Hv, 128] fp32 or bf16, final_state or None); conv_state
    [N, C, 3] bf16 updated in place.  The gates are g, beta [T, Hv] fp32, or
    (g = beta = None) formed from the projections a, b [T, Hv] bf16 with A_log,
    dt_bias [Hv] fp32.  With state_slot [N] int32, initial_state is a pool
    [n_slots, Hv, 128, 128] updated in place (returned as the final state) and
    conv_state a pool [n_slots, C, 3]; sequence n uses row state_slot[n]."""
    _need(x, "x", torch.bfloat16, 2)
    _inner_contig(x, "x")
    _need(conv_w, "conv_w", torch.bfloat16, 2)
    gate_args, Hv = _gate_args(g, beta, a, b, A_log, dt_bias)
    if state_slot is not None:
        _need(state_slot, "state_slot", torch.int32, 1)
        if initial_state is None:
            raise ValueError("state_slot needs the state pool as initial_state")
        final_state = initial_state
    _need(norm_w, "norm_w", torch.float32, 1)
    for t, nm in ((conv_w, "conv_w"), (norm_w, "norm_w")):
        if not t.is_contiguous():
            raise ValueError(f"{nm} must be contiguous")
    z2 = z.reshape(z.shape[0], z.shape[1] * z.shape[2]) if z.dim() == 3 else z
    _need(z2, "z", torch.bfloat16, 2)
    _inner_contig(z2, "z")
    T = x.shape[0]
    d = 128
    if conv_bias is not None:
        _need(conv_bias, "conv_bias", torch.float32, 1)
    if conv_state is not None:
        _need(conv_state, "conv_state", torch.bfloat16, 3)
        if not conv_state.is_contiguous():
            raise ValueError("conv_state must be contiguous")
    if cu_seqlens is not None:
        _need(cu_seqlens, "cu_seqlens", torch.int32, 1)
        n_seqs = cu_seqlens.shape[0] - 1
    elif n_seqs is None:
        if state_slot is not None:
            n_seqs = state_slot.shape[0]
        else:
            n_seqs = initial_state.shape[0] if initial_state is not None else 1
    odt = torch.bfloat16 if out_bf16 else torch.float32
    if out is None:
        out = torch.empty((T, Hv, d), dtype=odt, device=x.device)
    _need(out, "out", odt, 3)
    if not out.is_contiguous():
        raise ValueError("out must be contiguous")
    if initial_state is not None:
        _need(initial_state, "initial_state", torch.float32, 4)
    if final_state is None and output_final_state:
        final_state = torch.empty((n_seqs, Hv, d, d), dtype=torch.float32, device=x.device)
    if final_state is not None:
        _need(final_state, "final_state", torch.float32, 4)
    for t, nm in ((initial_state, "initial_state"), (final_state, "final_state")):
        if t is not None and not t.is_contiguous():
            raise ValueError(f"{nm} must be contiguous")
    ws_bytes = 0
    if n_seqs > 0:
        if workspace is None:
            workspace = torch.empty(gdn_mixer_fwd_workspace_bytes(n_seqs, T, Hk, Hv, d, out_bf16),
                                    dtype=torch.uint8, device=x.device)
        ws_bytes = workspace.numel()
    st = lib().gdn_mixer_fwd(_ptr(x), x.stride(0), _ptr(conv_w), _ptr(conv_bias), _ptr(conv_state),
                             *gate_args, _ptr(z2), z2.stride(0), _ptr(norm_w), _ptr(out),
                             1 if out_bf16 else 0, _ptr(initial_state), _ptr(final_state),
                             _ptr(state_slot),
                             initial_state.shape[0] if state_slot is not None else 0,
                             _ptr(cu_seqlens), n_seqs, T, Hk, Hv, d, scale, l2_eps, norm_eps,
                             _ptr(workspace), ws_bytes, _stream())
    _check(st, "gdn_mixer_fwd")
    return out, final_state


def gdn_decode_step(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
                    beta: torch.Tensor, state: torch.Tensor, *,
                    state_slot: Optional[torch.Tensor] = None, scale: float = 1.0,
                    o: Optional[torch.Tensor] = None) -> torch.Tensor:
    """One token per sequence; state [n_slots, Hv, 128, 128] fp32 updated in place."""
    for t, nm in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, nm, torch.bfloat16, 3)
        _inner_contig(t, nm)
    _need(g, "g", torch.float32, 2)
    _need(beta, "beta", torch.float32, 2)
    _need(state, "state", torch.float32, 4)
    if not (g.is_contiguous() and beta.is_contiguous() and state.is_contiguous()):
        raise ValueError("g, beta and state must be contiguous")
    N, Hk, dk = q.shape
    Hv, dv = v.shape[1], v.shape[2]
    if state_slot is not None:
        _need(state_slot, "state_slot", torch.int32, 1)
    if o is None:
        o = torch.empty((N, Hv, dv), dtype=torch.float32, device=q.device)
    st = lib().gdn_decode_step(_ptr(q), q.stride(0), _ptr(k), k.stride(0), _ptr(v), v.stride(0),
                               _ptr(g), _ptr(beta), _ptr(state), _ptr(state_slot), state.shape[0],
                               _ptr(o), N, Hk, Hv, dk, dv, scale, _stream())
    _check(st, "gdn_decode_step")
    return o


def gdn_decode_tokens(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
                      beta: torch.Tensor, state: torch.Tensor, n_tokens: int, *,
                      state_slot: Optional[torch.Tensor] = None, scale: float = 1.0,
                      o: Optional[torch.Tensor] = None) -> torch.Tensor:
    """n_tokens consecutive tokens per sequence (rows n * n_tokens + t of q, k, v,
    g, beta and o); state [n_slots, Hv, 128, 128] fp32 updated in place."""
    for t, nm in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, nm, torch.bfloat16, 3)
        _inner_contig(t, nm)
    _need(g, "g", torch.float32, 2)
    _need(beta, "beta", torch.float32, 2)
    _need(state, "state", torch.float32, 4)
    if not (g.is_contiguous() and beta.is_contiguous() and state.is_contiguous()):
        raise ValueError("g, beta and state must be contiguous")
    rows, Hk, dk = q.shape
    Hv, dv = v.shape[1], v.shape[2]
    if n_tokens < 1 or rows % n_tokens:
        raise ValueError("rows must be a multiple of n_tokens")
    if state_slot is not None:
        _need(state_slot, "state_slot", torch.int32, 1)
    if o is None:
        o = torch.empty((rows, Hv, dv), dtype=torch.float32, device=q.device)
    st = lib().gdn_decode_tokens(_ptr(q), q.stride(0), _ptr(k), k.stride(0), _ptr(v), v.stride(0),
                                 _ptr(g), _ptr(beta), _ptr(state), _ptr(state_slot), state.shape[0],
                                 _ptr(o), rows // n_tokens, n_tokens, Hk, Hv, dk, dv, scale, _stream())
    _check(st, "gdn_decode_tokens")
    return o


def _gate_args(g, beta, a, b, A_log, dt_bias):
    """(g, beta) given, or the projections (a, b bf16 [rows, Hv], A_log, dt_bias
    fp32 [Hv]): the C arguments g, beta, a, a_stride, b, b_stride, A_log, dt_bias."""
    if g is not None or beta is not None:
        if a is not None or b is not None or A_log is not None or dt_bias is not None:
            raise ValueError("pass either g and beta or a, b, A_log and dt_bias")
        _need(g, "g", torch.float32, 2)
        _need(beta, "beta", torch.float32, 2)
        if not (g.is_contiguous() and beta.is_contiguous()):
            raise ValueError("g and beta must be contiguous")
        return (_ptr(g), _ptr(beta), None, 0, None, 0, None, None), g.shape[1]
    for t, nm in ((a, "a"), (b, "b")):
        _need(t, nm, torch.bfloat16, 2)
        _inner_contig(t, nm)
    for t, nm in ((A_log, "A_log"), (dt_bias, "dt_bias")):
        _need(t, nm, torch.float32, 1)
    return (None, None, _ptr(a), a.stride(0), _ptr(b), b.stride(0), _ptr(A_log),
            _ptr(dt_bias)), a.shape[1]


def gdn_decode_mixer_step(x: torch.Tensor, conv_w: torch.Tensor, conv_state: torch.Tensor,
                          g: Optional[torch.Tensor], beta: Optional[torch.Tensor], z: torch.Tensor,
                          norm_w: torch.Tensor, state: torch.Tensor, *, Hk: int = 16,
                          a: Optional[torch.Tensor] = None, b: Optional[torch.Tensor] = None,
                          A_log: Optional[torch.Tensor] = None,
                          dt_bias: Optional[torch.Tensor] = None,
                          conv_bias: Optional[torch.Tensor] = None,
                          state_slot: Optional[torch.Tensor] = None, scale: float = 1.0,
                          l2_eps: float = 1e-6, norm_eps: float = 1e-6, out_bf16: bool = False,
                          out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """One decode step of the whole mixer (conv + SiLU + L2, the rule, the gated
    RMSNorm) for the new tokens x [N, C] bf16; conv_state [n_slots, C, 3] bf16 and
    state [n_slots, Hv, 128, 128] fp32 updated in place; z [N, Hv, 128] bf16.
    Returns out [N, Hv, 128] (fp32, or bf16 with out_bf16).  The gates are g,
    beta [N, Hv] fp32, or (g = beta = None) formed from the projections a, b
    [N, Hv] bf16 with A_log, dt_bias [Hv] fp32."""
    _need(x, "x", torch.bfloat16, 2)
    _need(conv_w, "conv_w", torch.bfloat16, 2)
    _need(conv_state, "conv_state", torch.bfloat16, 3)
    gate_args, _ = _gate_args(g, beta, a, b, A_log, dt_bias)
    _need(norm_w, "norm_w", torch.float32, 1)
    _need(state, "state", torch.float32, 4)
    for t, nm in ((conv_w, "conv_w"), (conv_state, "conv_state"),
                  (norm_w, "norm_w"), (state, "state")):
        if not t.is_contiguous():
            raise ValueError(f"{nm} must be contiguous")
    if x.stride(1) != 1:
        raise ValueError("x rows must be contiguous")
    z2 = z.reshape(z.shape[0], z.shape[1] * z.shape[2]) if z.dim() == 3 else z
    _need(z2, "z", torch.bfloat16, 2)
    if z2.stride(1) != 1:
        raise ValueError("z rows must be contiguous")
    N = x.shape[0]
    Hv, d = state.shape[1], state.shape[2]
    if conv_bias is not None:
        _need(conv_bias, "conv_bias", torch.float32, 1)
    if state_slot is not None:
        _need(state_slot, "state_slot", torch.int32, 1)
    odt = torch.bfloat16 if out_bf16 else torch.float32
    if out is None:
        out = torch.empty((N, Hv, d), dtype=odt, device=x.device)
    _need(out, "out", odt, 3)
    st = lib().gdn_decode_mixer_step(_ptr(x), x.stride(0), _ptr(conv_w), _ptr(conv_bias),
                                     _ptr(conv_state), *gate_args, _ptr(z2), z2.stride(0),
                                     _ptr(norm_w), _ptr(state), _ptr(state_slot), state.shape[0],
                                     _ptr(out), 1 if out_bf16 else 0, N, Hk, Hv, d, scale, l2_eps,
                                     norm_eps, _stream())
    _check(st, "gdn_decode_mixer_step")
    return out


def gdn_gated_rmsnorm(o: torch.Tensor, z: torch.Tensor, w: torch.Tensor, *,
                      out: Optional[torch.Tensor] = None, out_bf16: bool = False,
                      eps: float = 1e-6) -> torch.Tensor:
    """o [rows, Hv, 128] fp32, z [rows, Hv, 128] bf16, w [128] fp32 -> out."""
    _need(o, "o", torch.float32, 3)
    if not o.is_contiguous():
        raise ValueError("o must be contiguous")
    rows, Hv, dv = o.shape
    if z.dim() == 3:
        _inner_contig(z, "z")
        z2 = z.view(z.shape[0], z.shape[1] * z.shape[2])   # inner dims contiguous: a view
    else:
        z2 = z
    _need(z2, "z", torch.bfloat16, 2)
    _need(w, "w", torch.float32, 1)
    if out is None:
        out = torch.empty((rows, Hv, dv), dtype=torch.bfloat16 if out_bf16 else torch.float32,
                          device=o.device)
    st = lib().gdn_gated_rmsnorm(_ptr(o), _ptr(z2), z2.stride(0), _ptr(w.contiguous()), _ptr(out),
                                 1 if out_bf16 else 0, rows, Hv, dv, eps, _stream())
    _check(st, "gdn_gated_rmsnorm")
    return out


def gdn_validate_cu_seqlens(cu_seqlens: torch.Tensor, T_total: int) -> None:
    """Opt-in host check of cu_seqlens (synchronises the stream)."""
    _need(cu_seqlens, "cu_seqlens", torch.int32, 1)
    st = lib().gdn_validate_cu_seqlens(_ptr(cu_seqlens), cu_seqlens.shape[0] - 1, T_total,
                                       _stream())
    _check(st, "gdn_validate_cu_seqlens")


def gdn_calib_mfma_loop(n_iter: int, n_blocks: int,
                        out: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, float]:
    """The dense fp16 MFMA loop (a measurement aid): returns (out [4 n_blocks]
    fp32, the launch's flops)."""
    if out is None:
        out = torch.empty(4 * max(n_blocks, 0), dtype=torch.float32, device="cuda")
    _need(out, "out", torch.float32, 1)
    if out.numel() < 4 * n_blocks or not out.is_contiguous():
        raise ValueError("out needs 4 * n_blocks contiguous floats")
    h = lib()
    _check(h.gdn_calib_mfma_loop(n_iter, n_blocks, _ptr(out), _stream()), "gdn_calib_mfma_loop")
    return out, float(h.gdn_calib_mfma_loop_flops(n_iter, n_blocks))


def gdn_calib_stream_inplace(buf: torch.Tensor, n_blocks: int) -> int:
    """The streaming pass (a measurement aid): every 16-byte piece of the
    contiguous CUDA tensor buf read and written back unchanged; returns the
    HBM bytes of the launch (twice buf's size)."""
    if not buf.is_cuda or not buf.is_contiguous():
        raise ValueError("buf must be a contiguous CUDA tensor")
    nbytes = buf.numel() * buf.element_size()
    _check(lib().gdn_calib_stream_inplace(_ptr(buf), nbytes, n_blocks, _stream()),
           "gdn_calib_stream_inplace")
    return 2 * nbytes


def gdn_backward_workspace_bytes(n_seqs: int, T_total: int, Hv: int) -> int:
    return int(lib().gdn_backward_workspace_bytes(n_seqs, T_total, Hv))


def gdn_backward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
                 beta: torch.Tensor, grad_o: torch.Tensor, *,
                 initial_state: Optional[torch.Tensor] = None,
                 grad_final_state: Optional[torch.Tensor] = None,
                 cu_seqlens: Optional[torch.Tensor] = None, n_seqs: Optional[int] = None,
                 scale: float = 1.0, grad_initial_state: bool = True,
                 workspace: Optional[torch.Tensor] = None) -> dict:
    """Gradients of sum(grad_o * o) + sum(grad_final_state * S_T) of the rule.

    Inputs as gdn_chunk_fwd; grad_o [T, Hv, 128] fp32, grad_final_state
    [N, Hv, 128, 128] fp32 or None.  Returns a dict of fp32 tensors dq, dk
    [T, Hk, 128], dv [T, Hv, 128], dg, dbeta [T, Hv] and dh0 [N, Hv, 128, 128]
    (None unless grad_initial_state).  The workspace holds the state of every
    4th token, (T / 4 + N) x Hv x 64 KB, and 1-4 KB of partial sums per token
    and value head.
    """
    _qkv_checks(q, k, v)
    _need(g, "g", torch.float32, 2)
    _need(beta, "beta", torch.float32, 2)
    _need(grad_o, "grad_o", torch.float32, 3)
    if not (g.is_contiguous() and beta.is_contiguous() and grad_o.is_contiguous()):
        raise ValueError("g, beta and grad_o must be contiguous")
    T, Hk, dk = q.shape
    Hv, dv = v.shape[1], v.shape[2]
    if cu_seqlens is not None:
        _need(cu_seqlens, "cu_seqlens", torch.int32, 1)
        n_seqs = cu_seqlens.shape[0] - 1
    elif n_seqs is None:
        n_seqs = initial_state.shape[0] if initial_state is not None else 1
    for t, nm in ((initial_state, "initial_state"), (grad_final_state, "grad_final_state")):
        if t is not None:
            _need(t, nm, torch.float32, 4)
            if not t.is_contiguous():
                raise ValueError(f"{nm} must be contiguous")
    dev = q.device
    out = dict(dq=torch.empty((T, Hk, dk), dtype=torch.float32, device=dev),
               dk=torch.empty((T, Hk, dk), dtype=torch.float32, device=dev),
               dv=torch.empty((T, Hv, dv), dtype=torch.float32, device=dev),
               dg=torch.empty((T, Hv), dtype=torch.float32, device=dev),
               dbeta=torch.empty((T, Hv), dtype=torch.float32, device=dev),
               dh0=(torch.empty((n_seqs, Hv, dv, dk), dtype=torch.float32, device=dev)
                    if grad_initial_state else None))
    if workspace is None:
        need = gdn_backward_workspace_bytes(n_seqs, T, Hv)
        workspace = torch.empty(need, dtype=torch.uint8, device=dev) if need else None
    ws_bytes = 0 if workspace is None else workspace.numel()
    st = lib().gdn_backward(_ptr(q), q.stride(0), _ptr(k), k.stride(0), _ptr(v), v.stride(0),
                            _ptr(g), _ptr(beta), _ptr(initial_state), _ptr(grad_o),
                            _ptr(grad_final_state), _ptr(cu_seqlens), n_seqs, T, Hk, Hv, dk, dv,
                            scale, _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]),
                            _ptr(out["dg"]), _ptr(out["dbeta"]), _ptr(out["dh0"]),
                            _ptr(workspace), ws_bytes, _stream())
    _check(st, "gdn_backward")
    return out
