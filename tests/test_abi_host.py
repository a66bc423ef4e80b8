"""Host-side checks of the C ABI (no GPU needed): libgdn.so loads, exports every
function include/gdn.h declares, and rejects invalid arguments synchronously,
before any HIP call, with the documented status codes.  Pointers here are fake
addresses; every call is built to fail validation, so none is dereferenced."""
import ctypes
import os

import pytest

from gated_delta_rule_09_amd import ops

OK, NULL, SHAPE, UNSUP, WS, ALIAS = 0, -1, -2, -3, -4, -5

A = 0x7f0000000000          # fake, 256-byte aligned "device" addresses
MB = 1 << 20


def P(i):
    return A + i * 1024 * MB


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(ops.LIB_PATH):
        pytest.skip("libgdn.so not built")
    return ops.lib()


def test_exports_every_declared_function(lib):
    names = ops.header_functions()
    assert len(names) >= 10
    for n in names:
        assert hasattr(lib, n), f"{n} declared in gdn.h but not exported"


def test_abi_version_and_status_strings(lib):
    assert lib.gdn_abi_version() == 8
    for code, name in [(OK, "GDN_OK"), (NULL, "GDN_ERR_NULL"), (SHAPE, "GDN_ERR_SHAPE"),
                       (UNSUP, "GDN_ERR_UNSUPPORTED"), (WS, "GDN_ERR_WORKSPACE"),
                       (ALIAS, "GDN_ERR_ALIAS"), (-6, "GDN_ERR_HIP"), (-7, "GDN_ERR_SEQLENS")]:
        assert lib.gdn_status_string(code).decode() == name


def chunk(lib, **kw):
    a = dict(q=P(0), qs=2048, k=P(1), ks=2048, v=P(2), vs=6144, g=P(3), beta=P(4), o=P(5),
             h0=None, hT=None, cu=None, N=1, T=64, Hk=16, Hv=48, dk=128, dv=128, scale=1.0,
             ws=None, wsb=0, stream=None)
    a.update(kw)
    return lib.gdn_chunk_fwd(a["q"], a["qs"], a["k"], a["ks"], a["v"], a["vs"], a["g"],
                             a["beta"], a["o"], a["h0"], a["hT"], a["cu"], a["N"], a["T"],
                             a["Hk"], a["Hv"], a["dk"], a["dv"], a["scale"], a["ws"], a["wsb"],
                             a["stream"])


def test_chunk_fwd_validation(lib):
    assert chunk(lib, q=None) == NULL
    assert chunk(lib, o=None) == NULL
    assert chunk(lib, Hv=47) == SHAPE                 # Hv % Hk != 0
    assert chunk(lib, dk=64) == UNSUP
    assert chunk(lib, dv=256) == UNSUP
    assert chunk(lib, qs=1000) == SHAPE               # stride < Hk * dk
    assert chunk(lib, vs=6148) == SHAPE               # not a multiple of 8
    assert chunk(lib, T=65, N=2) == SHAPE             # equal split impossible
    assert chunk(lib, N=0, T=5) == SHAPE
    assert chunk(lib, q=P(0) + 2) == SHAPE            # misaligned
    assert chunk(lib, scale=float("inf")) == SHAPE
    # varlen needs a workspace of the advertised size
    need = lib.gdn_chunk_fwd_workspace_bytes(3, 64, 16, 48, 128)
    assert need > 0
    assert chunk(lib, cu=P(6), N=3) == WS
    assert chunk(lib, cu=P(6), N=3, ws=P(7), wsb=need - 1) == WS
    # o overlapping an input / final state overlapping o
    assert chunk(lib, o=P(0) + 4096) == ALIAS
    assert chunk(lib, hT=P(5)) == ALIAS
    # final state partially overlapping the initial state
    assert chunk(lib, h0=P(8), hT=P(8) + 4096) == ALIAS
    assert b"overlap" in lib.gdn_last_error()


def test_chunk_fwd_workspace_carries_state_for_long_sequences(lib):
    """Sequences of 32768 tokens or more (T_total / n_seqs) get room for the
    state carried between the segments of the overlapped launch."""
    carry = 48 * 128 * 128 * 4
    chunk_blobs = 16 * 33792 + 48 * 12544       # room for one more chunk
    for n in (1, 2):
        a = lib.gdn_chunk_fwd_workspace_bytes(n, n * 32767, 16, 48, 128)
        b = lib.gdn_chunk_fwd_workspace_bytes(n, n * 32768, 16, 48, 128)
        extra = b - a - n * carry
        assert chunk_blobs <= extra <= chunk_blobs + 4096, (n, b - a)


def test_calib_mfma_loop_validation(lib):
    assert lib.gdn_calib_mfma_loop(10, 4, None, None) == NULL
    assert lib.gdn_calib_mfma_loop(0, 4, P(0), None) == SHAPE
    assert lib.gdn_calib_mfma_loop(10, 0, P(0), None) == SHAPE
    assert lib.gdn_calib_mfma_loop(10, (1 << 20) + 1, P(0), None) == SHAPE
    assert lib.gdn_calib_mfma_loop(10, 4, P(0) + 2, None) == SHAPE
    # 4 waves per block, 8 products of 2*16*16*32 flops per wave and round
    assert lib.gdn_calib_mfma_loop_flops(10, 4) == 4 * 4 * 10 * 8 * 16384
    assert lib.gdn_calib_mfma_loop_flops(0, 4) == 0.0


def test_calib_stream_inplace_validation(lib):
    assert lib.gdn_calib_stream_inplace(None, 1024, 4, None) == NULL
    assert lib.gdn_calib_stream_inplace(P(0), 0, 4, None) == SHAPE
    assert lib.gdn_calib_stream_inplace(P(0), 1000, 4, None) == SHAPE      # not a multiple of 16
    assert lib.gdn_calib_stream_inplace(P(0), 1024, 0, None) == SHAPE
    assert lib.gdn_calib_stream_inplace(P(0), 1024, (1 << 20) + 1, None) == SHAPE
    assert lib.gdn_calib_stream_inplace(P(0) + 8, 1024, 4, None) == SHAPE  # misaligned


def test_chunk_fwd_bf16o_validation(lib):
    def c16(**kw):
        a = dict(q=P(0), qs=2048, k=P(1), ks=2048, v=P(2), vs=6144, g=P(3), beta=P(4), o=P(5),
                 h0=None, hT=None, cu=None, N=1, T=64, Hk=16, Hv=48, dk=128, dv=128, scale=1.0,
                 ws=None, wsb=0, stream=None)
        a.update(kw)
        return lib.gdn_chunk_fwd_bf16o(a["q"], a["qs"], a["k"], a["ks"], a["v"], a["vs"], a["g"],
                                       a["beta"], a["o"], a["h0"], a["hT"], a["cu"], a["N"], a["T"],
                                       a["Hk"], a["Hv"], a["dk"], a["dv"], a["scale"], a["ws"],
                                       a["wsb"], a["stream"])
    assert c16(o=None) == NULL
    assert c16(dk=64) == UNSUP
    assert c16(o=P(5) + 8) == SHAPE                   # o must be 16-byte aligned
    # a bf16 o of 64 x 48 x 128 elements is 786,432 bytes: ending 2 bytes into g overlaps it
    assert c16(o=P(3) - 786432 + 16) == ALIAS
    assert c16(o=P(3) - 786432) == WS                 # just below g: no overlap, no workspace


def test_decode_validation(lib):
    def dec(**kw):
        a = dict(q=P(0), qs=2048, k=P(1), ks=2048, v=P(2), vs=6144, g=P(3), b=P(4), st=P(5),
                 slot=None, nslots=4, o=P(6), N=4, Hk=16, Hv=48, dk=128, dv=128)
        a.update(kw)
        return lib.gdn_decode_step(a["q"], a["qs"], a["k"], a["ks"], a["v"], a["vs"], a["g"],
                                   a["b"], a["st"], a["slot"], a["nslots"], a["o"], a["N"],
                                   a["Hk"], a["Hv"], a["dk"], a["dv"], 1.0, None)
    assert dec(st=None) == NULL
    # an empty batch may pass NULL data pointers and enqueues nothing
    assert dec(q=None, k=None, v=None, g=None, b=None, st=None, o=None, N=0, nslots=0) == OK
    assert dec(nslots=3) == SHAPE                      # fewer slots than sequences, no map
    assert dec(Hk=5) == SHAPE
    assert dec(dk=96) == UNSUP
    assert dec(o=P(5) + 64) == ALIAS                   # o inside the state
    assert dec(st=P(2)) == ALIAS                       # state over v


def test_decode_tokens_validation(lib):
    def dec(**kw):
        a = dict(q=P(0), qs=2048, k=P(1), ks=2048, v=P(2), vs=6144, g=P(3), b=P(4), st=P(5),
                 slot=None, nslots=4, o=P(6), N=4, nt=3, Hk=16, Hv=48, dk=128, dv=128)
        a.update(kw)
        return lib.gdn_decode_tokens(a["q"], a["qs"], a["k"], a["ks"], a["v"], a["vs"], a["g"],
                                     a["b"], a["st"], a["slot"], a["nslots"], a["o"], a["N"],
                                     a["nt"], a["Hk"], a["Hv"], a["dk"], a["dv"], 1.0, None)
    assert dec(v=None) == NULL
    assert dec(q=None, k=None, v=None, g=None, b=None, st=None, o=None, N=0, nslots=0) == OK
    assert dec(nt=0) == UNSUP
    assert dec(nt=9) == UNSUP
    assert dec(nslots=3) == SHAPE
    assert dec(vs=6148) == SHAPE
    assert dec(q=P(0) + 8) == SHAPE                    # misaligned
    assert dec(o=P(5) + 64) == ALIAS                   # o inside the state
    # o's rows are N * n_tokens long: the last token row of o overlapping g
    assert dec(o=P(3) - 4 * 48 * 128 * 12 + 4) == ALIAS


def test_decode_mixer_step_validation(lib):
    def mix(**kw):
        a = dict(x=P(0), xs=10240, w=P(1), bias=None, cs=P(2), g=P(3), b=P(4), pa=None, pas=48,
                 pb=None, pbs=48, A=None, dt=None, z=P(5), zs=6144, nw=P(6), st=P(7), slot=None,
                 nslots=4, out=P(8), bf=0, N=4, Hk=16, Hv=48, d=128, l2=1e-6, ne=1e-6)
        a.update(kw)
        return lib.gdn_decode_mixer_step(a["x"], a["xs"], a["w"], a["bias"], a["cs"], a["g"],
                                         a["b"], a["pa"], a["pas"], a["pb"], a["pbs"], a["A"],
                                         a["dt"], a["z"], a["zs"], a["nw"], a["st"], a["slot"],
                                         a["nslots"], a["out"], a["bf"], a["N"], a["Hk"], a["Hv"],
                                         a["d"], 1.0, a["l2"], a["ne"], None)
    assert mix(z=None) == NULL
    assert mix(x=None, w=None, cs=None, g=None, b=None, z=None, nw=None, st=None, out=None,
               N=0) == OK
    assert mix(d=64) == UNSUP
    assert mix(Hk=8, Hv=48) == UNSUP                   # six value heads per key head
    assert mix(Hv=40) == SHAPE                          # Hv not a multiple of Hk
    assert mix(nslots=3) == SHAPE
    assert mix(xs=10000) == SHAPE
    assert mix(st=P(7) + 8) == SHAPE                    # state not 16-byte aligned
    assert mix(l2=-1.0) == SHAPE
    assert mix(out=P(7) + 64) == ALIAS                 # out inside the state
    assert mix(cs=P(0) + 16) == ALIAS                  # conv state over x
    assert mix(st=P(2) + 256) == ALIAS                 # state over the conv state
    proj = dict(g=None, b=None, pa=P(3), pb=P(3) + 4096, A=P(4), dt=P(4) + 256)
    assert mix(**dict(proj, g=P(9))) == NULL           # both gate sources
    assert mix(**dict(proj, dt=None)) == NULL          # incomplete projections
    assert mix(**dict(proj, pas=40)) == SHAPE          # a's stride below Hv
    assert mix(**dict(proj, pa=P(8))) == ALIAS         # a inside out


def test_chunk_pooled_validation(lib):
    def pooled(**kw):
        a = dict(q=P(0), qs=2048, k=P(1), ks=2048, v=P(2), vs=6144, g=P(3), b=P(4), o=P(5), bf=0,
                 st=P(6), slot=P(7), nslots=8, cu=None, N=2, T=128, ws=P(9), wsb=1 << 30)
        a.update(kw)
        return lib.gdn_chunk_fwd_pooled(a["q"], a["qs"], a["k"], a["ks"], a["v"], a["vs"], a["g"],
                                        a["b"], a["o"], a["bf"], a["st"], a["slot"], a["nslots"],
                                        a["cu"], a["N"], a["T"], 16, 48, 128, 128, 1.0, a["ws"],
                                        a["wsb"], None)
    assert pooled(slot=None) == NULL
    assert pooled(st=None) == NULL
    assert pooled(nslots=-1) == SHAPE
    assert pooled(slot=P(7) + 2) == SHAPE              # misaligned slot map
    assert pooled(o=P(6) + 1024) == ALIAS              # o inside the pool
    assert pooled(slot=P(6) + 4096) == ALIAS           # slot map inside the pool
    assert pooled(wsb=16) == WS


def test_chunk_gated_validation(lib):
    def gated(**kw):
        a = dict(q=P(0), qs=2048, k=P(1), ks=2048, v=P(2), vs=6144, a=P(3), as_=48, b=P(4),
                 bs=48, A=P(5), dt=P(5) + 256, o=P(6), h0=None, hT=P(7), cu=None, N=1, T=128,
                 ws=P(9), wsb=1 << 30)
        a.update(kw)
        return lib.gdn_chunk_fwd_gated(a["q"], a["qs"], a["k"], a["ks"], a["v"], a["vs"], a["a"],
                                       a["as_"], a["b"], a["bs"], a["A"], a["dt"], a["o"],
                                       a["h0"], a["hT"], a["cu"], a["N"], a["T"], 16, 48, 128,
                                       128, 1.0, a["ws"], a["wsb"], None)
    assert gated(a=None) == NULL
    assert gated(dt=None) == NULL
    assert gated(a=None, b=None, A=None, dt=None, q=None, k=None, v=None, o=None, hT=None,
                 N=0, T=0) == OK
    assert gated(as_=40) == SHAPE                       # a's token stride below Hv
    assert gated(A=P(5) + 2) == SHAPE                   # misaligned A_log
    assert gated(o=P(3) + 64) == ALIAS                  # o over a
    assert gated(hT=P(4)) == ALIAS                      # final state over b


def test_mixer_fwd_validation(lib):
    def mix(**kw):
        a = dict(x=P(0), xs=10240, w=P(1), bias=None, cs=None, g=P(2), b=P(3), pa=None, pas=48,
                 pb=None, pbs=48, A=None, dt=None, z=P(4), zs=6144, nw=P(5), out=P(6), bf=0,
                 h0=None, hT=P(7), slot=None, nslots=0, cu=None, N=1, T=128, d=128, ws=P(9),
                 wsb=1 << 30)
        a.update(kw)
        return lib.gdn_mixer_fwd(a["x"], a["xs"], a["w"], a["bias"], a["cs"], a["g"], a["b"],
                                 a["pa"], a["pas"], a["pb"], a["pbs"], a["A"], a["dt"],
                                 a["z"], a["zs"], a["nw"], a["out"], a["bf"], a["h0"], a["hT"],
                                 a["slot"], a["nslots"],
                                 a["cu"], a["N"], a["T"], 16, 48, a["d"], 1.0, 1e-6, 1e-6,
                                 a["ws"], a["wsb"], None)
    assert mix(z=None) == NULL
    assert mix(d=64) == UNSUP
    assert mix(xs=10000) == SHAPE
    assert mix(bias=P(8) + 4) == SHAPE                 # bias must be 16-byte aligned
    assert mix(out=P(0) + 4096) == ALIAS               # out over x
    assert mix(cs=P(7) + 64) == ALIAS                  # conv state over the final state
    assert mix(wsb=1024) == WS
    need = lib.gdn_mixer_fwd_workspace_bytes(1, 128, 16, 48, 128, 1)
    assert need > lib.gdn_mixer_fwd_workspace_bytes(1, 128, 16, 48, 128, 0)
    assert mix(bf=1, wsb=need - 256) == WS
    proj = dict(g=None, b=None, pa=P(2), pb=P(2) + 65536, A=P(3), dt=P(3) + 256)
    assert mix(**dict(proj, b=P(8))) == NULL           # both gate sources
    assert mix(**dict(proj, A=None)) == NULL           # incomplete projections
    assert mix(**dict(proj, pbs=47)) == SHAPE          # b's stride below Hv
    assert mix(**dict(proj, pa=P(7))) == ALIAS         # a inside the final state
    assert mix(slot=P(8), nslots=4, h0=P(7), hT=P(7) + 1024 * 1024) == SHAPE  # not one pool
    assert mix(slot=P(8) + 2, nslots=4, h0=P(7), hT=P(7)) == SHAPE       # misaligned slot map
    assert mix(slot=P(7) + 64, nslots=4, h0=P(7), hT=P(7)) == ALIAS      # slot map inside the pool


def backward(lib, **kw):
    a = dict(q=P(0), qs=2048, k=P(1), ks=2048, v=P(2), vs=6144, g=P(3), beta=P(4), h0=None,
             do=P(5), dhT=None, cu=None, N=1, T=64, Hk=16, Hv=48, dk=128, dv=128, scale=1.0,
             dq=P(6), dkk=P(7), dvv=P(8), dg=P(9), db=P(10), dh0=None, ws=None, wsb=0,
             stream=None)
    a.update(kw)
    return lib.gdn_backward(a["q"], a["qs"], a["k"], a["ks"], a["v"], a["vs"], a["g"], a["beta"],
                            a["h0"], a["do"], a["dhT"], a["cu"], a["N"], a["T"], a["Hk"], a["Hv"],
                            a["dk"], a["dv"], a["scale"], a["dq"], a["dkk"], a["dvv"], a["dg"],
                            a["db"], a["dh0"], a["ws"], a["wsb"], a["stream"])


def chunked_backward_bytes(n_seqs, T, Hv):
    """gdn_backward's workspace: per chunk slot (T // 64 + n_seqs of them) a
    slot -> sequence entry, and per (slot, value head) the 64 x 64 matrix of
    T and P, the state before and the state gradient after the chunk
    (128 x 128 each) and U, E, dR (64 x 128 each), fp32, every array
    256-byte aligned."""
    up = lambda b: (b + 255) // 256 * 256
    slots = T // 64 + n_seqs
    sh = slots * Hv
    return up(4 * slots) + up(sh * 64 * 64 * 4) + 2 * up(sh * 128 * 128 * 4) + 3 * up(sh * 64 * 128 * 4)


def test_backward_validation(lib):
    need = lib.gdn_backward_workspace_bytes(1, 64, 48)
    assert need == chunked_backward_bytes(1, 64, 48) == 23593216
    assert lib.gdn_backward_workspace_bytes(1, 0, 48) == 0
    for n_seqs, T in ((2, 80), (3, 1), (64, 2560), (65, 8192), (8, 8192)):
        assert lib.gdn_backward_workspace_bytes(n_seqs, T, 48) == chunked_backward_bytes(n_seqs, T, 48), n_seqs
    assert backward(lib, do=None) == NULL
    assert backward(lib, dg=None) == NULL
    assert backward(lib, Hv=40) == SHAPE
    assert backward(lib, dk=64) == UNSUP
    assert backward(lib, ks=1000) == SHAPE
    assert backward(lib, T=65, N=2) == SHAPE
    assert backward(lib, q=P(0) + 8) == SHAPE
    assert backward(lib, scale=float("nan")) == SHAPE
    assert backward(lib) == WS
    assert backward(lib, ws=P(11), wsb=need - 1) == WS
    assert backward(lib, ws=P(11) + 64, wsb=need) == WS          # not 256-byte aligned
    assert backward(lib, dq=P(0) + 4096, ws=P(11), wsb=need) == ALIAS   # output over an input
    assert backward(lib, dkk=P(6) + 4096, ws=P(11), wsb=need) == ALIAS  # two outputs overlap
    assert backward(lib, ws=P(10), wsb=need) == ALIAS                   # workspace over an output


def test_conv_validation(lib):
    def conv(**kw):
        a = dict(x=P(0), xs=10240, w=P(1), bias=None, y=P(2), ys=10240, cs=None, cu=None, N=1,
                 T=16, C=10240, nl2=32, hd=128, eps=1e-6)
        a.update(kw)
        return lib.gdn_conv1d_fwd(a["x"], a["xs"], a["w"], a["bias"], a["y"], a["ys"], a["cs"],
                                  a["cu"], a["N"], a["T"], a["C"], a["nl2"], a["hd"], a["eps"],
                                  None)
    assert conv(x=None) == NULL
    assert conv(hd=64) == UNSUP
    assert conv(C=10244) == UNSUP
    assert conv(nl2=81) == SHAPE
    assert conv(xs=10000) == SHAPE
    assert conv(y=P(0) + 16) == ALIAS
    assert conv(eps=-1.0) == SHAPE


def test_rmsnorm_validation(lib):
    def rn(**kw):
        a = dict(o=P(0), z=P(1), zs=6144, w=P(2), out=P(3), bf=0, rows=8, Hv=48, dv=128, eps=1e-6)
        a.update(kw)
        return lib.gdn_gated_rmsnorm(a["o"], a["z"], a["zs"], a["w"], a["out"], a["bf"],
                                     a["rows"], a["Hv"], a["dv"], a["eps"], None)
    assert rn(w=None) == NULL
    assert rn(dv=64) == UNSUP
    assert rn(zs=6000) == SHAPE
    assert rn(out=P(1)) == ALIAS                      # out over z
    assert rn(out=P(0), bf=1) == ALIAS                 # bf16 out cannot alias fp32 o
    assert rn(out=P(0) + 512) == ALIAS                 # partial alias with o


def test_chunk_map_and_seqlens_validation(lib):
    assert lib.gdn_chunk_map(None, 1, 1, P(0), P(1), P(2), None) == NULL
    assert lib.gdn_chunk_map(P(3), -1, 1, P(0), P(1), P(2), None) == SHAPE
    assert lib.gdn_validate_cu_seqlens(None, 1, 1, None) == NULL
    assert lib.gdn_validate_cu_seqlens(P(0), -2, 1, None) == SHAPE


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(ops, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(ops, "_lib_handle", None)
    with pytest.raises(RuntimeError, match="not built"):
        ops.lib()


def test_backward_chunk_slots_fit_the_workspace():
    """The arithmetic claim behind gdn_backward's per-chunk records: chunk c
    of sequence n (tokens s0 + 64 c ..) goes to slot (s0 + 64 c) // 64 + n,
    which gives distinct slots below T // 64 + N, the count the workspace
    holds, over random packings with empty, one-token and chunk-multiple
    sequences.  (This checks the scheme; the GPU tests run the kernels' own
    indexing on such packings.)"""
    import numpy as np
    r = np.random.default_rng(31)
    for _ in range(300):
        lens = r.integers(0, 300, size=int(r.integers(1, 12)))
        if r.integers(0, 3) == 0:
            lens[r.integers(0, len(lens))] = 1
        if r.integers(0, 3) == 0:
            lens[r.integers(0, len(lens))] = 64 * int(r.integers(1, 4))
        cu = np.concatenate([[0], np.cumsum(lens)])
        T, N = int(cu[-1]), len(lens)
        slots = [(int(cu[n]) + 64 * c) // 64 + n for n in range(N)
                 for c in range((int(lens[n]) + 63) // 64)]
        assert len(set(slots)) == len(slots)
        assert all(0 <= s < T // 64 + N for s in slots)


def test_build_flags_mixed_shape_mfma_accumulator_chains():
    """The build's assembly check: an MFMA whose accumulator input is the
    result of an MFMA of another shape a few instructions earlier is
    reported; a result rewritten in between (an LDS read, an MFMA of the same
    shape, also one with an immediate zero accumulator) is not."""
    from gated_delta_rule_09_amd import build as B
    bad = ["\tv_mfma_f32_16x16x32_f16 v[0:3], v[4:7], v[8:11], v[0:3]",
           "\tv_add_f32_e32 v20, v21, v22",
           "\tv_mfma_f32_16x16x16_f16 v[0:3], v[4:5], v[8:9], v[0:3]"]
    assert len(B.mixed_mfma_chains(bad)) == 1
    ok = ["\tv_mfma_f32_16x16x4_f32 v[110:113], v84, v238, v[102:105]",
          "\tds_read2_b64 v[108:111], v149 offset0:32 offset1:36",
          "\tv_mfma_f32_16x16x32_bf16 v[112:115], v[108:111], v[94:97], 0",
          "\tv_mfma_f32_16x16x32_bf16 v[108:111], v[108:111], v[100:103], v[112:115]"]
    assert B.mixed_mfma_chains(ok) == []
