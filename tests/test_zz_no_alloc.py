"""The prefill entry point that allocates nothing (gdn_chunk_fwd_noalloc, the
library's static device workspace) against gdn_chunk_fwd with a caller
workspace: the same kernels on the same inputs give the same bits, on two
calls in a row (the second smaller, so it reads a workspace holding the first
call's larger contents), and a call whose workspace would exceed the static
buffer is rejected before anything runs."""
import numpy as np
import pytest
import torch

from gated_delta_rule_09_amd import ops, synth
from tests.gpu_util import dev_bf16, dev_f32, dev_i32, log

pytestmark = pytest.mark.gpu


def _inputs(seed, lens, Hk, Hv):
    ci = synth.chunk_inputs(seed, sum(lens), Hk=Hk, Hv=Hv, lengths=lens, h0_std=0.05)
    args = (dev_bf16(ci.q), dev_bf16(ci.k), dev_bf16(ci.v), dev_f32(ci.g), dev_f32(ci.beta))
    return ci, args


def _pair(seed, lens, Hk, Hv):
    ci, args = _inputs(seed, lens, Hk, Hv)
    T, N = sum(lens), len(lens)
    cu = dev_i32(ci.cu_seqlens)
    h0 = dev_f32(ci.h0)
    o_ref, hT_ref = ops.gdn_chunk_fwd(*args, initial_state=h0, cu_seqlens=cu)
    o = torch.full((T, Hv, 128), float("nan"), dtype=torch.float32, device="cuda")
    hT = torch.full((N, Hv, 128, 128), float("nan"), dtype=torch.float32, device="cuda")
    ops.gdn_chunk_fwd_noalloc(*args, o, initial_state=h0, final_state=hT, cu_seqlens=cu)
    torch.cuda.synchronize()
    return o, hT, o_ref, hT_ref


def test_noalloc_equals_workspace_call_twice():
    # first call: 3 sequences, 16 / 48 heads (workspace ~ 36 MB)
    lens1 = [700, 1, 1300]
    log(f"noalloc call 1: lens={lens1}")
    o, hT, o_ref, hT_ref = _pair(5101, lens1, 16, 48)
    assert torch.equal(o, o_ref) and torch.equal(hT, hT_ref)
    # second call, smaller and of another head shape: it reads a workspace
    # that still holds the first call's larger contents
    lens2 = [65, 0, 130, 3]
    log(f"noalloc call 2: lens={lens2}")
    o, hT, o_ref, hT_ref = _pair(5102, lens2, 4, 12)
    assert torch.equal(o, o_ref) and torch.equal(hT, hT_ref)


def test_noalloc_rejects_what_the_buffer_cannot_hold():
    T = 8192   # ~146 MB of workspace at 16 / 48 heads
    log(f"noalloc over capacity: T={T}")
    q = torch.zeros((T, 16, 128), dtype=torch.bfloat16, device="cuda")
    v = torch.zeros((T, 48, 128), dtype=torch.bfloat16, device="cuda")
    g = torch.zeros((T, 48), dtype=torch.float32, device="cuda")
    o = torch.full((T, 48, 128), 7.0, dtype=torch.float32, device="cuda")
    with pytest.raises(ops.GdnError) as e:
        ops.gdn_chunk_fwd_noalloc(q, q, v, g, g, o, n_seqs=1)
    assert e.value.status == -4
    torch.cuda.synchronize()
    assert bool((o == 7.0).all())
