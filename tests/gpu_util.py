"""Helpers for the GPU parity tests: host <-> device transfer and the tolerance.

Tolerance (the mixer's accuracy bar, per output tensor): relative L2 error
<= 1e-3 and max |got - ref| <= 5e-3 * max |ref|, against the fp64 oracle.
bf16 outputs of a path whose fp32 result carries more than half a bf16 ulp of
error (the prefill's fp16 matrix-unit operands) are compared with the
unrounded oracle at rel-L2 <= 1e-3 + 2^-8 (1 + 1e-3) and max-abs <= 5e-3 +
2^-8 (1 + 5e-3): the fp32 bar plus bf16's unit roundoff, the largest relative
change one rounding makes, by the triangle inequality.  (Where the same call
can return fp32, the bf16 output is also pinned bit for bit to the fp32
output rounded.)  Where the fp32 result is accurate to far below that (the fp32
VALU paths: conv, decode, norm), bf16 outputs are held to the fp32 tolerance
and, in addition, compared on the bf16 grid: every element within one bf16 ulp of the oracle's rounded value
(both sides round once, the kernel from fp32, the oracle from fp64), except
where the kernel's fp32 arithmetic itself is off by more than that: a value
that comes out of cancellation (a conv sum whose terms nearly cancel) carries
an fp32 error of about 2^-24 of the cancelled terms, which can exceed one ulp
of the small result.  Such elements must be within 2^-16 * max|ref| absolute.
"""
import sys

import numpy as np
import torch

REL_L2 = 1e-3
MAX_ABS = 5e-3
BF16_U = 2.0 ** -8        # unit roundoff of bf16 (8 significant bits, round to nearest)


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def dev_bf16(a_u16: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a_u16).view(np.int16)).view(torch.bfloat16).cuda()


def dev_f32(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def dev_i32(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    if t.dtype == torch.bfloat16:
        u = t.cpu().view(torch.int16).numpy().view(np.uint16)
        return (u.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return t.cpu().numpy().astype(np.float64)


def errors(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    nr = np.linalg.norm(ref)
    rel = np.linalg.norm(got - ref) / nr if nr > 0 else np.linalg.norm(got - ref)
    mx = np.max(np.abs(ref)) if ref.size else 0.0
    mabs = np.max(np.abs(got - ref)) / mx if mx > 0 else (np.max(np.abs(got - ref)) if ref.size else 0.0)
    return rel, mabs


def assert_close(got, ref, name=""):
    got = np.asarray(got, dtype=np.float64)
    assert got.shape == np.shape(ref), f"{name}: shape {got.shape} vs {np.shape(ref)}"
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    rel, mabs = errors(got, ref)
    log(f"  {name}: rel_l2={rel:.3e} max_abs/max_ref={mabs:.3e}")
    assert rel <= REL_L2, f"{name}: rel-L2 {rel:.3e} > {REL_L2}"
    assert mabs <= MAX_ABS, f"{name}: max-abs {mabs:.3e} > {MAX_ABS} * max|ref|"


def bf16_ulp(x):
    x = np.abs(np.asarray(x, dtype=np.float64))
    e = np.floor(np.log2(np.maximum(x, 2.0 ** -126)))
    return 2.0 ** (e - 7)


BF16_ABS_FLOOR = 2.0 ** -16


def assert_bf16_within_1ulp(got, ref, name=""):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert_close(got, ref, name)
    d = np.abs(got - ref)
    over = d > bf16_ulp(ref) * 1.0000001
    mx = np.max(np.abs(ref)) if ref.size else 0.0
    bad = over & (d > BF16_ABS_FLOOR * mx)
    frac = np.mean(got != ref) if got.size else 0.0
    log(f"  {name}: bf16 mismatches {frac:.2e}, over 1 ulp {int(over.sum())}, "
        f"max |d|/ulp {np.max(d / bf16_ulp(ref)) if got.size else 0:.2f}, "
        f"max |d| over 1 ulp / max|ref| {np.max(d[over]) / mx if over.any() else 0:.2e}")
    assert not np.any(bad), f"{name}: {int(bad.sum())} elements differ by more than 1 bf16 ulp"


def assert_bf16_rounded_close(got, ref, name=""):
    """A bf16 output of a path whose fp32 result meets the bar against the
    unrounded oracle.  Rounding to bf16 moves each element x by at most
    2^-8 |x|, so by the triangle inequality rel-L2 <= 1e-3 + 2^-8 (1 + 1e-3)
    and max-abs <= (5e-3 + 2^-8 (1 + 5e-3)) max|ref|."""
    got = np.asarray(got, dtype=np.float64)
    assert got.shape == np.shape(ref), f"{name}: shape {got.shape} vs {np.shape(ref)}"
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    rel, mabs = errors(got, ref)
    log(f"  {name}: rel_l2={rel:.3e} max_abs/max_ref={mabs:.3e} (bf16-rounded)")
    assert rel <= REL_L2 + BF16_U * (1 + REL_L2), f"{name}: rel-L2 {rel:.3e} > 1e-3 + 2^-8"
    assert mabs <= MAX_ABS + BF16_U * (1 + MAX_ABS), f"{name}: max-abs {mabs:.3e} > 5e-3 + 2^-8"
