"""MI355X-native gated-delta-rule token mixer (gfx950 HIP kernels behind a C ABI).

The compute entry points live in ``gated_delta_rule_09_amd.ops`` and load the
HIP library ``libgdn.so`` on first use; they raise if it is missing.  There is
no CPU fallback.
"""
__all__ = ["synth"]
