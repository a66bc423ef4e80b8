"""Build libgdn.so (the gfx950 HIP kernels + C ABI) in-tree with hipcc.

Every source under csrc/ is compiled for gfx950 only, with packed-fp32 code
generation disabled, and linked into gated_delta_rule_09_amd/libgdn.so.

The build also checks that no kernel spills registers: the prefill scan is
written to fit its registers, and a register allocation that spills vector
registers into accumulator registers around its MFMA chains has produced wrong
results on gfx950, so a spill is treated as a build error.
"""
import concurrent.futures
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libgdn.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CFLAGS = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I", os.path.join(os.path.dirname(HERE), "include")]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, *CFLAGS, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [ln for ln in (r.stdout + r.stderr).splitlines()
            if "packed-fp32-ops' is not a recognized feature" not in ln]
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n" + "\n".join(msgs))
    if msgs:
        print("\n".join(msgs), file=sys.stderr)
    return obj


SPILL_MARKERS = ("Reload Reuse", "Spill", "Reload")


def _check_no_spills(src: str) -> None:
    """Compile `src` to gfx950 assembly and fail on any register spill or
    reload the compiler annotates."""
    asm = os.path.join(BUILD, os.path.basename(src) + ".s")
    cmd = [HIPCC, *CFLAGS, "--cuda-device-only", "-S", src, "-o", asm]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc -S failed on {src}:\n{r.stderr}")
    with open(asm) as f:
        bad = [ln.strip() for ln in f if ";" in ln and any(m in ln.split(";", 1)[1] for m in SPILL_MARKERS)]
    if bad:
        raise RuntimeError(f"{os.path.basename(src)}: the compiler spilled registers "
                           f"({len(bad)} spill/reload instructions, e.g. {bad[0]!r})")


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
        list(ex.map(_check_no_spills, srcs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
