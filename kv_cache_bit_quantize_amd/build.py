"""Build libkivi.so (HIP, gfx950) in-tree with hipcc."""
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libkivi.so")
SOURCES = ["kivi_api.hip", "kivi_quant.hip", "kivi_attn.hip", "kivi_attn_gqa.hip", "kivi_attn_fp16.hip",
           "kivi_attn_q4.hip", "kivi_attn_rope.hip", "kivi_probe.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # fp32 division and sqrt correctly rounded (the quantizer divides per element)
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    # no packed fp32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # matrix-instruction accumulators in ordinary VGPRs: the decode loop rescales them with
    # vector instructions, and accumulation registers would be copied back and forth
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
    # single-lane atomics stay single instructions: the optimizer would turn a work request
    # into a wave reduction whose result is broadcast (and waited for) at once
    "-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
    "-Wall", "-Wno-unused-command-line-argument",
]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature and says so; drop that line
    noise = "'-packed-fp32-ops' is not a recognized feature"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}): {' '.join(cmd)}\n{err}")
    return err


def build(verbose: bool = False, out: str = LIB, extra_flags=(), jobs: int = 8) -> str:
    """Compile every source to an object file (in parallel, each with its own gfx950 code
    object) and link them into ``out``.  ``extra_flags`` go on every compile and the link,
    e.g. ``-Xarch_host -fsanitize=address`` for a build whose host code is sanitized."""
    import concurrent.futures
    import tempfile
    with tempfile.TemporaryDirectory(prefix="kivi_build_") as tmp:
        objs, cmds = [], []
        for s in SOURCES:
            obj = os.path.join(tmp, os.path.splitext(s)[0] + ".o")
            objs.append(obj)
            cmds.append([HIPCC, *FLAGS, *extra_flags, "-c", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
                         os.path.join(CSRC, s), "-o", obj])
        link = [HIPCC, *FLAGS, *extra_flags, *objs, "-o", out + ".tmp"]
        if verbose:
            for c in cmds + [link]:
                print(" ".join(c), flush=True)
        with concurrent.futures.ThreadPoolExecutor(max(1, jobs)) as pool:
            errs = list(pool.map(_run, cmds))
        errs.append(_run(link))
    err = "\n".join(e for e in errs if e.strip())
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
