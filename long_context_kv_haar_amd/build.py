"""Build libwavefilter.so for gfx950 in place (hipcc, no GPU needed).

The per-step kernels are instantiated for every (input type, head dimension,
query tiles) combination.  wf_step.hip is compiled once per combination (and
once for its dispatcher), the units in parallel, then linked with the other
sources into one shared library.
"""

import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB_PATH = os.path.join(HERE, "libwavefilter.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    # keep float32 arithmetic in unpacked VALU instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # kernel arguments in the first 14 dwords arrive in scalar registers
    "-mllvm", "-amdgpu-kernarg-preload-count=14",
]

STEP_COMBOS = [(t, d, rt) for t in ("bf16_t", "float") for d in (128, 64) for rt in (1, 2, 3, 4)]


def _units():
    """(name, source, extra defines) of every compile unit."""
    units = [("wf_api", "wf_api.hip", []), ("wf_pyramid", "wf_pyramid.hip", []), ("wf_check", "wf_check.hip", []),
             ("wf_step_dispatch", "wf_step.hip", [])]
    for t, d, rt in STEP_COMBOS:
        units.append((f"wf_step_{t}_{d}_{rt}", "wf_step.hip",
                      [f"-DWF_STEP_T={t}", f"-DWF_STEP_D={d}", f"-DWF_STEP_RT={rt}"]))
    return units


def _filter(stderr):
    return "\n".join(l for l in stderr.splitlines() if "packed-fp32-ops" not in l)


def build(verbose=False, jobs=None):
    """Compile every HIP unit (in parallel) and link one shared library next to this file."""
    jobs = jobs or max(1, min(len(os.sched_getaffinity(0)), 16))
    units = _units()
    with tempfile.TemporaryDirectory(prefix="wf_build_") as tmpdir:
        def compile_unit(u):
            name, src, defs = u
            obj = os.path.join(tmpdir, name + ".o")
            cmd = [HIPCC] + FLAGS + defs + ["-c", "-o", obj, os.path.join(CSRC, src)]
            res = subprocess.run(cmd, capture_output=True, text=True)
            return name, obj, cmd, res

        if verbose:
            print(f"compiling {len(units)} units with {jobs} jobs", flush=True)
        with ThreadPoolExecutor(max_workers=jobs) as ex:
            results = list(ex.map(compile_unit, units))
        objs = []
        for name, obj, cmd, res in results:
            errs = _filter(res.stderr)
            if res.returncode != 0:
                raise RuntimeError(f"hipcc failed on {name}:\n{' '.join(cmd)}\n{errs}")
            if verbose and errs.strip():
                print(errs, file=sys.stderr)
            objs.append(obj)
        tmp = LIB_PATH + ".tmp"
        cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
        if verbose:
            print(" ".join(cmd[:6]) + f" ... ({len(objs)} objects)", flush=True)
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError("link failed:\n" + _filter(res.stderr))
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
