"""Build libdsa.so (the HIP kernels for gfx950 and the C ABI) in this package directory.

Every HIP source is compiled by hipcc for gfx950 with packed-fp32 instructions
disabled, then linked into one shared library.  Objects go to _build/ next to
this file.

Resource guard.  Every source is compiled with the compiler's per-kernel
resource remarks, and the build fails if a kernel uses scratch memory or
spills vector registers, for two reasons:
  * correctness: several kernels wait on hand-counted `s_waitcnt vmcnt(n)`
    over loads issued outside the compiler's bookkeeping (global_load_lds
    into an LDS ring).  Those counts are exact only while the compiler adds
    no vector memory operation of its own to the loops, and spills are such
    operations.  In a source that calls wait_vmcnt this is always an error;
  * time: on this stack a kernel with scratch memory pays about 3 us of
    dispatch set-up per launch, as much as a whole decode Top-K.  In the
    other sources DSA_ALLOW_SCRATCH=1 turns this failure into a report.
The per-kernel figures are written to _build/resource_usage.json.
"""
import json
import os
import re
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libdsa.so")
SOURCES = ["indexer.hip", "topk.hip", "sfa.hip", "append.hip", "prolog.hip", "scratch.hip", "dsa_api.cpp"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=gfx950", "-mcode-object-version=5", "-O3", "-std=c++17", "-fPIC", "-Wall",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I" + os.path.join(ROOT, "include"), "-I" + CSRC]
REMARKS = ["-Rpass-analysis=kernel-resource-usage"]
# Per-source extra hipcc flags (none at present).
EXTRA = {}

_FIELDS = {"VGPRs": "vgprs", "AGPRs": "agprs", "ScratchSize [bytes/lane]": "scratch_bytes",
           "SGPRs Spill": "sgpr_spill", "VGPRs Spill": "vgpr_spill", "LDS Size [bytes/block]": "lds_bytes",
           "Occupancy [waves/SIMD]": "occupancy"}
_REMARK = re.compile(r"remark:\s+(Function Name|[A-Za-z ]+(?:\[[^\]]*\])?):\s*(\S+)\s+\[-Rpass-analysis")


def resource_usage(text: str) -> dict:
    """Per-kernel resource figures from hipcc's kernel-resource-usage remarks."""
    usage, cur = {}, None
    for line in text.splitlines():
        m = _REMARK.search(line)
        if not m:
            continue
        key, val = m.group(1).strip(), m.group(2)
        if key == "Function Name":
            cur = usage.setdefault(val, {})
        elif cur is not None and key in _FIELDS:
            cur[_FIELDS[key]] = int(val)
    return usage


def resource_violations(usage: dict) -> list:
    """Kernels that use scratch memory or spill vector registers (see the module docstring)."""
    return sorted(f"{k}: scratch {v.get('scratch_bytes', 0)} B/lane, VGPR spill {v.get('vgpr_spill', 0)}"
                  for k, v in usage.items() if v.get("scratch_bytes", 0) > 0 or v.get("vgpr_spill", 0) > 0)


def compile_source(path: str, obj: str, verbose: bool = False) -> dict:
    """hipcc one source into `obj`; returns its kernels' resource usage.  Raises on a
    compile error or a resource violation."""
    lang = ["-x", "hip"] if path.endswith(".hip") else []
    name = os.path.basename(path)
    cmd = [HIPCC, *FLAGS, *EXTRA.get(name, []), *REMARKS, *lang, "-c", path, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    text = r.stdout + r.stderr
    msgs = "\n".join(l for l in text.splitlines() if "packed-fp32-ops" not in l and "remark:" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {name}:\n{msgs}")
    if msgs.strip() and verbose:
        print(msgs)
    usage = resource_usage(text)
    bad = resource_violations(usage)
    if bad and uses_counted_waits(path):
        raise RuntimeError(f"{name}: kernels using scratch memory or spilling vector registers "
                           "(hand-counted vmcnt waits would be wrong):\n  " + "\n  ".join(bad))
    if bad and os.environ.get("DSA_ALLOW_SCRATCH") != "1":
        raise RuntimeError(f"{name}: kernels using scratch memory or spilling vector registers "
                           "(about 3 us of dispatch set-up per launch; DSA_ALLOW_SCRATCH=1 only "
                           "reports them):\n  " + "\n  ".join(bad))
    if bad and verbose:
        print(f"{name}: spills (allowed by DSA_ALLOW_SCRATCH=1):\n  " + "\n  ".join(bad))
    return usage


def uses_counted_waits(path: str) -> bool:
    """Whether a source waits on hand-counted vmcnt values (calls wait_vmcnt)."""
    with open(path) as fh:
        return "wait_vmcnt" in fh.read()


def build(verbose: bool = False) -> str:
    os.makedirs(OUT, exist_ok=True)

    def one(src):
        return compile_source(os.path.join(CSRC, src), os.path.join(OUT, os.path.splitext(src)[0] + ".o"), verbose)

    with ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1)) as ex:
        usages = list(ex.map(one, SOURCES))
    report = {src: u for src, u in zip(SOURCES, usages)}
    with open(os.path.join(OUT, "resource_usage.json"), "w") as fh:
        json.dump(report, fh, indent=1, sort_keys=True)
    objs = [os.path.join(OUT, os.path.splitext(s)[0] + ".o") for s in SOURCES]
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
