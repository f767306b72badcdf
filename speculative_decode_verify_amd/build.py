"""Build the HIP library libverify_attn.so in-tree for gfx950.

    python -m speculative_decode_verify_amd.build              # build
    python -m speculative_decode_verify_amd.build --resources  # resource table

Compiles every source under csrc/ with hipcc into lib/libverify_attn.so.
Always recompiles (a build check must exercise the compiler).  With
--resources it instead prints, as a markdown table, what the compiler reports
for every kernel instance (-Rpass-analysis=kernel-resource-usage: VGPRs,
AGPRs, SGPRs, scratch, LDS, occupancy in waves per SIMD) and the workgroups
per CU those allow.  The build also records the revision and the compiler in
lib/build_info.json, which the benchmark copies into its output line.
"""
import json
import os
import re
import shutil
import subprocess
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB_DIR = os.path.join(HERE, "lib")
LIB = os.path.join(LIB_DIR, "libverify_attn.so")
# the same sources with VA_PHASE_TRACE: per-workgroup phase timestamps
# (include/verify_probe.h); loaded only by `bench.py --phases`
TRACE_LIB = os.path.join(LIB_DIR, "libverify_attn_trace.so")

SOURCES = ["verify_attn.hip", "sample.hip", "probe.hip", "plan.cpp"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # no packed-FP32 instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in VGPRs: the online-softmax rescale is VALU work on them
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
]


def hipcc():
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _git_revision():
    try:
        rev = subprocess.run(["git", "-C", ROOT, "rev-parse", "HEAD"], capture_output=True, text=True,
                             timeout=20).stdout.strip()
        dirty = subprocess.run(["git", "-C", ROOT, "status", "--porcelain", "--untracked-files=no"],
                               capture_output=True, text=True, timeout=20).stdout.strip()
        return (rev or None), bool(dirty)
    except Exception:
        return None, None


def _hipcc_version():
    try:
        out = subprocess.run([hipcc(), "--version"], capture_output=True, text=True, timeout=60).stdout
        return " | ".join(l.strip() for l in out.splitlines() if l.strip())[:400]
    except Exception:
        return None


def build(verbose=False, trace=True):
    """Compile the library (and, with trace, its trace build: the two hipcc
    runs go in parallel)."""
    os.makedirs(LIB_DIR, exist_ok=True)
    jobs = []
    for out, extra in [(LIB, [])] + ([(TRACE_LIB, ["-DVA_PHASE_TRACE"])] if trace else []):
        cmd = [hipcc(), *HIPCC_FLAGS, *extra,
               "-I", os.path.join(ROOT, "include"), "-I", CSRC,
               *[os.path.join(CSRC, s) for s in SOURCES], "-o", out + ".tmp"]
        if verbose:
            print(" ".join(cmd), flush=True)
        jobs.append((out, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
    failed = []
    for out, p in jobs:
        log = p.communicate()[0]
        if p.returncode != 0:
            sys.stderr.write(log)
            failed.append(os.path.basename(out))
    if failed:
        raise RuntimeError(f"hipcc failed building {', '.join(failed)}")
    for out, _ in jobs:
        os.replace(out + ".tmp", out)
    rev, dirty = _git_revision()
    info = {"git_revision": rev, "worktree_modified": dirty, "hipcc": _hipcc_version(),
            "flags": HIPCC_FLAGS, "built_at_utc": time.strftime("%Y-%m-%dT%H:%M:%SZ", time.gmtime())}
    with open(os.path.join(LIB_DIR, "build_info.json"), "w") as f:
        json.dump(info, f, indent=1)
    return LIB


# waves per workgroup of each kernel, from its launch shape
def _waves(name):
    m = re.match(r".*split_kernel<(\d+), (\d+), (\d+), (\d+), (\d+),", name)
    if m:
        _, w, fmt, _, npw = map(int, m.groups())
        return w + (2 if fmt == 1 else 0) + npw
    m = re.match(r".*combine_kernel<(\d+), (\d+),", name)
    if m:
        return int(m.group(2))
    if "kv_write_kernel" in name or "accept_kernel" in name:
        return 1
    return 4  # ring_write, sample and probe kernels: 256 threads


def resource_table():
    """Compile every HIP source for the device with the compiler's resource
    remarks and return a markdown table (one row per kernel instance)."""
    rows = []
    for src in SOURCES:
        if not src.endswith(".hip"):
            continue
        cmd = [hipcc(), *[f for f in HIPCC_FLAGS if f not in ("-shared", "-fPIC")], "--cuda-device-only", "-c",
               "-o", os.devnull, "-Rpass-analysis=kernel-resource-usage",
               "-I", os.path.join(ROOT, "include"), "-I", CSRC, os.path.join(CSRC, src)]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            sys.stderr.write(r.stderr)
            raise RuntimeError("hipcc failed")
        cur = None
        for line in r.stderr.splitlines():
            m = re.search(r"remark: Function Name: (\S+)", line)
            if m:
                cur = {"mangled": m.group(1)}
                rows.append(cur)
                continue
            m = re.search(r"remark:\s+([A-Za-z ]+?)(?: \[[^\]]*\])?: (\d+)", line)
            if m and cur is not None:
                cur[m.group(1).strip()] = int(m.group(2))
    names = subprocess.run(["c++filt"], input="\n".join(x["mangled"] for x in rows), capture_output=True,
                           text=True).stdout.splitlines()
    out = ["| kernel | waves/WG | VGPRs | AGPRs | SGPRs | scratch B/lane | LDS B/WG | occupancy waves/SIMD "
           "| WGs per CU (waves, LDS) |", "|---|---|---|---|---|---|---|---|---|"]
    for x, n in zip(rows, names):
        n = n.replace("va_detail::", "").replace("va_sample_detail::", "").replace("va_probe_detail::", "")
        n = re.sub(r"\(.*\)$", "", n)
        wv = _waves(n)
        occ = x.get("Occupancy", 0)
        lds = x.get("LDS Size", 0)
        by_waves = (4 * occ) // wv if wv else 0
        by_lds = 163840 // lds if lds else by_waves
        out.append(f"| `{n}` | {wv} | {x.get('VGPRs', '?')} | {x.get('AGPRs', '?')} | {x.get('TotalSGPRs', '?')} "
                   f"| {x.get('ScratchSize', '?')} | {lds} | {occ} | {min(by_waves, by_lds)} |")
    return "\n".join(out)


if __name__ == "__main__":
    if "--resources" in sys.argv:
        print(resource_table())
    else:
        print(build(verbose=True))
