#!/usr/bin/env python3
"""Benchmark of multi-row speculative-verification decode attention on one MI355X.

Workload (the full-attention single-GPU share): 1 KV head, 6 query heads,
head_dim 128, 8 query rows with 4..8 live, causal mask at the boundary, bf16
K/V/q ~ N(0,1), sink logits ~ N(0,1), KV capacity preallocated at 262,144
keys, contexts 1K, 4K, 16K, 32K, 64K, 128K and 192K; split count chosen by
the plan.  One step = one verify call (split + combine) at each of the seven
contexts.

Cold-cache rule: for whole steps every context of every replica has its own
256K-capacity cache (6 replicas x 7 contexts); step i reads replica i % 6,
so about 1.4 GB of distinct KV is streamed between two reads of the same
bytes, more than the 256 MB Infinity Cache.  Capacity beyond each read
extent is NaN: reading it would poison the output, which the full-size
parity check below catches.  Per-kernel times rotate, per context, over a
pool of at least 1 GiB of replicas of that context's read extent.

Timing (HIP graphs replayed on the stream the library launches on, HIP
events around each replay):
  * value / ms_per_step: `steps` back-to-back steps.
  * per context, each over `kernel_reps` back-to-back launches: split alone,
    combine alone, split + combine pairs (us_per_call, what one call costs:
    the combine reads the partials the split has just written), the plain
    read of the same bytes, and the device-state split and combine.  The
    roofline takes the split kernel's average.
The CPU baseline times the float64 oracle on the same stored bytes (one pass
over the seven contexts) and doubles as a full-size parity check of the GPU
outputs of replica 0.

Prints one JSON line, with a `provenance` object: GPU name and ISA, compute
units, ROCm / HIP / torch versions, the library's build record (git revision,
hipcc version, flags), hashes of the library and the kernel source, the
command line, and the clock levels the driver's sysfs tables show right after
the timed region.

`--compare LIB [LIB ...]` times other builds of the library against the
built one instead (split alone and split + combine pairs per context, cold
pools as above) in drift-cancelling order: rounds alternate ABC... and
...CBA, and the built library appears twice, as arms A and A', so the A/A
spread bounds run-to-run noise.  It prints one JSON line with the median,
minimum and maximum per arm.
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

CONTEXTS = [1024, 4096, 16384, 32768, 65536, 131072, 196608]
ROWS, HQ, HKV, D, CAP = 8, 6, 1, 128, 262144
HBM_PEAK_GBS = 8000.0   # MI355X HBM3E, published
REPLICAS = 6
METRIC = "verify-attn µs/call and KV-read GB/s (% HBM peak), 8 rows×6 heads, 1K–192K ctx"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "split_kernel_verify_sweep_traffic.json")
UTIL_FILE = os.path.join(ROOT, "profiles", "split_kernel_verify_sweep_util.json")
UTIL_COUNTERS = ("SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_INSTS_MFMA SQ_LDS_BANK_CONFLICT "
                 "SQ_LDS_IDX_ACTIVE")
WAVE_COUNTERS = "SQ_WAVE_CYCLES SQ_WAIT_ANY SQ_WAIT_INST_ANY SQ_ACTIVE_INST_VALU"
INST_COUNTERS = "SQ_INSTS_VALU SQ_INSTS_MFMA SQ_INSTS_LDS SQ_INSTS_SALU"
COPY_PROBE_MIB = 1024
KERNEL_SRC = os.path.join(ROOT, "speculative_decode_verify_amd", "csrc", "verify_attn.hip")
SAMPLE_SRC = os.path.join(ROOT, "speculative_decode_verify_amd", "csrc", "sample.hip")


POOL_BYTES = 1 << 30  # every per-kernel timing rotates over at least this many distinct bytes


def cold_pool(torch, synth, dev, nbytes, seed, tail=0):
    """A flat uint8 pool of n replicas of nbytes each (n >= 6, n * nbytes >=
    1 GiB) plus `tail` bytes, filled with N(0,1) bf16 drawn on the GPU in
    256 MiB pieces.  Returns (pool, n)."""
    n = max(REPLICAS, -(-POOL_BYTES // nbytes))
    pool = torch.empty(n * nbytes + tail, dtype=torch.uint8, device=dev)
    flat = pool.view(torch.bfloat16)
    piece = 1 << 27
    for off in range(0, flat.numel(), piece):
        m = min(piece, flat.numel() - off)
        flat[off:off + m] = synth.normal_bf16_device((m,), seed + off // piece, dev)
    return pool, n


def _sysfs_device_dir(torch):
    """The sysfs directory of the GPU torch uses (matched by PCI address),
    else the first DRM card that exposes clock levels; None if neither."""
    import glob
    try:
        p = torch.cuda.get_device_properties(0)
        d = f"/sys/bus/pci/devices/{p.pci_domain_id:04x}:{p.pci_bus_id:02x}:{p.pci_device_id:02x}.0"
        if os.path.exists(os.path.join(d, "pp_dpm_sclk")):
            return d
    except Exception:  # noqa: BLE001
        pass
    cards = [c for c in sorted(glob.glob("/sys/class/drm/card*/device")) if os.path.exists(os.path.join(c, "pp_dpm_sclk"))]
    return cards[0] if cards else None


def _sysfs_clocks(torch):
    """Current gfx (sclk) and memory (mclk) clock levels from the driver's
    sysfs tables (the level marked '*'), read right after the timed region.
    A file read: the process that holds the GPU starts no other program."""
    d = _sysfs_device_dir(torch)
    if d is None:
        return {"error": "no pp_dpm_sclk in sysfs"}

    def current(name):
        try:
            for line in open(os.path.join(d, name)):
                if line.rstrip().endswith("*"):
                    return line.split(":", 1)[1].replace("*", "").strip()
        except OSError:
            return None
        return None
    return {"sclk": current("pp_dpm_sclk"), "mclk": current("pp_dpm_mclk"),
            "source": f"{d}/pp_dpm_sclk and pp_dpm_mclk (current level), read right after the timed region"}


def _sysfs_product(torch):
    d = _sysfs_device_dir(torch)
    for name in ("product_name", "device"):
        try:
            v = open(os.path.join(d, name)).read().strip() if d else ""
            if v:
                return v if name == "product_name" else f"PCI device {v}"
        except OSError:
            pass
    return None


def provenance(torch, clocks=None):
    """Where a result came from: hardware, software, build and command."""
    props = torch.cuda.get_device_properties(0)
    lib = os.path.join(ROOT, "speculative_decode_verify_amd", "lib", "libverify_attn.so")
    info_path = os.path.join(ROOT, "speculative_decode_verify_amd", "lib", "build_info.json")
    build = {}
    if os.path.exists(info_path):
        try:
            build = json.load(open(info_path))
        except Exception:  # noqa: BLE001
            build = {}
    rocm = None
    try:
        rocm = open("/opt/rocm/.info/version").read().strip()
    except OSError:
        pass
    lib_hash = None
    if os.path.exists(lib):
        with open(lib, "rb") as f:
            lib_hash = hashlib.sha256(f.read()).hexdigest()[:16]
    return {"gpu": _sysfs_product(torch) or props.name, "gpu_runtime_name": props.name, "arch": getattr(props, "gcnArchName", None),
            "compute_units": props.multi_processor_count, "rocm": rocm, "hip_runtime": torch.version.hip,
            "torch": torch.__version__, "git_revision": build.get("git_revision"),
            "worktree_modified": build.get("worktree_modified"), "hipcc": build.get("hipcc"),
            "build_flags": build.get("flags"), "built_at_utc": build.get("built_at_utc"),
            "library_sha16": lib_hash, "kernel_source_sha16": kernel_hash(),
            "command": " ".join([os.path.basename(sys.executable)] + sys.argv), "clocks": clocks}


def kv_bytes(hi):
    """Algorithmic KV bytes of one call: every visible key's K and V once (bf16)."""
    return hi * HKV * 4 * D


def kernel_hash():
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def wave_cycles(d, kname, py):
    """Wave-cycle breakdown of the split kernels from a `--pmc` run of
    WAVE_COUNTERS (pmc_waves/, log waves.log) and one of INST_COUNTERS
    (pmc_insts/, insts.log) and, when present, the same two runs of an
    earlier kernel source (pmc_waves_before/, pmc_insts_before/,
    waves_before.log, with the revision it was built from in
    waves_before.rev): the share of wave
    cycles spent waiting on anything (barriers, memory and LDS counters),
    waiting on instruction dependencies and issuing VALU, and the
    instructions issued per MFMA instruction.  The counters are whole-GPU
    totals per dispatch."""
    import csv
    import collections
    kinds = [("split_kernel<128,3,0,4,2,false>", "sweep (D 128, 3 consumers, bf16)"),
             ("split_kernel<128,6,0,4,2,false>", "tree (D 128, 6 consumers, bf16)"),
             ("split_kernel<128,3,0,4,2,false,rows2>", "tree, two row groups (D 128, 3 consumers each, bf16)"),
             ("split_kernel<128,6,1,8,1,false>", "quantised tree (E4M3 keys, INT8 values)")]

    def table(subs, log):
        paths = [os.path.join(d, sub, "bench_counter_collection.csv") for sub in subs]
        if not all(os.path.exists(p) for p in paths):
            return None, None
        line = None
        for x in open(os.path.join(d, log)):
            if x.startswith("{") and '"metric"' in x:
                line = json.loads(x)
        vals = collections.defaultdict(lambda: collections.defaultdict(list))
        for path in paths:
            for r in csv.DictReader(open(path)):
                n = kname(r["Kernel_Name"])
                wgs = int(r["Grid_Size"]) // int(r["Workgroup_Size"])
                for key, _ in kinds:
                    if key in n:
                        vals[(key, wgs)][r["Counter_Name"]].append(float(r["Counter_Value"]))
        rows = {}
        for (key, wgs), v in vals.items():
            a = {c: sum(x) / len(x) for c, x in v.items()}
            cyc = a.get("SQ_WAVE_CYCLES", 0.0)
            mf = a.get("SQ_INSTS_MFMA", 0.0)
            if not cyc or not mf:
                continue
            rows[(key, wgs)] = dict(
                dispatches=len(v["SQ_WAVE_CYCLES"]), wait_any=100 * a["SQ_WAIT_ANY"] / cyc,
                wait_inst=100 * a["SQ_WAIT_INST_ANY"] / cyc, valu_active=100 * a["SQ_ACTIVE_INST_VALU"] / cyc,
                valu_per_mfma=a["SQ_INSTS_VALU"] / mf, lds_per_mfma=a["SQ_INSTS_LDS"] / mf,
                salu_per_mfma=a["SQ_INSTS_SALU"] / mf, mfma=mf)
        return rows, line

    after, al = table(("pmc_waves", "pmc_insts"), "waves.log")
    if after is None:
        return
    for log in ("waves.log", "insts.log"):
        for x in open(os.path.join(d, log)):
            if x.startswith("{") and '"metric"' in x and json.loads(x)["kernel_hash"] != kernel_hash():
                raise SystemExit("wave counters of another kernel source")
    before, bl = table(("pmc_waves_before", "pmc_insts_before"), "waves_before.log")
    rev = None
    if before is not None and os.path.exists(os.path.join(d, "waves_before.rev")):
        rev = open(os.path.join(d, "waves_before.rev")).read().strip()
    tail = f"-o bench -- {py} --steps 2 --warmup 0 --kernel-reps 4 --no-cpu-baseline"
    o = ["# split_kernel wave cycles: waits, VALU and instructions per MFMA", "",
         f"kernel source sha256[:16]: {kernel_hash()}", "",
         f"command: rocprofv3 --pmc {WAVE_COUNTERS} -f csv -d <dir>/pmc_waves {tail}",
         f"command: rocprofv3 --pmc {INST_COUNTERS} -f csv -d <dir>/pmc_insts {tail}", ""]
    if before is not None:
        o += [f"before: the same two commands in a checkout of {rev or 'an earlier revision'} "
              f"(kernel source sha256[:16] {bl['kernel_hash'] if bl else '?'}), library built there with "
              "`python -m speculative_decode_verify_amd.build`", ""]
    o += ["Shares are of SQ_WAVE_CYCLES: wait any = SQ_WAIT_ANY (barriers, memory and LDS counters), "
          "wait inst = SQ_WAIT_INST_ANY (instruction dependencies), VALU = SQ_ACTIVE_INST_VALU. "
          "Per MFMA = SQ_INSTS_VALU, SQ_INSTS_LDS, SQ_INSTS_SALU over SQ_INSTS_MFMA.", "",
          "| kernel | workgroups | source | dispatches | wait any % | wait inst % | VALU % | VALU per MFMA | "
          "LDS per MFMA | SALU per MFMA |", "|---|---|---|---|---|---|---|---|---|---|"]
    for key, label in kinds:
        wg = sorted({w for (k, w) in list(after) + list(before or {}) if k == key})
        for w in wg:
            for tag, t in (("before", before), ("after", after)):
                r = (t or {}).get((key, w))
                if r is None:
                    continue
                o.append(f"| {label} | {w} | {tag} | {r['dispatches']} | {r['wait_any']:.1f} | {r['wait_inst']:.1f} | "
                         f"{r['valu_active']:.1f} | {r['valu_per_mfma']:.2f} | {r['lds_per_mfma']:.2f} | "
                         f"{r['salu_per_mfma']:.2f} |")
    name = os.path.join(ROOT, "profiles", "split_kernel_wave_cycles.md")
    open(name, "w").write("\n".join(o) + "\n")
    print(f"wrote {name}")


def trace_workgroups(r):
    """Workgroups of one kernel-trace row: each grid dimension (in work-items)
    over the workgroup's extent in it; a dimension the file omits counts 1."""
    n = 1
    for ax in "XYZ":
        g, w = r.get(f"Grid_Size_{ax}"), r.get(f"Workgroup_Size_{ax}")
        if g and w:
            n *= int(g) // int(w)
    return n


IC_COUNTERS = "SQC_ICACHE_MISSES SQC_ICACHE_HITS SQC_ICACHE_MISSES_DUPLICATE SQC_DCACHE_MISSES SQC_DCACHE_HITS SQ_WAVES"


def icache_table(d, kname, py):
    """profiles/split_kernel_icache.md from a `--pmc` run of IC_COUNTERS
    (pmc_ic/, log ic.log) at 1K and 64K: instruction- and scalar-cache
    misses of the sweep's split kernel, the combine and the plain read."""
    import csv
    import collections
    path = os.path.join(d, "pmc_ic", "ic_counter_collection.csv")
    if not os.path.exists(path):
        return
    for x in open(os.path.join(d, "ic.log")):
        if x.startswith("{") and '"metric"' in x and json.loads(x)["kernel_hash"] != kernel_hash():
            raise SystemExit("cache counters of another kernel source")
    agg = collections.defaultdict(lambda: collections.defaultdict(list))
    for r in csv.DictReader(open(path)):
        n = kname(r["Kernel_Name"])
        if "split_kernel<128,3,0,4,2,false>" in n:
            name = "split_kernel<128,3,0,4,2,false>"
        elif "combine_kernel<" in n:
            name = n[n.index("combine_kernel<"):n.index(">", n.index("combine_kernel<")) + 1]
        elif "read_probe_kernel" in n:
            name = "read_probe_kernel"
        else:
            continue
        wgs = int(r["Grid_Size"]) // int(r["Workgroup_Size"])
        agg[(name, wgs)][r["Counter_Name"]].append(float(r["Counter_Value"]))
    o = ["# split_kernel instruction- and scalar-cache counters (sweep, 1K and 64K)", "",
         f"kernel source sha256[:16]: {kernel_hash()}", "",
         f"command: rocprofv3 --pmc {IC_COUNTERS} -f csv -d <dir>/pmc_ic -o ic -- {py} --steps 2 --warmup 0 "
         "--kernel-reps 4 --no-cpu-baseline --ctx 1024 --ctx 65536", "",
         "Whole-GPU totals per dispatch, averaged over the dispatches of each kernel and grid (the SQC "
         "counters are summed over every instruction and scalar cache).", "",
         "| kernel | workgroups | dispatches | I-cache misses | per workgroup | I-cache hits | duplicate misses "
         "| K-cache misses | K-cache hits |", "|---|---|---|---|---|---|---|---|---|"]
    for (name, wgs), v in sorted(agg.items()):
        a = {c: sum(x) / len(x) for c, x in v.items()}
        o.append(f"| {name} | {wgs} | {len(v['SQ_WAVES'])} | {a['SQC_ICACHE_MISSES']:.0f} | "
                 f"{a['SQC_ICACHE_MISSES'] / wgs:.1f} | {a['SQC_ICACHE_HITS']:.0f} | "
                 f"{a['SQC_ICACHE_MISSES_DUPLICATE']:.0f} | {a['SQC_DCACHE_MISSES']:.0f} | {a['SQC_DCACHE_HITS']:.0f} |")
    name = os.path.join(ROOT, "profiles", "split_kernel_icache.md")
    open(name, "w").write("\n".join(o) + "\n")
    print(f"wrote {name}")



def phase_table(d, py):
    """profiles/split_kernel_phases.md from the `--phases` run (phases.log)."""
    path = os.path.join(d, "phases.log")
    if not os.path.exists(path):
        return
    line = None
    for x in open(path):
        if x.startswith("{") and '"phases"' in x:
            line = json.loads(x)
    if line is None:
        raise SystemExit("no phases line in phases.log")
    if line["kernel_hash"] != kernel_hash():
        raise SystemExit("phase records of another kernel source")
    cols = [("splits", "splits"), ("chunks_per_split", "chunks / split"), ("entry_spread", "entry spread"),
            ("args", "args"), ("first_dma_issued", "1st DMA issued"), ("chunk0_in_lds", "chunk 0 in LDS"),
            ("step", "chunk step"), ("barrier_share", "barrier share of steps"),
            ("last_step_issued", "last step issued"), ("partials_written", "partials written"),
            ("split_span", "split span"), ("gap_to_combine", "gap to combine"), ("comb_args", "comb args"),
            ("comb_first_batch", "comb 1st batch"), ("comb_folded", "comb folded"),
            ("comb_written", "comb written"), ("comb_span", "comb span"), ("pair_span", "pair span"),
            ("us_per_call", "us / call, 4-call graphs"), ("waits", "barrier wait per step: consumers c0.. / producer (its DMA wait) / decoder (converting)")]
    o = ["# split_kernel / combine_kernel phases (trace build, per-workgroup clock stamps)", "",
         f"kernel source sha256[:16]: {line['kernel_hash']}", "",
         f"command: {py} --phases", "",
         "The trace build (lib/libverify_attn_trace.so, the same sources compiled with VA_PHASE_TRACE) stores "
         "the 100 MHz constant-rate GPU clock (s_memrealtime, common to all CUs) at phase boundaries, one record "
         "per workgroup (include/verify_probe.h). Each case replays graphs of 4 back-to-back split + combine "
         "calls over cold replicas and reads the records of the last pair; values are medians over 12 replays, "
         "in us. Per-workgroup phases are means over workgroups and measured from that workgroup's entry "
         "(args, 1st DMA issued, chunk 0 in LDS, comb args / 1st batch / folded / written); 'chunk step' "
         "is (last step issued - chunk 0 in LDS) / chunks (the span holds every chunk's step); 'barrier "
         "share' is consumer wave 0's time at barriers over that span; 'barrier wait per step' is each role's time at the later barriers (consumer waves in order, "
         "the first producer wave, with its wait for its DMA in brackets, the first decoder wave, with its "
         "conversion time per chunk in brackets) per step: the role that waits least at the barriers holds the step; 'last step issued', 'partials written' (wave 0) and the spans are from the first "
         "workgroup's entry; 'gap to combine' runs from the last split workgroup's partials to the first combine "
         "workgroup's entry. 'us / call' divides the event time of the 6 graph replays by their 24 calls, graph "
         "launches included (longer than back-to-back calls of one long graph).", "",
         "| case | " + " | ".join(c[1] for c in cols) + " |", "|---" * (len(cols) + 1) + "|"]
    for c in line["phases"]:
        nw = sum(1 for k in c if k.startswith("wait_c"))
        c = dict(c, waits=", ".join(f"{c[f'wait_c{w}']:.3f}" for w in range(nw))
                 + f" / {c['wait_prod']:.3f} ({c['dma_prod']:.3f})"
                 + (f" / {c['wait_dec']:.3f} ({c['conv_dec']:.3f})" if "wait_dec" in c else ""))
        o.append(f"| {c['case']} | " + " | ".join(str(c.get(k)) for k, _ in cols) + " |")
    name = os.path.join(ROOT, "profiles", "split_kernel_phases.md")
    open(name, "w").write("\n".join(o) + "\n")
    print(f"wrote {name}")


def sample_hash():
    with open(SAMPLE_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def summarize_profiles(d):
    """Turn the rocprofv3 outputs of one profiling session into the committed
    summaries: kernel durations (kernel trace) and HBM bytes per split launch
    (FETCH_SIZE and WRITE_SIZE, each scaled by what the counter reads for a
    plain copy of known size).  `d` holds trace/, pmc_fetch/, pmc_write/,
    pmc_copy_fetch/, pmc_copy_write/ and the bench logs trace.log, fetch.log,
    write.log written by the commands listed in the summaries.  Each summary
    is written only when its own runs are in `d` (the sampler's from
    trace_sampler/ and sampler_trace.log, the KV write's from trace_kvw/ and
    kvw.log), so one part can be refreshed alone."""
    import csv
    import collections

    def kname(n):
        """Kernel name without spaces; split_kernel's last two template
        arguments, the fused append and the row groups, become ",append"
        when set and ",rows2" for two row groups, and are dropped otherwise."""
        n = n.replace(" ", "")
        if "split_kernel<" in n:
            i = n.index("split_kernel<") + len("split_kernel<")
            j = n.index(">", i)
            args = n[i:j].split(",")
            if len(args) >= 7:  # earlier sources have no row-group argument
                args = (args[:6] + (["append"] if args[6] == "true" else [])
                        + ([f"rows{args[7]}"] if len(args) > 7 and args[7] != "1" else []))
            n = n[:i] + ",".join(args) + n[j:]
        return n

    def bench_line(log):
        for line in open(os.path.join(d, log)):
            if line.startswith("{") and '"metric"' in line:
                return json.loads(line)
        raise SystemExit(f"no bench line in {log}")

    def counters(sub, name):
        rows = list(csv.DictReader(open(os.path.join(d, sub, name))))
        return [(r["Kernel_Name"], int(r["Grid_Size"]) // int(r["Workgroup_Size"]), float(r["Counter_Value"]))
                for r in rows]

    py = "python -u bench.py"
    # the attention sweep's summaries need its kernel trace and traffic runs;
    # the sampler and kv-write summaries below need only their own runs
    if os.path.exists(os.path.join(d, "trace.log")):
        hashes = {bench_line(x)["kernel_hash"] for x in ("trace.log", "fetch.log", "write.log")}
        if len(hashes) != 1 or kernel_hash() not in hashes:
            raise SystemExit(f"profiles were taken of another kernel source: {hashes} vs {kernel_hash()}")
        copy_bytes = COPY_PROBE_MIB << 20
        cf = [v for n, g, v in counters("pmc_copy_fetch", "copy_counter_collection.csv") if "copyBuffer" in n]
        cw = [v for n, g, v in counters("pmc_copy_write", "copy_counter_collection.csv") if "copyBuffer" in n]
        f_scale = copy_bytes / (sum(cf) / len(cf) * 1024)
        w_scale = copy_bytes / (sum(cw) / len(cw) * 1024)
        def static_split(n):  # the sweep's kernel: static plan, D 128, 3 consumer waves, bf16
            return "split_kernel<128,3,0,4,2,false>" in kname(n)

        fe = [(g, v) for n, g, v in counters("pmc_fetch", "bench_counter_collection.csv") if static_split(n)]
        wr = [(g, v) for n, g, v in counters("pmc_write", "bench_counter_collection.csv") if static_split(n)]
        if len(fe) != len(wr):
            raise SystemExit("fetch and write runs saw different split launches")
        per_launch = [f * f_scale * 1024 + w * w_scale * 1024 for (_, f), (_, w) in zip(fe, wr)]
        traffic = sum(per_launch) / len(per_launch)
        contexts = bench_line("fetch.log")["config"]["contexts"]
        splits = [e["splits"] for e in bench_line("fetch.log")["sweep"]]
        json.dump({"kernel_hash": kernel_hash(), "contexts": contexts, "splits": splits,
                   "hbm_bytes_per_launch": round(traffic),
                   "fetch_scale": round(f_scale, 4), "write_scale": round(w_scale, 4), "launches": len(per_launch)},
                  open(TRAFFIC_FILE, "w"), indent=1)

        trace = list(csv.DictReader(open(os.path.join(d, "trace", "bench_kernel_trace.csv"))))
        dur = collections.defaultdict(list)
        for r in trace:
            n = kname(r["Kernel_Name"])
            kind = ("split_kernel" if "split_kernel" in n else "combine_kernel" if "combine_kernel" in n
                    else "read_probe_kernel" if "read_probe_kernel" in n else None)
            if kind and "<" in n:
                kind += n[n.index("<"):n.index(">") + 1].replace(" ", "")
            if kind:
                dur[(kind, n, trace_workgroups(r))].append(
                    (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1000.0)
        bl = bench_line("trace.log")
        out = []
        out.append("# split_kernel / combine_kernel, full-attention verify sweep (Hkv 1, Hq 6, D 128, 8 rows, ctx 1K-192K)")
        out.append("")
        out.append(f"kernel source sha256[:16]: {kernel_hash()}")
        out.append("")
        out.append("## Kernel durations (rocprofv3 kernel trace)")
        out.append("")
        out.append(f"command: rocprofv3 --kernel-trace --stats -f csv -d <dir>/trace -o bench -- {py} --steps 10 --warmup 3")
        out.append("")
        out.append("| kernel | workgroups | launches | avg us | min us | max us |")
        out.append("|---|---|---|---|---|---|")
        tot = collections.defaultdict(list)
        for (kind, n, wgs), v in sorted(dur.items(), key=lambda x: (x[0][0], x[0][2])):
            tot[kind] += v
            out.append(f"| {kind} | {wgs} | {len(v)} | {sum(v) / len(v):.2f} | {min(v):.2f} | {max(v):.2f} |")
        for kind in ("split_kernel", "combine_kernel"):
            for flag, label in (("false>", "static plan"), ("true>", "device state")):
                v = [x for k, x in tot.items() if k.startswith(kind) and k.endswith(flag) for x in x]
                if v:
                    out.append(f"| {kind} ({label}, all) | all | {len(v)} | {sum(v) / len(v):.2f} | {min(v):.2f} "
                               f"| {max(v):.2f} |")
        v = tot.get("read_probe_kernel")
        if v:
            out.append(f"| read_probe_kernel (plain read of the same bytes, all) | all | {len(v)} | "
                       f"{sum(v) / len(v):.2f} | {min(v):.2f} | {max(v):.2f} |")
        out.append("")
        out.append("bench line of the same command (events; the trace itself slows the launches): "
                   f"roofline avg_launch_us {bl['roofline']['avg_launch_us']}, value {bl['value']} GB/s")
        sw = [x for (kind, n, wgs), v in dur.items() if static_split(n) for x in v]
        line = (f"roofline kernel (sweep split launches, static plan, D 128, 3 consumers): trace average "
                f"{sum(sw) / len(sw):.2f} us over {len(sw)} launches")
        if os.path.exists(os.path.join(d, "bench.log")):
            pl = bench_line("bench.log")
            if pl["kernel_hash"] == kernel_hash():
                line += (f"; the same bench without the profiler ({py} --steps 10 --warmup 3): avg_launch_us "
                         f"{pl['roofline']['avg_launch_us']}, value {pl['value']} GB/s")
        out.append("")
        out.append(line)
        out.append("")
        out.append("## HBM traffic of split_kernel (rocprofv3 --pmc, one counter per run)")
        out.append("")
        out.append(f"command: rocprofv3 --pmc FETCH_SIZE -f csv -d <dir>/pmc_fetch -o bench -- {py} --steps 2 --warmup 0 --kernel-reps 4 --no-cpu-baseline")
        out.append(f"command: rocprofv3 --pmc WRITE_SIZE -f csv -d <dir>/pmc_write -o bench -- {py} --steps 2 --warmup 0 --kernel-reps 4 --no-cpu-baseline")
        out.append(f"calibration: rocprofv3 --pmc FETCH_SIZE|WRITE_SIZE ... -- {py} --copy-probe {COPY_PROBE_MIB}"
                   f" (device copy of {COPY_PROBE_MIB} MiB: FETCH_SIZE reads {sum(cf) / len(cf):.0f} KiB,"
                   f" WRITE_SIZE {sum(cw) / len(cw):.0f} KiB -> scale {f_scale:.4f} / {w_scale:.4f})")
        out.append("")
        out.append("| workgroups | launches | FETCH_SIZE KiB | WRITE_SIZE KiB | HBM bytes (scaled) |")
        out.append("|---|---|---|---|---|")
        byg = collections.defaultdict(list)
        for (g, f), (_, w) in zip(fe, wr):
            byg[g].append((f, w))
        for g in sorted(byg):
            v = byg[g]
            fa = sum(x[0] for x in v) / len(v)
            wa = sum(x[1] for x in v) / len(v)
            out.append(f"| {g} | {len(v)} | {fa:.1f} | {wa:.1f} | {(fa * f_scale + wa * w_scale) * 1024:.0f} |")
        out.append("")
        out.append(f"mean HBM bytes per split launch over the sweep: {traffic:.0f}"
                   f" (algorithmic KV bytes per launch: {bl['roofline']['algorithmic_bytes_per_launch']})")

        up = os.path.join(d, "pmc_util", "bench_counter_collection.csv")
        if os.path.exists(up):
            if bench_line("util.log")["kernel_hash"] != kernel_hash():
                raise SystemExit("utilisation counters of another kernel source")
            # Counter values are whole-GPU totals per dispatch (SQ_INSTS_MFMA of
            # the 33-workgroup launch is exactly 33 x 3 waves x 16).  Busy
            # fractions divide by the kernel-trace duration of the same kernel
            # and grid at the 2.4 GHz peak clock (a lower bound if the clock ran
            # lower); GRBM_GUI_ACTIVE is not used, since under --pmc it also
            # counts the serialised launch around each dispatch.
            kinds = [("split_kernel<128,3,0,4,2,false>", "split: sweep (D 128, 3 consumers, bf16)"),
                     ("split_kernel<64,3,0,8,2,false>", "split: window ring (D 64, 3 consumers)"),
                     ("split_kernel<128,6,0,4,2,false>", "split: tree (D 128, 6 consumers, bf16)"),
                     ("split_kernel<128,3,0,4,2,false,rows2>", "split: tree, two row groups (3 consumers each)"),
                     ("split_kernel<128,6,1,8,1,false>", "split: quantised tree (6 consumers, 2 decoders)")]
            tdur = collections.defaultdict(list)
            for (kind, n, wgs), v in dur.items():
                tdur[(kind, wgs)] += v
            vals = collections.defaultdict(lambda: collections.defaultdict(list))
            for r in csv.DictReader(open(up)):
                n = kname(r["Kernel_Name"])
                wgs = int(r["Grid_Size"]) // int(r["Workgroup_Size"])
                for key, _ in kinds:
                    if key in n:
                        vals[(key, wgs)][r["Counter_Name"]].append(float(r["Counter_Value"]))
            out += ["", "## MFMA and LDS activity of split_kernel (rocprofv3 --pmc, one run)", "",
                    f"command: rocprofv3 --pmc {UTIL_COUNTERS} -f csv -d <dir>/pmc_util -o bench -- {py} --steps 2 "
                    "--warmup 0 --kernel-reps 4 --no-cpu-baseline", "",
                    "MFMA busy % = SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x trace duration x 2.4 GHz); MFMA TFLOP/s = "
                    "SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512 / trace duration; LDS conflict = SQ_LDS_BANK_CONFLICT / "
                    "(SQ_LDS_IDX_ACTIVE - SQ_LDS_BANK_CONFLICT).", "",
                    "| kernel | workgroups | dispatches | MFMA per dispatch | trace us | MFMA busy % | MFMA TFLOP/s | "
                    "LDS conflict |", "|---|---|---|---|---|---|---|---|"]
            summary = {}
            tot_busy = tot_us = 0.0
            for key, label in kinds:
                for (k2, wgs) in sorted(x for x in vals if x[0] == key):
                    v = vals[(k2, wgs)]
                    t = tdur.get((key, wgs))
                    if not t or not v.get("SQ_VALU_MFMA_BUSY_CYCLES"):
                        continue
                    us = sum(t) / len(t)
                    busy = sum(v["SQ_VALU_MFMA_BUSY_CYCLES"]) / len(v["SQ_VALU_MFMA_BUSY_CYCLES"])
                    mops = sum(v["SQ_INSTS_VALU_MFMA_MOPS_BF16"]) / len(v["SQ_INSTS_VALU_MFMA_MOPS_BF16"])
                    ninst = sum(v["SQ_INSTS_MFMA"]) / len(v["SQ_INSTS_MFMA"])
                    conf = sum(v["SQ_LDS_BANK_CONFLICT"])
                    act = sum(v["SQ_LDS_IDX_ACTIVE"])
                    pct = 100 * busy / (1024 * us * 1e-6 * 2.4e9)
                    tf = mops * 512 / (us * 1e-6) / 1e12
                    lc = conf / (act - conf) if act > conf else 0.0
                    out.append(f"| {label} | {wgs} | {len(v['SQ_VALU_MFMA_BUSY_CYCLES'])} | {ninst:.0f} | {us:.2f} | "
                               f"{pct:.1f} | {tf:.1f} | {lc:.3f} |")
                    summary[f"{key}@{wgs}"] = {"mfma_busy_pct": round(pct, 2), "mfma_tflops": round(tf, 1),
                                               "lds_conflict": round(lc, 4)}
                    if key == kinds[0][0]:
                        tot_busy += busy * len(t)
                        tot_us += us * len(t)
            if tot_us:
                sweep_pct = 100 * tot_busy / (1024 * tot_us * 1e-6 * 2.4e9)
                out += ["", f"sweep kernel, launches weighted as in the trace: MFMA busy {sweep_pct:.1f}%"]
                json.dump({"kernel_hash": kernel_hash(), "kernel": kinds[0][0], "mfma_busy_pct": round(sweep_pct, 2),
                           "clock_ghz": 2.4, "by_kernel": summary}, open(UTIL_FILE, "w"), indent=1)
        name = os.path.join(ROOT, "profiles", "split_kernel_verify_sweep.md")
        open(name, "w").write("\n".join(out) + "\n")
        print(f"wrote {name} and {TRAFFIC_FILE}")

    wave_cycles(d, kname, py)
    phase_table(d, py)
    icache_table(d, kname, py)

    st = os.path.join(d, "trace_sampler", "sampler_kernel_trace.csv")
    if os.path.exists(st):
        rows = [r for r in csv.DictReader(open(st)) if "sample_kernel" in r["Kernel_Name"] or
                "accept_kernel" in r["Kernel_Name"]]
        by = collections.defaultdict(list)
        for r in rows:
            n = r["Kernel_Name"]
            i = n.index("sample_detail::") + len("sample_detail::")
            name = n[i:n.index("(") if "(" in n else len(n)].replace(" ", "")
            wgs = trace_workgroups(r)
            by[(name, wgs)].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1000.0)

        def sampler_line(log):
            for line in open(os.path.join(d, log)):
                if line.startswith("{") and "va_sample_accept" in line:
                    return json.loads(line)
            raise SystemExit(f"no sampler line in {log}")
        sl = sampler_line("sampler_trace.log")
        if sl["kernel_hash"] != sample_hash():
            raise SystemExit("sampler profile of another kernel source")
        o = ["# sample_kernel, sampling of 8 verification rows and acceptance of 7 drafts "
             "(top-k 20, top-p 0.95, FP32 logits)", "",
             f"kernel source sha256[:16]: {sample_hash()}", "",
             f"command: rocprofv3 --kernel-trace --stats -f csv -d <dir>/trace_sampler -o sampler -- {py} --sampler "
             "--no-cpu-baseline", "",
             "workgroups = tiles x rows: 160 for the 160,000-token vocabulary, 24 for the 20,000-token share; "
             "<true> runs the acceptance in the last row.", "",
             "| kernel | workgroups | launches | avg us | min us | max us |", "|---|---|---|---|---|---|"]
        for (name, wgs), v in sorted(by.items()):
            if len(v) < 10:
                continue  # the single eager calls before capture
            o.append(f"| {name} | {wgs} | {len(v)} | {sum(v) / len(v):.2f} | {min(v):.2f} | {max(v):.2f} |")
        o += ["", "bench line of the same command (graph replay, events):", ""]
        for c in sl["cases"]:
            o.append(f"- {c['case']} (V = {c['vocab']}): sample + accept {c['us_per_call']} us, sample only "
                     f"{c['sample_only_us']} us per call; logits {c['logit_bytes']} bytes")
        plain = os.path.join(d, "sampler.log")
        if os.path.exists(plain):
            pl = sampler_line("sampler.log")
            o += ["", f"the same without the profiler ({py} --sampler):", ""]
            for c in pl["cases"]:
                cb = c.get("cpu_baseline")
                o.append(f"- {c['case']}: {c['us_per_call']} us per call (sample only {c['sample_only_us']} us)"
                         + (f"; oracle {cb['value']} us per call on one host thread" if cb else ""))
        sname = os.path.join(ROOT, "profiles", "sample_kernel_sampling_acceptance.md")
        open(sname, "w").write("\n".join(o) + "\n")
        print(f"wrote {sname}")

    kt = os.path.join(d, "trace_kvw", "kvw_kernel_trace.csv")
    if os.path.exists(kt):
        rows = [r for r in csv.DictReader(open(kt)) if "kv_write_kernel" in r["Kernel_Name"]]
        by = collections.defaultdict(list)
        for r in rows:
            n = r["Kernel_Name"]
            by[n[n.index("kv_write_kernel"):n.index(">") + 1].replace(" ", "")].append(
                (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1000.0)
        kl = None
        for line in open(os.path.join(d, "kvw.log")):
            if line.startswith("{") and "verify_kv_write" in line:
                kl = json.loads(line)
        if kl is None or kl["kernel_hash"] != kernel_hash():
            raise SystemExit("kv-write profile missing or of another kernel source")
        o = ["# kv_write_kernel, the rows' KV written before the read (window ring bf16; tree cache E4M3 + INT8)", "",
             f"kernel source sha256[:16]: {kernel_hash()}", "",
             f"command: rocprofv3 --kernel-trace --stats -f csv -d <dir>/trace_kvw -o kvw -- {py} --kv-write", "",
             "| kernel | launches | avg us | min us | max us |", "|---|---|---|---|---|"]
        for k, v in sorted(by.items()):
            o.append(f"| {k} | {len(v)} | {sum(v) / len(v):.2f} | {min(v):.2f} | {max(v):.2f} |")
        o += ["", "bench line of the same command (graph replay, events; slowed by the trace):", ""]
        for c in kl["cases"]:
            o.append(f"- {c['case']}: {c['rows']} rows x {c['kv_heads']} KV heads x D {c['head_dim']}: "
                     f"{c['us_per_call']} us per call, {c['bytes_per_call']} bytes moved")
        plain = os.path.join(d, "kvw_plain.log")
        if os.path.exists(plain):
            for line in open(plain):
                if line.startswith("{") and "verify_kv_write" in line:
                    pl = json.loads(line)
                    o += ["", f"the same without the profiler ({py} --kv-write):", ""]
                    for c in pl["cases"]:
                        o.append(f"- {c['case']}: {c['us_per_call']} us per call")
        kname = os.path.join(ROOT, "profiles", "kv_write_kernel_ring_and_tree_cache.md")
        open(kname, "w").write("\n".join(o) + "\n")
        print(f"wrote {kname}")


def bench_kv_write(torch, va, synth, dev, reps=200):
    """Time verify_kv_write at the configurations that write rows before the
    read: the window ring (bf16, 8 rows, 1 KV head, D 64, 4160 slots) and the
    quantised tree cache (16 rows, 4 KV heads, D 128, at a 64K prefix), from a
    graph of back-to-back launches.  Prints one JSON line (not the sweep's)."""
    cases = []
    g = synth.gen(9100)
    for name, rows, hkv, d, quant, first_pos, ring in (
            ("window ring, bf16", 8, 1, 64, False, 194560, 4160),
            ("tree cache, E4M3 keys + INT8 values", 16, 4, 128, True, 65536, 0)):
        k_new = synth.normal_bf16((rows, hkv, d), g).to(dev)
        v_new = synth.normal_bf16((rows, hkv, d), g).to(dev)
        slots = ring if ring else first_pos + rows + 64
        if quant:
            kc = torch.zeros((hkv, slots, d), dtype=torch.uint8, device=dev)
            vc = torch.zeros((hkv, slots, d), dtype=torch.int8, device=dev)
            vs = torch.zeros((hkv, slots), dtype=torch.float32, device=dev)
            moved = rows * hkv * (2 * d * 2 + 2 * d + 4)   # bf16 rows in, codes + scale out
        else:
            kc = torch.zeros((hkv, slots, d), dtype=torch.bfloat16, device=dev)
            vc = torch.zeros((hkv, slots, d), dtype=torch.bfloat16, device=dev)
            vs = None
            moved = rows * hkv * 2 * d * 2 * 2             # bf16 rows in and out
        cases.append((name, rows, hkv, d, first_pos, ring, k_new, v_new, kc, vc, vs, moved))
    out = []
    for name, rows, hkv, d, first_pos, ring, k_new, v_new, kc, vc, vs, moved in cases:
        def launches():
            for _ in range(reps):
                va.verify_kv_write(k_new, v_new, first_pos, kc, vc, v_scale=vs, ring_slots=ring,
                                   stream=torch.cuda.current_stream())
        launches()
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr):
            launches()
        gr.replay()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        gr.replay()
        b.record()
        torch.cuda.synchronize()
        us = a.elapsed_time(b) * 1e3 / reps
        out.append({"case": name, "rows": rows, "kv_heads": hkv, "head_dim": d, "us_per_call": round(us, 3),
                    "bytes_per_call": moved, "gb_s": round(moved / (us * 1e-6) / 1e9, 2)})
    print(json.dumps({"metric": "verify_kv_write us/call", "unit": "us", "higher_is_better": False,
                      "launch": "HIP graph replay, back to back", "cases": out,
                      "kernel_hash": kernel_hash()}), flush=True)


def bench_sampler(torch, va, synth, dev, reps=100, replicas=4, cpu_seconds=5.0, cpu=True):
    """Sampling of 8 verification rows (top-k 20, top-p 0.95, temperature 1)
    plus acceptance of their 7 drafts, over the full 160,000-token vocabulary
    and over a 20,000-token share, with FP32 logits resident in HBM
    (`replicas` copies read in turn).  The draft's lists come from va_sample
    on perturbed logits (untimed).  A third case takes the target's own
    lists and samples as the drafts (q = p, so every draft is accepted: the
    acceptance walks all rows).  Timed from graphs of back-to-back calls;
    the full-size outputs of replica 0 are checked against the oracle.
    Prints one JSON line (not the sweep's)."""
    import numpy as np
    from oracle import sampling as osamp
    n, k, top_p, seed, pos0 = 8, 20, 0.95, 20260, 123456
    out = []
    for name, V, all_accepted in (("full vocabulary", 160000, False), ("one GPU's share of eight", 20000, False),
                                  ("full vocabulary, every draft accepted", 160000, True)):
        g = synth.gen(9300 + V)
        zs = [synth.logits_f32(n, V, g, "lm") for _ in range(replicas)]
        if all_accepted:
            zs = [zs[0].clone() for _ in range(replicas)]
        zd = zs[0][: n - 1] + 0.5 * torch.randn((n - 1, V), generator=g)
        zg = [z.to(dev) for z in zs]
        if all_accepted:
            dr = va.va_sample(zg[0], seed=seed, first_position=pos0)
        else:
            dr = va.va_sample(zd.to(dev), seed=seed, first_position=pos0, purpose=3)
        q = (dr["ids"][: n - 1].contiguous(), dr["probs"][: n - 1].contiguous(), dr["kept"][: n - 1].contiguous(),
             dr["tokens"][: n - 1].contiguous())
        p = va.sample_params(n, V, top_k=k, top_p=top_p, seed=seed, first_position=pos0)
        ws = va.sample_workspace_for(p, dev)
        o = dict(ids=torch.empty((n, k), dtype=torch.int32, device=dev),
                 probs=torch.empty((n, k), dtype=torch.float32, device=dev),
                 kept=torch.empty(n, dtype=torch.int32, device=dev),
                 tokens=torch.empty(n, dtype=torch.int32, device=dev))
        acc = torch.empty(1, dtype=torch.int32, device=dev)
        toks = torch.empty(n, dtype=torch.int32, device=dev)

        def fused(i):
            va.va_sample_accept(zg[i % replicas], *q, top_k=k, top_p=top_p, seed=seed, first_position=pos0,
                                workspace=ws, out=o, accepted=acc, out_tokens=toks,
                                stream=torch.cuda.current_stream())

        def sample_only(i):
            va.va_sample(zg[i % replicas], top_k=k, top_p=top_p, seed=seed, first_position=pos0, workspace=ws,
                         out=o, stream=torch.cuda.current_stream())
        # full-size check of replica 0 against the oracle (decisions away from their margins)
        fused(0)
        torch.cuda.synchronize()
        res = {kk: v.cpu().numpy() for kk, v in o.items()}
        t0 = time.perf_counter()
        ref = osamp.sample(zs[0].double().numpy(), k, float(np.float32(top_p)), 1.0, seed, pos0, 0)
        qn = [x.cpu().numpy() for x in q]
        a_ref, t_ref, margin = osamp.accept(res["ids"], res["probs"], res["kept"], res["tokens"], *qn, n, seed,
                                            pos0)
        t_oracle = time.perf_counter() - t0
        ok = all(np.array_equal(res["ids"][r], ref[r]["ids"]) for r in range(n))
        ok = ok and all(int(res["tokens"][r]) == ref[r]["token"] for r in range(n)
                        if ref[r]["topp_margin"] > 1e-5 and ref[r]["draw_margin"] > 1e-5)
        ok = ok and (margin <= 1e-6 or (int(acc.item()) == a_ref and list(toks.cpu().numpy()[: a_ref + 1]) == t_ref))
        times = {}
        for label, fn in (("sample_accept", fused), ("sample", sample_only)):
            def launches(fn=fn):
                for i in range(reps):
                    fn(i)
            launches()
            gr = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gr):
                launches()
            gr.replay()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            gr.replay()
            b.record()
            torch.cuda.synchronize()
            times[label] = a.elapsed_time(b) * 1e3 / reps
            del gr
        nbytes = n * V * 4
        case = {"case": name, "rows": n, "vocab": V, "top_k": k, "top_p": top_p, "drafts": n - 1,
                "us_per_call": round(times["sample_accept"], 3), "sample_only_us": round(times["sample"], 3),
                "logit_bytes": nbytes, "logit_gb_s": round(nbytes / (times["sample_accept"] * 1e-6) / 1e9, 1),
                "pct_hbm_peak": round(100 * nbytes / (times["sample_accept"] * 1e-6) / 1e9 / HBM_PEAK_GBS, 2),
                "parity": {"pass": bool(ok), "accepted": int(acc.item())}}
        if all_accepted and int(acc.item()) != n - 1:
            raise SystemExit("the every-draft-accepted case did not accept every draft")
        if cpu:
            passes, t_cpu = 1, t_oracle
            while t_cpu < cpu_seconds and passes < 50:
                t0 = time.perf_counter()
                osamp.sample(zs[passes % replicas].double().numpy(), k, float(np.float32(top_p)), 1.0, seed, pos0, 0)
                osamp.accept(res["ids"], res["probs"], res["kept"], res["tokens"], *qn, n, seed, pos0)
                t_cpu += time.perf_counter() - t0
                passes += 1
            case["cpu_baseline"] = {"value": round(t_cpu / passes * 1e6, 1), "unit": "us/call", "cores": 1,
                                    "kind": "oracle", "sample": f"{passes} calls, float64 numpy"}
        out.append(case)
    print(json.dumps({"metric": "va_sample_accept us/call (8 rows, 7 drafts, top-k 20, top-p 0.95)", "unit": "us",
                      "higher_is_better": False, "launch": "HIP graph replay, back to back", "cases": out,
                      "kernel_hash": sample_hash()}), flush=True)


def bench_other_configs(torch, va, synth, dev, reps=200, replicas=4):
    """The other configurations of the verification call, each timed as one
    call (ring write where the rows' K/V go to the ring first, split,
    combine) from a graph of `reps` back-to-back calls over cold caches (at
    least `replicas` and at least 1 GiB of them, read in turn):
      window  Hkv 1, Hq 6, D 64, 8 rows (5 live), window 4,096 over a
              4,160-slot ring, rows at 5,120 / 51,200 / 194,560, sink on;
      tree    Hkv 4, Hq 24, D 128, a 16-node random tree over a 2K / 8K /
              32K prefix, no sink;
      tree-q  the same tree over a 64K prefix, keys E4M3 after the rotation,
              values INT8 with an FP32 scale per (token, head).
    KV bytes are the algorithmic read (visible keys once per KV head).
    Window and bf16 tree calls are also timed with the rows' KV write inside
    the split launch (verify_attn_split_append: us_per_call_append_fused),
    and tree calls with the write as a launch of its own
    (us_per_call_with_kv_write); the tree's plain call reads a cache that
    already holds the node keys."""
    out = []
    g = synth.gen(9500)
    cases = []
    for t0 in (5120, 51200, 194560):
        cases.append(("window", dict(rows=8, live_rows=5, q_heads=6, kv_heads=1, head_dim=64, mask="window",
                                     first_pos=t0, window=4096, ring_slots=4160), t0))
    for P in (2048, 8192, 32768):
        cases.append(("tree", dict(rows=16, live_rows=16, q_heads=24, kv_heads=4, head_dim=128, mask="tree",
                                   prefix_len=P, parent=synth.random_tree(16, g), kv_capacity=P + 16 + 64), P))
    cases.append(("tree-q", dict(rows=16, live_rows=16, q_heads=24, kv_heads=4, head_dim=128, mask="tree",
                                 kv_fmt="e4m3_wht_i8", prefix_len=65536, parent=synth.random_tree(16, g),
                                 kv_capacity=65536 + 16 + 64), 65536))
    cur = torch.cuda.current_stream
    for kind, kw, pos in cases:
        plan = va.Plan(**kw)
        hkv, d, rows, hq = kw["kv_heads"], kw["head_dim"], kw["rows"], kw["q_heads"]
        slots = kw.get("ring_slots") or kw["kv_capacity"]
        quant = kind == "tree-q"
        lo, hi = plan.info["lo"], plan.info["hi"]
        kv_bytes = hkv * (hi - lo) * ((2 * d + 4) if quant else 4 * d)
        q = synth.normal_bf16((rows, hq, d), g).to(dev)
        sink = synth.normal_f32((hq,), g).to(dev) if kind == "window" else None
        # replicas of the cache (K, V and, quantised, the scales) in one pool
        # of at least 1 GiB, read in turn
        esz = 1 if quant else 2
        kvb = hkv * slots * d * esz
        per = 2 * kvb + (hkv * slots * 4 if quant else 0)
        nrep = max(replicas, -(-POOL_BYTES // per))
        n = nrep
        pool = torch.empty(n * per, dtype=torch.uint8, device=dev)
        if quant:
            kv_all = pool.view(n, per)
            kv_all[:, :kvb] = torch.randint(0, 126, (n, kvb), dtype=torch.uint8, device=dev)
            kv_all[:, kvb:2 * kvb] = torch.randint(-127, 128, (n, kvb), dtype=torch.int8, device=dev).view(torch.uint8)
            kv_all[:, 2 * kvb:] = (torch.rand((n, hkv * slots), device=dev) * 0.02).view(torch.uint8)
        else:
            flat = pool.view(torch.bfloat16)
            piece = 1 << 27
            for off in range(0, flat.numel(), piece):
                m = min(piece, flat.numel() - off)
                flat[off:off + m] = synth.normal_bf16_device((m,), 7000 + pos % 997 + off // piece, dev)
        reps_kv = []
        for r in range(n):
            base = pool[r * per:(r + 1) * per]
            if quant:
                k = base[:kvb].view(hkv, slots, d)
                v = base[kvb:2 * kvb].view(torch.int8).view(hkv, slots, d)
                vs = base[2 * kvb:].view(torch.float32).view(hkv, slots)
            else:
                kv = base.view(torch.bfloat16).view(2, hkv, slots, d)
                k, v, vs = kv[0], kv[1], None
            reps_kv.append((k, v, vs))
        k_new = synth.normal_bf16((rows, hkv, d), g).to(dev)
        v_new = synth.normal_bf16((rows, hkv, d), g).to(dev)
        ws = va.workspace_for(plan, dev)
        o = torch.empty((rows, hq, d), dtype=torch.float32, device=dev)
        lse = torch.empty((rows, hq), dtype=torch.float32, device=dev)

        def one(i, split_only=False, fused=False, write=False):
            k, v, vs = reps_kv[i % nrep]
            if fused:  # the rows' KV write inside the split launch
                va.verify_attn_split_append(plan, q, k_new, v_new, k, v, ws, stream=cur())
            else:
                if kind == "window" and not split_only:
                    va.swa_ring_write(k_new, v_new, pos, k, v, stream=cur())
                if write:  # the tree's node keys written first, a launch of their own
                    va.verify_kv_write(k_new, v_new, pos, k, v, stream=cur())
                va.verify_attn_split(plan, q, k, v, ws, v_scale=vs, stream=cur())
            if not split_only:
                va.verify_attn_combine(plan, ws, o, lse=lse, sink=sink, stream=cur())
        times = {}
        passes = [("call", False, False, False), ("split", True, False, False)]
        if kind == "tree":
            passes.append(("write_call", False, False, True))
        if kind in ("window", "tree"):
            passes.append(("fused", False, True, False))
        for label, so, fu, wr in passes:
            for i in range(2):
                one(i, so, fu, wr)
            gr = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gr):
                for i in range(reps):
                    one(i, so, fu, wr)
            gr.replay()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            gr.replay()
            b.record()
            torch.cuda.synchronize()
            times[label] = a.elapsed_time(b) * 1e3 / reps
            del gr
        extra = {}
        if "write_call" in times:  # verify_kv_write + split + combine
            extra["us_per_call_with_kv_write"] = round(times["write_call"], 2)
        if "fused" in times:  # verify_attn_split_append + combine: the KV write inside the split launch
            extra["us_per_call_append_fused"] = round(times["fused"], 2)
        out.append({"config": kind, "position": pos, "splits": plan.splits, "kv_bytes": kv_bytes,
                    "us_per_call": round(times["call"], 2), **extra, "split_us": round(times["split"], 2),
                    "kv_gbs_split": round(kv_bytes / (times["split"] * 1e-6) / 1e9, 1),
                    "pct_hbm_peak_split": round(100 * kv_bytes / (times["split"] * 1e-6) / 1e9 / HBM_PEAK_GBS, 1)})
        del reps_kv, pool
    return out


def bench_phases(torch, va, synth, dev, graphs=6, pairs=4, replays=12):
    """Phase timestamps of split and combine launches from the trace build
    of the library (lib/libverify_attn_trace.so; include/verify_probe.h):
    the sweep's seven contexts (as timed above) and the bf16 and quantised
    trees at 32K / 64K.  Each case captures `graphs` graphs of `pairs`
    back-to-back split + combine calls over distinct cold replicas and
    replays them in turn; after each replay the records of its last pair
    are read.  Reported (us, medians over replays; "mean" over workgroups):
    the spread of workgroup entries, the arguments' arrival, the first DMA
    issue, chunk 0's arrival in LDS, the chunks' steps, the last
    step, the partials' stores, the gap to the combine's first workgroup
    and the combine's phases; `us_per_call` times the same graphs with
    events (the trace build's own speed, for comparison with the product's)."""
    import ctypes
    import statistics
    import numpy as np
    import speculative_decode_verify_amd._binding as binding
    product = binding.load_library()
    binding._LIB = None
    saved = binding._LIB_PATH
    binding._LIB_PATH = binding.trace_library_path()
    lib = binding.load_library()
    binding._LIB_PATH = saved
    lib.va_trace_read.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_int]
    stream = torch.cuda.current_stream()
    tick_us = 0.01  # s_memrealtime runs at 100 MHz

    def records(which, n):
        buf = np.zeros((n, 24 if which == 0 else 8), dtype=np.uint64)
        if lib.va_trace_read(which, buf.ctypes.data, n) != 0:
            raise RuntimeError("va_trace_read failed")
        return buf.astype(np.int64)

    cases = []
    for ctx in CONTEXTS:
        g = synth.gen(2000 + ctx // 1024)
        live = synth.live_count(g)
        hi = ctx + live
        nb = kv_bytes(hi)
        pool, npool = cold_pool(torch, synth, dev, nb, seed=60_000 + ctx)
        q = synth.normal_bf16((ROWS, HQ, D), g).to(dev)
        sink = synth.normal_f32((HQ,), g).to(dev)
        plan = va.Plan(rows=ROWS, live_rows=live, q_heads=HQ, kv_heads=HKV, head_dim=D, mask="causal",
                       first_pos=ctx, kv_capacity=CAP, scale=1 / math.sqrt(D))

        def kv_of(i, pool=pool, npool=npool, hi=hi):
            fl = pool.view(torch.bfloat16)
            kb = (i % npool) * hi * 2 * D
            vb = kb + hi * D
            return fl[kb:kb + hi * D].view(HKV, hi, D), fl[vb:vb + hi * D].view(HKV, hi, D), None
        cases.append(dict(name=f"sweep {ctx // 1024}K", plan=plan, q=q, sink=sink, kv_of=kv_of, npool=npool,
                          rows=ROWS, hq=HQ, d=D, live=live, keep=pool, waves=-(-ROWS * (HQ // HKV) // 16)))
    g = synth.gen(9500)
    for quant, P in ((False, 32768), (True, 65536)):
        kw = dict(rows=16, live_rows=16, q_heads=24, kv_heads=4, head_dim=128, mask="tree", prefix_len=P,
                  parent=synth.random_tree(16, g), kv_capacity=P + 16 + 64, scale=1 / math.sqrt(128))
        if quant:
            kw["kv_fmt"] = "e4m3_wht_i8"
        plan = va.Plan(**kw)
        hkv, d, slots = 4, 128, kw["kv_capacity"]
        kvb = hkv * slots * d * (1 if quant else 2)
        per = 2 * kvb + (hkv * slots * 4 if quant else 0)
        n = max(REPLICAS, -(-POOL_BYTES // per))
        pool = torch.empty(n * per, dtype=torch.uint8, device=dev)
        if quant:
            kv_all = pool.view(n, per)
            kv_all[:, :kvb] = torch.randint(0, 126, (n, kvb), dtype=torch.uint8, device=dev)
            kv_all[:, kvb:2 * kvb] = torch.randint(-127, 128, (n, kvb), dtype=torch.int8, device=dev).view(torch.uint8)
            kv_all[:, 2 * kvb:] = (torch.rand((n, hkv * slots), device=dev) * 0.02).view(torch.uint8)
        else:
            flat = pool.view(torch.bfloat16)
            for off in range(0, flat.numel(), 1 << 27):
                m = min(1 << 27, flat.numel() - off)
                flat[off:off + m] = synth.normal_bf16_device((m,), 61_000 + off // (1 << 27), dev)

        def kv_of(i, pool=pool, n=n, per=per, kvb=kvb, quant=quant, hkv=hkv, slots=slots, d=d):
            base = pool[(i % n) * per:(i % n + 1) * per]
            if quant:
                return (base[:kvb].view(hkv, slots, d), base[kvb:2 * kvb].view(torch.int8).view(hkv, slots, d),
                        base[2 * kvb:].view(torch.float32).view(hkv, slots))
            kv = base.view(torch.bfloat16).view(2, hkv, slots, d)
            return kv[0], kv[1], None
        cases.append(dict(name=("quantised tree 64K" if quant else "tree 32K"), plan=plan,
                          q=synth.normal_bf16((16, 24, 128), g).to(dev), sink=None, kv_of=kv_of, npool=n,
                          rows=16, hq=24, d=128, live=16, keep=pool, waves=6, quant=quant))

    out = []
    binding._LIB = lib
    try:
        for c in cases:
            plan = c["plan"]
            ws = va.workspace_for(plan, dev)
            o = torch.empty((c["rows"], c["hq"], c["d"]), dtype=torch.float32, device=dev)
            lse = torch.empty((c["rows"], c["hq"]), dtype=torch.float32, device=dev)
            nsw = plan.splits * plan.problem.kv_heads * plan.info["row_groups"]
            ncw = c["rows"] * c["hq"] * (c["d"] // 32)
            grs = []
            for gi in range(graphs):
                gr = torch.cuda.CUDAGraph()
                with torch.cuda.graph(gr):
                    for j in range(pairs):
                        k, v, vs = c["kv_of"](gi * pairs + j)
                        cur = torch.cuda.current_stream()
                        va.verify_attn_split(plan, c["q"], k, v, ws, v_scale=vs, stream=cur)
                        va.verify_attn_combine(plan, ws, o, lse=lse, sink=c["sink"], stream=cur)
                grs.append(gr)
            for gr in grs:
                gr.replay()
            torch.cuda.synchronize()
            rows = []
            for r in range(replays):
                grs[r % graphs].replay()
                torch.cuda.synchronize()
                sp = records(0, nsw)
                cb = records(1, ncw)
                # combine record index: h + Hq * (row * D/32 + d slice)
                live_wg = (np.arange(ncw) // c["hq"]) // (c["d"] // 32) < c["live"]
                cb = cb[live_wg]
                t0 = sp[:, 0].min()
                busy = sp[:, 7] > 0
                steps = np.maximum(sp[busy, 7] - 1, 1)
                rows.append(dict(
                    entry_spread=(sp[:, 0].max() - t0),
                    args=(sp[:, 1] - sp[:, 0]).mean(),
                    first_dma_issued=(sp[busy, 2] - sp[busy, 0]).mean(),
                    chunk0_in_lds=(sp[busy, 3] - sp[busy, 0]).mean(),
                    chunk0_in_lds_last=(sp[busy, 3].max() - t0),
                    step=((sp[busy, 4] - sp[busy, 3]) / np.maximum(sp[busy, 7], 1)).mean(),
                    barrier_share=(sp[busy, 6] / np.maximum(sp[busy, 4] - sp[busy, 3], 1)).mean(),
                    last_step_issued=(sp[busy, 4] - t0).mean(),
                    partials_written=(sp[busy, 5] - t0).mean(),
                    split_span=(sp[busy, 5].max() - t0),
                    gap_to_combine=(cb[:, 0].min() - sp[busy, 5].max()),
                    comb_entry_spread=(cb[:, 0].max() - cb[:, 0].min()),
                    comb_args=(cb[:, 1] - cb[:, 0]).mean(),
                    comb_first_batch=(cb[:, 2] - cb[:, 0]).mean(),
                    comb_folded=(cb[:, 3] - cb[:, 0]).mean(),
                    comb_written=(cb[:, 4] - cb[:, 0]).mean(),
                    comb_span=(cb[:, 4].max() - cb[:, 0].min()),
                    pair_span=(cb[:, 4].max() - t0),
                    # each role's time at the later barriers per step: the
                    # role that waits least holds the chunk's step
                    **{f"wait_c{w}": (sp[busy, 8 + w] / steps).mean() for w in range(c["waves"])},
                    dma_prod=(sp[busy, 14] / steps).mean(),
                    wait_prod=(sp[busy, 15] / steps).mean(),
                    **({"wait_dec": (sp[busy, 16] / steps).mean(),
                        "conv_dec": (sp[busy, 17] / np.maximum(sp[busy, 7], 1)).mean()} if c.get("quant") else {})))
            med = {k: round(statistics.median(float(x[k]) for x in rows) * (1 if k == "barrier_share" else tick_us), 3)
                   for k in rows[0]}
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for gr in grs:
                gr.replay()
            b.record(stream)
            torch.cuda.synchronize()
            med["us_per_call"] = round(a.elapsed_time(b) * 1e3 / (graphs * pairs), 3)
            out.append(dict(case=c["name"], splits=plan.splits, workgroups=nsw, chunks_per_split=
                            round(float(plan.info["chunks"]) / plan.splits, 2) if "chunks" in plan.info else None,
                            **med))
            print(json.dumps(out[-1]), flush=True)
            del grs, ws
    finally:
        binding._LIB = product
    return out


def compare_libraries(torch, va, synth, dev, args):
    """Split alone and split + combine pairs of several library builds, per
    context, over cold pools (as pass B), in alternating order with the
    built library as two arms (A and A')."""
    import statistics
    import speculative_decode_verify_amd._binding as binding
    contexts = args.ctx or CONTEXTS
    stream = torch.cuda.current_stream()
    built = binding.load_library()
    arms = [("A", built), ("A'", built)]
    for i, path in enumerate(args.compare):
        binding._LIB = None
        saved = binding._LIB_PATH
        binding._LIB_PATH = os.path.abspath(path)
        arms.append((f"B{i}:{os.path.basename(path)}", binding.load_library()))
        binding._LIB_PATH = saved
    binding._LIB = built
    cases = []
    for ctx in contexts:
        g = synth.gen(2000 + ctx // 1024)
        live = synth.live_count(g)
        hi = ctx + live
        nb = kv_bytes(hi)
        pool, npool = cold_pool(torch, synth, dev, nb, seed=50_000 + ctx)
        q = synth.normal_bf16((ROWS, HQ, D), g).to(dev)
        sink = synth.normal_f32((HQ,), g).to(dev)
        cases.append(dict(ctx=ctx, live=live, hi=hi, nb=nb, pool=pool, npool=npool, q=q, sink=sink))
    state = {}
    for name, lib in arms:
        binding._LIB = lib
        for c in cases:
            plan = va.Plan(rows=ROWS, live_rows=c["live"], q_heads=HQ, kv_heads=HKV, head_dim=D, mask="causal",
                           first_pos=c["ctx"], kv_capacity=CAP, scale=1 / math.sqrt(D), splits=args.splits)
            state[(name, c["ctx"])] = (plan, va.workspace_for(plan, dev),
                                       torch.empty((ROWS, HQ, D), dtype=torch.float32, device=dev),
                                       torch.empty((ROWS, HQ), dtype=torch.float32, device=dev))
    binding._LIB = built

    def kv_of(c, i):
        fl = c["pool"].view(torch.bfloat16)
        kb = (i % c["npool"]) * c["hi"] * 2 * D
        vb = kb + c["hi"] * D
        return fl[kb:kb + c["hi"] * D].view(HKV, c["hi"], D), fl[vb:vb + c["hi"] * D].view(HKV, c["hi"], D)

    def timed(fn):
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr):
            fn()
        gr.replay()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        gr.replay()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / args.kernel_reps * 1e3

    res = {}
    for r in range(args.rounds):
        order = arms if r % 2 == 0 else arms[::-1]
        for name, lib in order:
            binding._LIB = lib
            for c in cases:
                plan, ws, out, lse = state[(name, c["ctx"])]

                def splits(c=c, plan=plan, ws=ws):
                    for i in range(args.kernel_reps):
                        k, v = kv_of(c, i)
                        va.verify_attn_split(plan, c["q"], k, v, ws, stream=torch.cuda.current_stream())

                def pairs(c=c, plan=plan, ws=ws, out=out, lse=lse):
                    for i in range(args.kernel_reps):
                        k, v = kv_of(c, i)
                        cur = torch.cuda.current_stream()
                        va.verify_attn_split(plan, c["q"], k, v, ws, stream=cur)
                        va.verify_attn_combine(plan, ws, out, lse=lse, sink=c["sink"], stream=cur)
                res.setdefault((name, c["ctx"], "split_us"), []).append(timed(splits))
                res.setdefault((name, c["ctx"], "us_per_call"), []).append(timed(pairs))
    binding._LIB = built
    table = {}
    for (name, ctx, what), xs in res.items():
        table.setdefault(name, {}).setdefault(str(ctx), {})[what] = {
            "median": round(statistics.median(xs), 3), "min": round(min(xs), 3), "max": round(max(xs), 3)}
    aa = {str(c["ctx"]): {w: round(abs(table["A"][str(c["ctx"])][w]["median"] -
                                       table["A'"][str(c["ctx"])][w]["median"]), 3)
                          for w in ("split_us", "us_per_call")} for c in cases}
    print(json.dumps({"compare": table, "aa_spread_us": aa, "rounds": args.rounds, "reps": args.kernel_reps,
                      "order": "alternating (forward, reversed)", "provenance": provenance(torch)}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--ctx", type=int, action="append", help="restrict to these contexts")
    ap.add_argument("--splits", type=int, default=0, help="force the split count (0: plan chooses)")
    ap.add_argument("--replicas", type=int, default=REPLICAS)
    ap.add_argument("--kernel-reps", type=int, default=200, help="event-timed launches per context")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="oracle time to spend on the CPU baseline")
    ap.add_argument("--summarize-profiles", metavar="DIR",
                    help="write the profiles/ summaries from one profiling session's outputs (no GPU)")
    ap.add_argument("--kv-write", action="store_true",
                    help="only time verify_kv_write (the rows' KV written into the cache before the read)")
    ap.add_argument("--sampler", action="store_true",
                    help="time va_sample_accept (sampling + acceptance) instead of the attention sweep")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB five times (HBM counter calibration)")
    ap.add_argument("--compare", nargs="+", metavar="LIB",
                    help="time these builds of the library against the built one (ABBA rounds, A/A arm)")
    ap.add_argument("--rounds", type=int, default=4, help="--compare: rounds (alternating order)")
    ap.add_argument("--phases", action="store_true",
                    help="phase timestamps of split and combine from the trace build of the library")
    args = ap.parse_args()
    if args.summarize_profiles:
        summarize_profiles(args.summarize_profiles)
        return

    if args.gpus != 1:
        if int(os.environ.get("RANK", "0")) == 0:
            print(f"bench.py: this build runs on one GPU only (asked for --gpus {args.gpus}); "
                  "the verification call is a single-GPU kernel and no multi-GPU path exists.", flush=True)
        sys.exit(2)

    import numpy as np
    import torch
    import speculative_decode_verify_amd as va
    from speculative_decode_verify_amd import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_probe:
        n = args.copy_probe << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": n, "launches": 5}), flush=True)
        return
    if args.kv_write:
        bench_kv_write(torch, va, synth, dev)
        return
    if args.sampler:
        bench_sampler(torch, va, synth, dev, cpu=not args.no_cpu_baseline)
        return
    if args.compare:
        compare_libraries(torch, va, synth, dev, args)
        return
    if args.phases:
        res = bench_phases(torch, va, synth, dev)
        print(json.dumps({"phases": res, "kernel_hash": kernel_hash(), "unit": "us",
                          "library": "lib/libverify_attn_trace.so", "provenance": provenance(torch)}), flush=True)
        return
    contexts = args.ctx or CONTEXTS
    stream = torch.cuda.current_stream()

    # ---------------- inputs ----------------
    cases = []
    for ctx in contexts:
        g = synth.gen(2000 + ctx // 1024)
        live = synth.live_count(g)
        hi = ctx + live
        q = synth.normal_bf16((ROWS, HQ, D), g).to(dev)
        sink = synth.normal_f32((HQ,), g).to(dev)
        plan = va.Plan(rows=ROWS, live_rows=live, q_heads=HQ, kv_heads=HKV, head_dim=D, mask="causal",
                       first_pos=ctx, kv_capacity=CAP, scale=1 / math.sqrt(D), splits=args.splits)
        kvs = []
        for r in range(args.replicas):
            k = torch.full((HKV, CAP, D), float("nan"), dtype=torch.bfloat16, device=dev)
            v = torch.full((HKV, CAP, D), float("nan"), dtype=torch.bfloat16, device=dev)
            k[:, :hi] = synth.normal_bf16_device((HKV, hi, D), 10_000 * r + ctx, dev)
            v[:, :hi] = synth.normal_bf16_device((HKV, hi, D), 10_000 * r + ctx + 1, dev)
            kvs.append((k, v))
        ws = va.workspace_for(plan, dev)
        out = torch.empty((ROWS, HQ, D), dtype=torch.float32, device=dev)
        lse = torch.empty((ROWS, HQ), dtype=torch.float32, device=dev)
        cases.append(dict(ctx=ctx, live=live, hi=hi, q=q, sink=sink, plan=plan, kvs=kvs, ws=ws, out=out, lse=lse))
    torch.cuda.synchronize()

    def call(c, rep):
        # launched on the current stream: the timing stream, or a graph's capture stream
        k, v = c["kvs"][rep]
        cur = torch.cuda.current_stream()
        va.verify_attn_split(c["plan"], c["q"], k, v, c["ws"], stream=cur)
        va.verify_attn_combine(c["plan"], c["ws"], c["out"], lse=c["lse"], sink=c["sink"], stream=cur)

    def step(i):
        for c in cases:
            call(c, i % args.replicas)

    # ---------------- parity of replica 0 at full size (kept for the CPU leg) ----------------
    for c in cases:
        call(c, 0)
    torch.cuda.synchronize()
    gpu_out0 = [(c["out"].double().cpu().numpy(), c["lse"].double().cpu().numpy()) for c in cases]

    # ---------------- HIP graphs of the work ----------------
    # Launching from Python costs ~10 us of host time per call, more than a
    # small-context kernel runs, so timed work is replayed from HIP graphs
    # (as a serving loop would launch it); the eager rate is reported beside.
    def capture(fn):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        return g

    step_graphs = [capture(lambda r=r: [call(c, r) for c in cases]) for r in range(args.replicas)]
    torch.cuda.synchronize()
    # a replayed step must reproduce the eager result bit for bit
    step_graphs[0].replay()
    torch.cuda.synchronize()
    for c, (o0, l0) in zip(cases, gpu_out0):
        if not (np.array_equal(c["out"].double().cpu().numpy(), o0) and
                np.array_equal(c["lse"].double().cpu().numpy(), l0)):
            raise SystemExit("graph replay differs from the eager launch")

    # ---------------- pass A: whole steps ----------------
    for i in range(args.warmup):
        step_graphs[i % args.replicas].replay()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t_wall = time.perf_counter()
    e0.record(stream)
    for i in range(args.steps):
        step_graphs[(args.warmup + i) % args.replicas].replay()
    e1.record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    ms_total = e0.elapsed_time(e1)
    ms_per_step = ms_total / args.steps
    bytes_per_step = sum(kv_bytes(c["hi"]) for c in cases)
    value = bytes_per_step / (ms_per_step * 1e-3) / 1e9

    # eager launches, for reference (host-bound at small contexts)
    e0.record(stream)
    for i in range(args.steps):
        step(i)
    e1.record(stream)
    torch.cuda.synchronize()
    eager_ms_per_step = e0.elapsed_time(e1) / args.steps

    # ---------------- passes B, B2, C: per-kernel times over cold pools ----------------
    # Per context, every timed launch reads a replica of that context's
    # extent from a pool of at least 1 GiB (the never-read capacity tail is
    # not allocated), so no launch finds its bytes in the 256 MB MALL or an
    # L2.  Each kernel is timed over kernel_reps back-to-back launches
    # replayed from a graph on the launch stream.
    #   B   the split and the combine of the static plan;
    #   B2  a plain streaming read of the same bytes (va_read_probe: one
    #       launch, 16-byte loads, a full grid), the ceiling the split
    #       kernel's rate is compared with beside the 8 TB/s peak;
    #   C   the device-state entry points: one plan for a bucket covering
    #       the whole sweep (8 rows at the largest context) fixes the grid;
    #       each context's positions and live rows come from a state record
    #       in device memory.  The outputs must match the static call's
    #       (same partials; the combine may order its FP32 sum differently).
    bucket = va.Plan(rows=ROWS, live_rows=ROWS, q_heads=HQ, kv_heads=HKV, head_dim=D, mask="causal",
                     first_pos=max(contexts), kv_capacity=CAP, scale=1 / math.sqrt(D))
    bws = va.workspace_for(bucket, dev)
    bout = torch.empty((ROWS, HQ, D), dtype=torch.float32, device=dev)
    blse = torch.empty((ROWS, HQ), dtype=torch.float32, device=dev)
    probe_sink = torch.zeros(1, dtype=torch.int32, device=dev)
    sweep = []
    split_bytes, split_ms, probe_bytes, probe_ms = 0.0, 0.0, 0.0, 0.0

    def timed(fn):
        g = capture(fn)
        g.replay()
        a, b = (torch.cuda.Event(enable_timing=True) for _ in range(2))
        a.record(stream)
        g.replay()
        b.record(stream)
        torch.cuda.synchronize()
        del g
        return a.elapsed_time(b) / args.kernel_reps

    for c in cases:
        # replica r: K at pool bytes [r*nb, r*nb + nb/2), V after it; the
        # views handed to the bucket's state calls are as long as the bucket
        # (their never-read tails alias the next replicas and a pool tail)
        nb = kv_bytes(c["hi"])
        bucket_slots = bucket.info["hi"]
        pool, npool = cold_pool(torch, synth, dev, nb, seed=50_000 + c["ctx"], tail=2 * bucket_slots * D * 2)
        fl = pool.view(torch.bfloat16)

        def kv_of(i, slots=None, c=c, fl=fl, npool=npool):
            slots = slots or c["hi"]
            kb = (i % npool) * c["hi"] * 2 * D
            vb = kb + c["hi"] * D
            return (fl[kb:kb + slots * D].view(HKV, slots, D), fl[vb:vb + slots * D].view(HKV, slots, D))

        def splits(c=c, kv_of=kv_of):
            for i in range(args.kernel_reps):
                k, v = kv_of(i)
                va.verify_attn_split(c["plan"], c["q"], k, v, c["ws"], stream=torch.cuda.current_stream())

        def combines(c=c):
            for i in range(args.kernel_reps):
                va.verify_attn_combine(c["plan"], c["ws"], c["out"], lse=c["lse"], sink=c["sink"],
                                       stream=torch.cuda.current_stream())

        def pairs(c=c, kv_of=kv_of):
            for i in range(args.kernel_reps):
                k, v = kv_of(i)
                cur = torch.cuda.current_stream()
                va.verify_attn_split(c["plan"], c["q"], k, v, c["ws"], stream=cur)
                va.verify_attn_combine(c["plan"], c["ws"], c["out"], lse=c["lse"], sink=c["sink"], stream=cur)

        def reads(nb=nb, pool=pool, npool=npool):
            for i in range(args.kernel_reps):
                r = i % npool
                va.va_read_probe(pool[r * nb:(r + 1) * nb], nb, probe_sink, stream=torch.cuda.current_stream())
        st = va.pack_state(first_pos=c["ctx"], live_rows=c["live"]).to(dev)

        def ssplits(c=c, st=st, kv_of=kv_of):
            for i in range(args.kernel_reps):
                k, v = kv_of(i, bucket_slots)
                va.verify_attn_split_state(bucket, st, c["q"], k, v, bws, stream=torch.cuda.current_stream())

        def scombines(c=c, st=st):
            for i in range(args.kernel_reps):
                va.verify_attn_combine_state(bucket, st, bws, bout, lse=blse, sink=c["sink"],
                                             stream=torch.cuda.current_stream())
        def spairs(c=c, st=st, kv_of=kv_of):
            for i in range(args.kernel_reps):
                k, v = kv_of(i, bucket_slots)
                cur = torch.cuda.current_stream()
                va.verify_attn_split_state(bucket, st, c["q"], k, v, bws, stream=cur)
                va.verify_attn_combine_state(bucket, st, bws, bout, lse=blse, sink=c["sink"], stream=cur)
        s_avg, c_avg, p_avg = timed(splits), timed(combines), timed(pairs)
        r_avg = timed(reads)
        ss_avg, sc_avg, sp_avg = timed(ssplits), timed(scombines), timed(spairs)
        del pool, fl
        split_bytes += nb * args.kernel_reps
        split_ms += s_avg * args.kernel_reps
        probe_bytes += nb * args.kernel_reps
        probe_ms += r_avg * args.kernel_reps
        gbs = nb / (s_avg * 1e-3) / 1e9
        sweep.append({
            "ctx": c["ctx"], "live": c["live"], "splits": c["plan"].splits, "kv_bytes": nb,
            "cold_pool_replicas": npool,
            "us_per_call": round(p_avg * 1e3, 2),
            "split_us": round(s_avg * 1e3, 2), "combine_us": round(c_avg * 1e3, 2),
            "kv_gbs_split": round(gbs, 1), "pct_hbm_peak_split": round(100 * gbs / HBM_PEAK_GBS, 1),
            "kv_gbs_call": round(nb / (p_avg * 1e-3) / 1e9, 1),
            "read_probe_us": round(r_avg * 1e3, 2), "read_probe_gbs": round(nb / (r_avg * 1e-3) / 1e9, 1),
            "state_split_us": round(ss_avg * 1e3, 2), "state_combine_us": round(sc_avg * 1e3, 2),
            "state_us_per_call": round(sp_avg * 1e3, 2),
        })
        # the state path against a static call with the same split count (the
        # bucket's, at most one granule each) on replica 0 of pass A: the
        # same partials, the combine's FP32 order apart
        k, v = c["kvs"][0]
        p0 = c["plan"].problem
        eq = va.Plan(rows=ROWS, live_rows=c["live"], q_heads=HQ, kv_heads=HKV, head_dim=D, mask="causal",
                     first_pos=c["ctx"], kv_capacity=CAP, scale=p0.scale,
                     splits=max(1, min(bucket.splits, c["plan"].info["chunks"])))
        eq_ws = va.workspace_for(eq, dev)
        eq_out, eq_lse = torch.empty_like(c["out"]), torch.empty_like(c["lse"])
        va.verify_attn_split(eq, c["q"], k, v, eq_ws, stream=stream)
        va.verify_attn_combine(eq, eq_ws, eq_out, lse=eq_lse, sink=c["sink"], stream=stream)
        va.verify_attn_split_state(bucket, st, c["q"], k, v, bws, stream=stream)
        va.verify_attn_combine_state(bucket, st, bws, bout, lse=blse, sink=c["sink"], stream=stream)
        torch.cuda.synchronize()
        L = c["live"]
        if not (torch.allclose(bout[:L], eq_out[:L], rtol=1e-5, atol=1e-6) and
                torch.allclose(blse[:L], eq_lse[:L], rtol=1e-6, atol=1e-5)):
            raise SystemExit(f"state path differs from the static call at ctx {c['ctx']}")
        del eq_ws
    achieved = split_bytes / (split_ms * 1e-3) / 1e9
    read_ceiling = probe_bytes / (probe_ms * 1e-3) / 1e9
    launches = len(cases) * args.kernel_reps

    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        try:
            tr = json.load(open(TRAFFIC_FILE))
            if (tr.get("kernel_hash") == kernel_hash() and tr.get("contexts") == contexts
                    and tr.get("splits") == [c["plan"].splits for c in cases]):
                traffic = tr.get("hbm_bytes_per_launch")
        except Exception:
            traffic = None

    mfma_busy = None
    if os.path.exists(UTIL_FILE):
        try:
            ut = json.load(open(UTIL_FILE))
            if ut.get("kernel_hash") == kernel_hash():
                mfma_busy = ut.get("mfma_busy_pct")
        except Exception:
            mfma_busy = None

    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                "kernel": "split_kernel<D=128,W=3,bf16,NST=4,NPW=2,STATE=false>", "algorithmic_bytes_per_launch": round(split_bytes / launches),
                "avg_launch_us": round(split_ms / launches * 1e3, 2), "launches": launches,
                "mfma_busy_pct": mfma_busy,
                "read_ceiling": {"kernel": "read_probe_kernel (plain 16-byte streaming read)",
                                 "achieved": round(read_ceiling, 1),
                                 "avg_launch_us": round(probe_ms / launches * 1e3, 2),
                                 "split_frac_of_ceiling": round(achieved / read_ceiling, 4)}}

    clocks = _sysfs_clocks(torch)

    # ---------------- pass D: the other configurations ----------------
    other = bench_other_configs(torch, va, synth, dev)

    # ---------------- CPU baseline (oracle) + full-size parity ----------------
    cpu = None
    parity = None
    if not args.no_cpu_baseline:
        from oracle import attn as oattn
        from oracle.masks import Problem
        try:
            from threadpoolctl import threadpool_info
            threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"]
                          or [1])
        except Exception:
            threads = 1
        t_cpu = 0.0
        max_err, max_lse = 0.0, 0.0
        ok = True
        host = []
        for c in cases:
            k, v = c["kvs"][0]
            host.append((k[:, :c["hi"]].double().cpu().numpy(), v[:, :c["hi"]].double().cpu().numpy(),
                         c["q"].double().cpu().numpy(), c["sink"].double().cpu().numpy(),
                         Problem("causal", ROWS, c["live"], first_pos=c["ctx"])))
        # The sample: whole passes over the sweep (replica 0's stored bytes)
        # until about 10 s of oracle time, at most 20 passes; the first pass
        # is also the full-size parity check.
        passes = 0
        t_ctx = [0.0] * len(cases)
        while passes < 20 and (passes == 0 or t_cpu < args.cpu_seconds):
            for i, (c, (kc, vc, qc, sc, p), (o_gpu, l_gpu)) in enumerate(zip(cases, host, gpu_out0)):
                t = time.perf_counter()
                ro, rl = oattn.verify_attn_ref(p, qc, oattn.Cache(kc, vc), 1 / math.sqrt(D), sc)
                dt = time.perf_counter() - t
                t_cpu += dt
                t_ctx[i] += dt
                if passes:
                    continue
                L = c["live"]
                err = np.abs(o_gpu[:L] - ro[:L])
                ok &= bool(np.all(err <= 2e-3 + 1e-2 * np.abs(ro[:L])))
                ok &= bool(np.all(o_gpu[L:] == 0))
                dl = np.abs(l_gpu[:L] - rl[:L])
                ok &= bool(np.all(dl <= 1e-4))
                max_err = max(max_err, float(err.max()))
                max_lse = max(max_lse, float(dl.max()))
            passes += 1
        for entry, tc in zip(sweep, t_ctx):
            entry["oracle_s_per_call"] = round(tc / passes, 5)
        cpu = {"value": round(passes * bytes_per_step / t_cpu / 1e9, 4), "unit": "GB/s", "cores": int(threads),
               "kind": "oracle",
               "sample": f"{passes} passes over the {len(cases)} contexts (replica 0's stored bytes), "
                         f"float64 numpy, {t_cpu:.1f} s"}
        parity = {"max_abs_err": max_err, "max_lse_err": max_lse, "pass": ok,
                  "gate": "|err| <= 2e-3 + 1e-2|ref|, |dlse| <= 1e-4, padding rows 0"}

    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "full-attention verify sweep: Hkv 1, Hq 6, D 128, 8 rows (4-8 live), "
                               "causal, sink on, capacity 262144, ctx 1K-192K, cold KV",
                   "contexts": contexts, "replicas": args.replicas, "splits": "plan" if not args.splits else args.splits,
                   "launch": "HIP graph replay",
                   "state_bucket": f"{ROWS} rows at {max(contexts)}, {bucket.splits} splits"},
        "eager_launch_ms_per_step": round(eager_ms_per_step, 4),
        "roofline": roofline, "cpu_baseline": cpu, "parity": parity, "sweep": sweep, "other_configs": other,
        "wall_s_timed": round(t_wall, 4), "kernel_hash": kernel_hash(),
        "provenance": provenance(torch, clocks),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
