"""Benchmark: paged-attention decode on one MI355X.

One step = the whole hot path for one decode iteration of the batch: the
write of every sequence's new token into the paged pools (paged_kv_write),
then paged attention over every sequence's full context (the decode kernel,
plus the split merge kernel when a sequence is split over several
workgroups).  Inputs are synthetic and already resident in HBM when timing
starts.

Default workload: Llama-3-8B-shaped GQA decode -- 256 sequences, 32 query
heads sharing 8 KV heads, head_dim 128, bf16 pools in 16-token blocks,
context lengths log-uniform in [256, 8192], physical blocks shuffled.

Prints one JSON line.  `value` is decode tokens/s (sequences advanced by one
token per second, write + attention).  `roofline` rates the decode call (the
dominant cost) against MI355X HBM peak using the algorithmic KV bytes
(sum_s L_s * H_kv * D * 2 * elt) and the call's average duration from HIP
events recorded on the launch stream inside the timed loop; its `traffic`
is the HBM byte count per call from rocprofv3 counters, read from the
committed summary under profiles/ when that summary was taken on the
current kernel source (null otherwise).  `cpu_baseline` times the CPU oracle
on the same workload, and `check` compares every output element with it.

    python bench.py [--gpus 1] [--steps 50] [--warmup 10] [--workload gqa8b]

Measurement helpers (not part of the step):
    python bench.py --copy-calibration       plain 1 GiB device copy, for counter scaling
    python bench.py --summarize-trace DIR    rocprofv3 --stats CSV -> markdown
    python bench.py --summarize-traffic ...  rocprofv3 --pmc CSVs -> profiles/ traffic file
"""
from __future__ import annotations

import argparse
import csv
import ctypes
import glob
import hashlib
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PROFILES = os.path.join(ROOT, "profiles")
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak
COPY_BYTES = 1 << 30
TOL = {"f32": 1e-5, "bf16": 2e-2, "fp8": 6e-2}
CPU_RUNS = 3  # timed oracle runs (after one warm-up); the median is reported
WORKLOAD_DESC = {
    "tiny": "tiny fp32 paged decode: lens {7,16,33,100}, 4/4 heads, D=64",
    "13b": "LLaMA-2-13B-shaped bf16 decode: B=64, 40/40 heads, D=128, lens U[128,2048]",
    "gqa8b": "Llama-3-8B-shaped GQA bf16 decode: B=256, 32 q / 8 kv heads, D=128, lens log-U[256,8192]",
    "prefix": "shared-prefix bf16 decode: 32 prompts x 8 samples, 32/8 heads, D=128, 1024-token aliased prefix",
    "spec4": "speculative verification: the gqa8b batch with 4 new query tokens per sequence (1024 rows), bf16",
    "chunk512": "chunked prefill: 16 sequences x 512 new tokens on contexts U[2048, 8192], 32/8 heads, D=128, bf16",
    "longfp8": "long-context fp8-e4m3 KV decode: B=16, 64 q / 8 kv heads, D=128, lens U[16384,32768], 512-token partitions",
}
# Sources whose change invalidates counter figures taken on the decode call.
DECODE_SOURCES = ["paged_kv_cache_369_amd/csrc/paged_decode.hip", "paged_kv_cache_369_amd/csrc/pkv_internal.h",
                  "paged_kv_cache_369_amd/csrc/capi.cpp", "paged_kv_cache_369_amd/build.py"]


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def decode_source_digest() -> str:
    h = hashlib.sha256()
    for rel in DECODE_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_file(workload: str, directory: str = PROFILES) -> str:
    """profiles/paged_decode_<workload>_hbm_traffic.json, or paged_prefill_<workload> for a '-prefill' key."""
    if workload.endswith("-prefill"):
        return os.path.join(directory, f"paged_prefill_{workload[:-len('-prefill')]}_hbm_traffic.json")
    return os.path.join(directory, f"paged_decode_{workload}_hbm_traffic.json")


def load_traffic(workload: str):
    """HBM bytes per decode call from the committed counter summary, if taken on this source."""
    path = traffic_file(workload)
    if not os.path.exists(path):
        return None, "no counter summary"
    with open(path) as f:
        t = json.load(f)
    if t.get("source_digest") != decode_source_digest():
        return None, "counter summary predates the current decode source"
    return int(t["bytes_per_call"]), os.path.relpath(path, ROOT)


def run_heads(group: int) -> int:
    """Query heads one decode run serves: the largest divisor of the GQA group that is at most 16."""
    for g in range(min(group, 16), 1, -1):
        if group % g == 0:
            return g
    return 1


def cascade_read_bytes(w) -> int:
    """KV bytes the shared-prefix decode reads for a workload with consistent sharing arrays: each chunk of
    16 / run_heads consecutive group members reads the group's shared tokens once, and every sequence reads
    its own tokens after them."""
    members = 16 // run_heads(w.num_heads // w.num_kv_heads)
    tokens = 0
    for s, L in enumerate(w.context_lens.tolist()):
        pb = min(max(int(w.prefix_blocks[s]), 0), L // 16)
        if pb > 0 and (s - int(w.prefix_leader[s])) % members == 0:
            tokens += pb * 16
        tokens += L - pb * 16
    return tokens * w.num_kv_heads * w.head_dim * 2 * w.kv_elt_bytes()


def varlen_read_bytes(w) -> int:
    """KV bytes paged_attention_varlen reads: every group of 16 / run_heads new tokens of a sequence reads its
    context up to the group's last token, once per run of query heads."""
    rh = run_heads(w.num_heads // w.num_kv_heads)
    tpr = 16 // rh
    runs = w.num_heads // rh
    tokens = 0
    for s, L in enumerate(w.context_lens.tolist()):
        n = int(w.cu_q[s + 1] - w.cu_q[s])
        for g in range(0, n, tpr):
            tokens += L - n + min(g + tpr, n)
    return tokens * runs * w.head_dim * 2 * w.kv_elt_bytes()


def prefill_flops(w) -> int:
    """Algorithmic flops of causal attention of every new token over its visible positions: per query row and
    head, 2 * D per visible position for the scores and 2 * D for the weighted sum of values."""
    vis = 0
    for s, L in enumerate(w.context_lens.tolist()):
        n = int(w.cu_q[s + 1] - w.cu_q[s])
        vis += n * (L - n) + n * (n + 1) // 2
    return 4 * w.head_dim * w.num_heads * vis


def prefill_read_bytes(w) -> int:
    """KV bytes the tiled prefill reads from the pools at most: each wave (32 / G new tokens of one sequence and
    KV head) reads the context up to its last token; waves that share a context on one XCD meet in its L2."""
    tpw = 32 // (w.num_heads // w.num_kv_heads)
    tokens = 0
    for s, L in enumerate(w.context_lens.tolist()):
        n = int(w.cu_q[s + 1] - w.cu_q[s])
        for t in range(0, n, tpw):
            tokens += L - n + min(t + tpw, n)
    return tokens * w.num_kv_heads * w.head_dim * 2 * w.kv_elt_bytes()


def kernel_key(args) -> str:
    """The kernel an SQ counter summary covers (a substring of its name): the prefill's for --prefill (bf16/fp8
    pools run paged_prefill_lds_kernel, f32 pools paged_prefill_kernel), else the decode's."""
    return "paged_prefill" if args.prefill else "paged_decode_kernel"


def call_kernels(args) -> list:
    """Every kernel one timed call launches (substrings of their names): the shared-prefix decode is the
    decode kernel and then the merge of prefix and suffix states."""
    return [kernel_key(args)] + (["cascade_merge_kernel"] if args.cascade else [])


def profile_key(args) -> str:
    return args.workload + ("-cascade" if args.cascade else "") + ("-prefill" if args.prefill else "")


def _dev(a, dtype, torch):
    a = np.ascontiguousarray(a)
    if dtype == "bf16":
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(a).cuda()


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


# ---------------------------------------------------------------------------
# measurement helpers
# ---------------------------------------------------------------------------

def copy_calibration(torch, steps: int) -> int:
    """A plain device-to-device copy of COPY_BYTES per launch.

    Reads and writes exactly COPY_BYTES each; rocprofv3's FETCH_SIZE and
    WRITE_SIZE for this launch give the scale between those counters and
    true HBM bytes on this machine.
    """
    src = torch.ones(COPY_BYTES // 2, dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / steps
    print(json.dumps({"copy_bytes": COPY_BYTES, "avg_us": us, "copy_GBps_read_plus_write": 2 * COPY_BYTES / us / 1e3}),
          flush=True)
    return 0


def plain_read(torch, pkv, nbytes: int, reps: int = 10) -> dict:
    """A plain streaming read on the same GPU, beside the decode: pkv_stream_read over a buffer as large as the
    decode's KV bytes (16-byte loads over a chip-filling grid).  Timed with events after two warm-ups."""
    n16 = max(nbytes // 16, 1 << 16)
    buf = torch.ones(n16 * 4, dtype=torch.int32, device="cuda")
    sink = torch.zeros(pkv.STREAM_SINK_WORDS, dtype=torch.int32, device="cuda")
    for _ in range(2):
        pkv.pkv_stream_read(buf, sink)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        pkv.pkv_stream_read(buf, sink)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / reps
    del buf
    return {"GBps": 16 * n16 / us / 1e3, "bytes": 16 * n16, "avg_us": us,
            "kernel": "pkv_stream_read over a buffer of the decode's KV size (a plain streaming read)"}


READ_PROBE_CASES = [(2048, 4, 3), (2048, 8, 3), (2048, 16, 3), (2048, 4, 4), (2048, 16, 4),
                    (4096, 4, 2), (4096, 8, 2), (4096, 16, 2)]


def read_probe(torch, pkv, out_path: str, reps: int = 20) -> int:
    """Markdown table of pkv_tile_read (the decode's gathered K/V tile reads, no arithmetic) over 800 MB per
    launch (two 400 MB pools, a shuffled list of every tile), for each supported tile size, V load width and
    depth, next to pkv_stream_read over the same 800 MB.  Events around `reps` launches after three warm-ups."""
    pool = 400 << 20
    k = torch.ones(pool // 4, dtype=torch.int32, device="cuda")
    v = torch.ones(pool // 4, dtype=torch.int32, device="cuda")
    sink = torch.zeros(pkv.TILE_SINK_WORDS, dtype=torch.int32, device="cuda")
    gen = torch.Generator().manual_seed(7)
    rows = ["| tile (K + V) | V load width | tiles in flight | µs per launch | GB/s |", "|---|---|---|---|---|"]
    for tb, vw, depth in READ_PROBE_CASES:
        n = pool // tb
        ids = torch.randperm(n, generator=gen).to(torch.int32).cuda()
        for _ in range(3):
            pkv.pkv_tile_read(k, v, ids, n, tb, vw, depth, sink)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            pkv.pkv_tile_read(k, v, ids, n, tb, vw, depth, sink)
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / reps
        kind = "fp8, D=128" if tb == 2048 else "bf16, D=128"
        rows.append(f"| {tb // 1024} KiB + {tb // 1024} KiB ({kind}) | {vw} B | {depth} | {us:.1f} | "
                    f"{2 * pool / us / 1e3:.0f} |")
    del k, v
    pr = plain_read(torch, pkv, 2 * pool, reps)
    rows.append(f"| plain streaming read (`pkv_stream_read`, 16 B) | — | 4 per thread | {pr['avg_us']:.1f} | "
                f"{pr['GBps']:.0f} |")
    text = "\n".join([
        "# Gathered K/V tile reads on MI355X (the decode's stream without its arithmetic)", "",
        "Command (run from the repository root):", "",
        "    python3 bench.py --read-probe", "",
        "`pkv_tile_read`: 2048 one-wave workgroups (the decode's occupancy for bf16 and fp8 at head_dim 128), "
        "each reading an equal share of a shuffled list of every tile id, the K tile and then the V tile of each, "
        "with nontemporal loads; K by 16-byte lane loads, V by the width given.  800 MB per launch "
        f"(two 400 MB pools), the mean of {reps} launches after three warm-ups.", ""] + rows) + "\n"
    with open(out_path, "w") as f:
        f.write(text)
    print(text)
    return 0


def _csv_rows(directory: str, suffix: str):
    files = sorted(glob.glob(os.path.join(directory, "**", "*" + suffix), recursive=True))
    if not files:
        raise SystemExit(f"no *{suffix} under {directory}")
    with open(files[0]) as f:
        return list(csv.DictReader(f))


def summarize_trace(directory: str, command: str, last: int = 0) -> int:
    """Markdown table of a rocprofv3 --kernel-trace --stats run (kernel_stats.csv); with last > 0, also the
    mean duration of each kernel's last `last` dispatches (the timed steps, after the warm-up ones), from
    kernel_trace.csv."""
    rows = _csv_rows(directory, "kernel_stats.csv")
    short = lambda name: name.replace("void ", "").replace("pkv::(anonymous namespace)::", "").split("(")[0]
    print(f"Command: `{command}`\n")
    print("| kernel | calls | average (us) | min (us) | max (us) | share of GPU time |")
    print("|---|---|---|---|---|---|")
    for r in rows:
        print(f"| `{short(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | {float(r['MinNs']) / 1e3:.1f} | "
              f"{float(r['MaxNs']) / 1e3:.1f} | {float(r['Percentage']):.1f} % |")
    if last > 0:
        per = {}
        for r in sorted(_csv_rows(directory, "kernel_trace.csv"), key=lambda r: int(r["Start_Timestamp"])):
            per.setdefault(short(r["Kernel_Name"]), []).append(
                (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
        print(f"\nMean of each kernel's last {last} dispatches (the timed steps):\n")
        print("| kernel | dispatches | mean (us) |")
        print("|---|---|---|")
        for k, v in per.items():
            if len(v) >= last and ("pkv" in k or "paged" in k):
                print(f"| `{k}` | {last} | {float(np.mean(v[-last:])):.1f} |")
    return 0


def _per_kernel(directory: str, counter: str):
    out = {}
    for r in _csv_rows(directory, "counter_collection.csv"):
        if r["Counter_Name"] != counter:
            continue
        out.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return out


def _pick(per_kernel, key):
    vals = [v for k, vs in per_kernel.items() if key in k for v in vs]
    return sum(vals) / len(vals) if vals else 0.0


# Longest context each workload's length law allows: what a contiguous allocator must reserve per sequence.
CASCADE_NOTE = ", decoded by paged_attention_decode_cascade (each shared prefix read once per chunk of samples)"

MAX_LEN = {"tiny": 100, "13b": 2048, "gqa8b": 8192, "prefix": 1024 + 512, "longfp8": 32768, "spec4": 8192,
           "chunk512": 8192}


def utilisation_rows():
    """KV memory utilisation: contiguous max-length reservation against paging (16-token blocks), per workload,
    and for the shared-prefix workload with the library's block manager sharing each prompt's blocks."""
    import paged_kv_cache_369_amd as pkv
    from paged_kv_cache_369_amd import workloads as W
    rows = []
    for name in ("tiny", "13b", "gqa8b", "prefix", "longfp8"):
        lens = W.context_lengths(name).astype(np.int64)
        tokens = int(lens.sum())
        reserved = len(lens) * MAX_LEN[name]
        paged = int(sum(-(-int(x) // 16) * 16 for x in lens))
        row = {"workload": name, "seqs": len(lens), "tokens": tokens, "max_len": MAX_LEN[name],
               "reserved_util": tokens / reserved, "paged_util": tokens / paged,
               "seqs_per_reserved_slot_budget": reserved / paged}
        if name == "prefix":
            # prompts forked into their samples: a prefix block is held once for all samples
            bm = pkv.BlockManager(len(lens) * 200, 200)
            sid = 0
            for p0 in range(0, len(lens), 8):
                root = sid
                bm.add(root)
                bm.append(root, 1024)
                for k in range(1, 8):
                    bm.fork(root, sid + k)
                for k in range(8):
                    bm.append(sid + k, int(lens[p0 + k]) - 1024)
                sid += 8
            free, used, live, held, pending = bm.stats()
            bm.close()
            row.update({"shared_blocks_used": used, "shared_tokens_held": held,
                        "shared_util": tokens / (used * 16), "block_copies": pending})
        rows.append(row)
    return rows


PREFIX_CACHE_POOLS = (256 * 96, 4096, 3328)


def prefix_cache_stream(seed: int = 11):
    """Prompt token ids of the prefix-caching request stream: the shared-prefix workload's 256 sequences in a
    seeded order, each one of 32 system prompts of 1024 ids followed by its own ids."""
    from paged_kv_cache_369_amd import workloads as W
    lens = W.context_lengths("prefix").astype(np.int64)
    rng = np.random.default_rng(seed)
    systems = rng.integers(0, 32000, size=(32, 1024), dtype=np.int32)
    order = rng.permutation(len(lens))
    return [np.concatenate([systems[s // 8], rng.integers(0, 32000, size=int(lens[s]) - 1024, dtype=np.int32)])
            for s in order]


def prefix_cache_rows(live: int = 64, seed: int = 11):
    """Automatic prefix caching on a request stream with the shared-prefix workload's shapes: its 256 sequences
    arrive one by one in a seeded order as prompts (one of 32 system prompts of 1024 token ids, then the
    sequence's own ids); at most `live` are held at once (the oldest is freed when another arrives).  Per pool
    size: prompt tokens, tokens reused from the cache (not computed, not written), evictions, peak blocks used."""
    import paged_kv_cache_369_amd as pkv
    prompts = prefix_cache_stream(seed)
    total = int(sum(len(p) for p in prompts))
    rows = []
    for pool in PREFIX_CACHE_POOLS:
        bm = pkv.BlockManager(pool, 96)
        bm.enable_prefix_caching()
        held, reused, peak = [], 0, 0
        for i, p in enumerate(prompts):
            if len(held) == live:
                bm.free(held.pop(0))
            _, cached = bm.add_prompt(i, p)
            reused += cached
            held.append(i)
            peak = max(peak, bm.stats()[1])
        registered, evictable, looked, hits, evictions = bm.cache_stats()
        bm.close()
        rows.append({"pool_blocks": pool, "live": live, "requests": len(prompts), "prompt_tokens": total,
                     "reused_tokens": reused, "reused_frac": reused / total,
                     "best_possible": (len(prompts) - 32) * 1024 / total, "blocks_looked_up": looked,
                     "blocks_reused": hits, "evictions": evictions, "peak_blocks_used": peak})
    return rows


def utilisation(args) -> int:
    rows = utilisation_rows()
    print("| workload | seqs | tokens | reserve per seq | reserved util | paged util | paged + shared prefix |")
    print("|---|---|---|---|---|---|---|")
    for r in rows:
        extra = f"{r['shared_util']:.2f} (logical tokens per physical slot)" if "shared_util" in r else "—"
        print(f"| {r['workload']} | {r['seqs']} | {r['tokens']} | {r['max_len']} | {r['reserved_util']:.3f} | "
              f"{r['paged_util']:.4f} | {extra} |")
    print(json.dumps(rows))
    pc = prefix_cache_rows()
    print()
    print("| pool blocks | live requests | prompt tokens | reused tokens | reused share (best possible) | "
          "evictions | peak blocks used |")
    print("|---|---|---|---|---|---|---|")
    for r in pc:
        print(f"| {r['pool_blocks']} | {r['live']} | {r['prompt_tokens']} | {r['reused_tokens']} | "
              f"{r['reused_frac']:.3f} ({r['best_possible']:.3f}) | {r['evictions']} | {r['peak_blocks_used']} |")
    print(json.dumps(pc))
    return 0


def summarize_counters(args) -> int:
    """Markdown table of SQ/GRBM counters of the decode (or, with --prefill, the prefill) kernel (one or more
    --pmc runs)."""
    vals = {}
    for d in args.counter_dirs:
        for r in _csv_rows(d, "counter_collection.csv"):
            if kernel_key(args) not in r["Kernel_Name"]:
                continue
            vals.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    if not vals:
        raise SystemExit(f"no {kernel_key(args)} rows in the counter runs")
    mean = {k: sum(v) / len(v) for k, v in vals.items()}
    from paged_kv_cache_369_amd import workloads as W
    lines = [f"# SQ counters of `{kernel_key(args)}`, workload `{profile_key(args)}`", "",
             WORKLOAD_DESC[args.workload] + (CASCADE_NOTE if args.cascade else ""), "",
             "Commands (run from the repository root):", ""]
    lines += [f"    {c}" for c in args.commands]
    lines += ["", "Mean over the profiled dispatches (each counter summed over the device by rocprofv3).", "",
              "| counter | value per dispatch |", "|---|---|"]
    for k in sorted(mean):
        lines.append(f"| `{k}` | {mean[k]:.6g} |")
    derived = []
    if "SQ_LDS_BANK_CONFLICT" in mean and mean.get("SQ_LDS_IDX_ACTIVE", 0) > 0:
        derived.append(f"- LDS bank-conflict cycles per LDS-active cycle (`SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE`): "
                       f"{mean['SQ_LDS_BANK_CONFLICT'] / mean['SQ_LDS_IDX_ACTIVE']:.4f}")
    if "SQ_INSTS_VMEM_RD" in mean and "SQ_WAVES" in mean and mean["SQ_WAVES"] > 0:
        derived.append(f"- vector memory read instructions per wave (`SQ_INSTS_VMEM_RD / SQ_WAVES`): "
                       f"{mean['SQ_INSTS_VMEM_RD'] / mean['SQ_WAVES']:.1f}")
    if "SQ_INSTS_VALU" in mean and "SQ_WAVES" in mean and mean["SQ_WAVES"] > 0:
        derived.append(f"- VALU instructions per wave (`SQ_INSTS_VALU / SQ_WAVES`): "
                       f"{mean['SQ_INSTS_VALU'] / mean['SQ_WAVES']:.0f}")
    hits, misses = mean.get("TCC_HIT_sum", mean.get("TCC_HIT")), mean.get("TCC_MISS_sum", mean.get("TCC_MISS"))
    if hits is not None and misses is not None and hits + misses > 0:
        derived.append(f"- L2 hit rate (`TCC_HIT / (TCC_HIT + TCC_MISS)`): {hits / (hits + misses):.3f}")
    if "SQ_WAVE_CYCLES" in mean and mean.get("SQ_BUSY_CYCLES", 0) > 0:
        derived.append(f"- wave-cycles per busy SQ cycle (`SQ_WAVE_CYCLES / SQ_BUSY_CYCLES`): "
                       f"{mean['SQ_WAVE_CYCLES'] / mean['SQ_BUSY_CYCLES']:.2f}")
    if "SQ_INSTS_MFMA" in mean and "SQ_WAVES" in mean and mean["SQ_WAVES"] > 0:
        derived.append(f"- matrix instructions per wave (`SQ_INSTS_MFMA / SQ_WAVES`): "
                       f"{mean['SQ_INSTS_MFMA'] / mean['SQ_WAVES']:.0f}")
    if "SQ_VALU_MFMA_BUSY_CYCLES" in mean and mean.get("SQ_BUSY_CYCLES", 0) > 0:
        derived.append(f"- matrix-busy cycles per busy SQ cycle (`SQ_VALU_MFMA_BUSY_CYCLES / SQ_BUSY_CYCLES`): "
                       f"{mean['SQ_VALU_MFMA_BUSY_CYCLES'] / mean['SQ_BUSY_CYCLES']:.3f}")
    if derived:
        lines += ["", "Ratios:", ""] + derived
    lines += ["", f"Decode source digest `{decode_source_digest()}`."]
    os.makedirs(args.out_dir, exist_ok=True)
    stem = f"paged_prefill_{args.workload}" if args.prefill else f"paged_decode_{profile_key(args)}"
    path = os.path.join(args.out_dir, f"{stem}_sq_counters.md")
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(path)
    return 0


def summarize_traffic(args) -> int:
    """Scale FETCH_SIZE / WRITE_SIZE of the decode call by the copy calibration; write profiles/ files."""
    cf = _pick(_per_kernel(args.copy_fetch, "FETCH_SIZE"), "copyBuffer")
    cw = _pick(_per_kernel(args.copy_write, "WRITE_SIZE"), "copyBuffer")
    if cf <= 0 or cw <= 0:
        raise SystemExit("copy calibration kernel not found in the counter runs")
    fscale = COPY_BYTES / (cf * 1024)
    wscale = COPY_BYTES / (cw * 1024)
    fetch = _per_kernel(args.dec_fetch, "FETCH_SIZE")
    write = _per_kernel(args.dec_write, "WRITE_SIZE")
    kernels = {}
    for key in call_kernels(args):
        f_kib, w_kib = _pick(fetch, key), _pick(write, key)
        kernels[key] = {"fetch_kib": f_kib, "write_kib": w_kib,
                        "fetch_bytes": f_kib * 1024 * fscale, "write_bytes": w_kib * 1024 * wscale}
    total = sum(k["fetch_bytes"] + k["write_bytes"] for k in kernels.values())
    from paged_kv_cache_369_amd import workloads as W
    w = W.make(args.workload)
    kv = (cascade_read_bytes(w) if args.cascade else prefill_read_bytes(w) if args.prefill else
          varlen_read_bytes(w) if w.cu_q is not None else w.kv_bytes())
    rec = {"workload": profile_key(args), "source_digest": decode_source_digest(),
           "copy_calibration": {"bytes": COPY_BYTES, "fetch_kib": cf, "write_kib": cw,
                                "fetch_scale": fscale, "write_scale": wscale},
           "kernels": kernels, "bytes_per_call": int(round(total)), "algorithmic_kv_bytes": kv,
           "commands": args.commands}
    os.makedirs(args.out_dir, exist_ok=True)
    with open(traffic_file(profile_key(args), args.out_dir), "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    md = traffic_file(profile_key(args), args.out_dir).replace(".json", ".md")
    with open(md, "w") as f:
        f.write(f"# HBM traffic of one {'prefill' if args.prefill else 'decode'} call, workload `{profile_key(args)}`\n\n")
        f.write(f"{WORKLOAD_DESC[args.workload]}{CASCADE_NOTE if args.cascade else ''}.\n\n"
                "Commands (run from the repository root):\n\n")
        for c in args.commands:
            f.write(f"    {c}\n")
        f.write("\nCounter scale from the plain 1 GiB device copy (`__amd_rocclr_copyBuffer`): "
                f"FETCH_SIZE reads {cf:.0f} KiB (scale {fscale:.4f}), WRITE_SIZE reads {cw:.0f} KiB "
                f"(scale {wscale:.4f}).\n\n")
        f.write("| kernel | FETCH_SIZE (KiB/dispatch) | WRITE_SIZE (KiB/dispatch) | scaled read (MB) | scaled write (MB) |\n")
        f.write("|---|---|---|---|---|\n")
        for key, k in kernels.items():
            f.write(f"| `{key}` | {k['fetch_kib']:.0f} | {k['write_kib']:.0f} | {k['fetch_bytes'] / 1e6:.1f} | "
                    f"{k['write_bytes'] / 1e6:.1f} |\n")
        f.write(f"\nTotal per call: {total / 1e6:.1f} MB of HBM traffic against {kv / 1e6:.1f} MB of "
                f"{'KV bytes the waves request (reads of one context by several waves counted each time)' if args.prefill else 'algorithmic KV bytes'} "
                f"(ratio {total / kv:.4f}).  Kernel source digest `{rec['source_digest']}`.\n")
    print(json.dumps({"bytes_per_call": rec["bytes_per_call"], "ratio_to_kv": total / kv}))
    return 0


# ---------------------------------------------------------------------------
# the benchmark
# ---------------------------------------------------------------------------

def oracle_baseline(w, out_dev, q_dtype, max_seqs: int):
    """Time the CPU oracle (as it stands) on the first max_seqs sequences and compare every output."""
    import oracle  # test infrastructure, used only for this reported baseline and check
    npd = {"f32": np.float32, "bf16": np.uint16, "fp8": np.uint8}[w.cache_dtype]
    nb, hkv, d = w.layout.num_blocks, w.num_kv_heads, w.head_dim
    kp = np.zeros(oracle.k_pool_shape(nb, hkv, d, w.cache_dtype), dtype=npd)
    vp = np.zeros(oracle.v_pool_shape(nb, hkv, d, w.cache_dtype), dtype=npd)
    for b in w.layout.history:
        oracle.kv_write(b.k, b.v, w.in_dtype, kp, vp, w.cache_dtype, b.slots, k_scale=w.k_scale, v_scale=w.v_scale)
    oracle.kv_write(w.new_k, w.new_v, w.in_dtype, kp, vp, w.cache_dtype, w.layout.new_slots,
                    k_scale=w.k_scale, v_scale=w.v_scale)
    if max_seqs < 0:  # the longest prefix of sequences within about 4e9 query-row x token x head x dim products
        rows_per = np.diff(w.cu_q) if w.cu_q is not None else np.ones(w.num_seqs, dtype=np.int64)
        cost = np.cumsum(rows_per.astype(np.float64) * w.context_lens * w.num_heads * w.head_dim)
        n = max(1, int(np.searchsorted(cost, 4e9, side="right")))
        n = min(n, w.num_seqs)
    else:
        n = min(max_seqs, w.num_seqs)
    sl = slice(0, n)
    rows = int(w.cu_q[n]) if w.cu_q is not None else n

    def run():
        if w.cu_q is not None:  # several new tokens per sequence: the rows of the first n sequences
            return oracle.paged_attention_varlen(np.ascontiguousarray(w.q[:rows]), w.q_dtype,
                                                 np.ascontiguousarray(w.cu_q[:n + 1]), kp, vp, w.cache_dtype,
                                                 np.ascontiguousarray(w.layout.block_table[sl]),
                                                 np.ascontiguousarray(w.context_lens[sl]), w.scale, w.k_scale,
                                                 w.v_scale)
        return oracle.paged_attention(np.ascontiguousarray(w.q[sl]), w.q_dtype, kp, vp, w.cache_dtype,
                                      np.ascontiguousarray(w.layout.block_table[sl]),
                                      np.ascontiguousarray(w.context_lens[sl]), w.scale, w.k_scale, w.v_scale)

    # one untimed warm-up, then the median of CPU_RUNS timed runs (wall clock, no generation or I/O inside)
    ref = run()
    times = []
    for _ in range(CPU_RUNS):
        t0 = time.perf_counter()
        ref = run()
        times.append(time.perf_counter() - t0)
    dt = float(np.median(times))
    import torch
    o = out_dev[:rows].detach().cpu()
    got = (o.view(torch.int16).numpy().view(np.uint16).astype(np.uint32) << 16).view(np.float32) \
        if q_dtype == "bf16" else o.numpy()
    err = float(np.max(np.abs(got.astype(np.float64) - ref))) if ref.size else 0.0
    return n, rows, dt, times, oracle.num_threads(0), err


def timeline_summary(rows, kv_bytes: int, desc: str, command: str) -> str:
    """Markdown summary of one decode call's per-wave stamps (pkv_timeline_read rows: entry, first tile,
    1/4, 1/2, 3/4 of the tiles, end in 100 MHz ticks; hardware wave id | XCD << 32 | tiles << 40; last tile)."""
    r = rows[rows[:, 0] != 0].astype(np.int64)
    t0 = r[:, 0].min()
    us = (r[:, :6] - t0) / 100.0  # microseconds after the first wave's entry
    ent, first, q1, q2, q3, end = (us[:, i] for i in range(6))
    hw = r[:, 6] & 0xffffffff
    xcc = (r[:, 6] >> 32) & 0xf
    tiles = r[:, 6] >> 40
    last = (r[:, 7] - t0) / 100.0
    slot = hw & 0xf
    n = len(r)
    out = [f"# Per-wave timeline of one decode call, {desc}", "",
           "Command (run from the repository root; the instrumented library is the same sources with "
           "PKV_TIMELINE defined, each wave adding seven clock reads and one 64-byte store):", "",
           f"    {command}", "",
           f"{n} waves with a stretch; times in µs after the first wave's entry (real-time clock, 100 MHz). "
           f"Last wave ends at {end.max():.1f} µs.", "",
           "| wave slot | waves | entry p50 | first tile p50 | 25 % p50 | 50 % p50 | 75 % p50 | last tile p50 | "
           "end p10 | end p50 | end p90 | end max | close after last tile p50 / p90 / max |",
           "|---|---|---|---|---|---|---|---|---|---|---|---|---|"]
    med = lambda x: float(np.median(x)) if len(x) else float("nan")
    pct = lambda x, p: float(np.percentile(x, p)) if len(x) else float("nan")
    for sl in sorted(set(slot.tolist())):
        m = slot == sl
        cl = end[m] - last[m]
        out.append(f"| {sl} | {int(m.sum())} | {med(ent[m]):.1f} | {med(first[m]):.1f} | {med(q1[m]):.1f} | "
                   f"{med(q2[m]):.1f} | {med(q3[m]):.1f} | {med(last[m]):.1f} | {pct(end[m], 10):.1f} | "
                   f"{med(end[m]):.1f} | {pct(end[m], 90):.1f} | {end[m].max():.1f} | "
                   f"{med(cl):.1f} / {pct(cl, 90):.1f} / {cl.max():.1f} |")
    out += ["", "Mean end by XCD and wave slot (µs):", "",
            "| XCD | " + " | ".join(f"slot {sl}" for sl in sorted(set(slot.tolist()))) + " |",
            "|---|" + "---|" * len(set(slot.tolist()))]
    for x in sorted(set(xcc.tolist())):
        cells = []
        for sl in sorted(set(slot.tolist())):
            m = (xcc == x) & (slot == sl)
            cells.append(f"{end[m].mean():.1f}" if m.any() else "-")
        out.append(f"| {x} | " + " | ".join(cells) + " |")
    # aggregate rate: each wave's tiles done, linear between its stamps, times the mean bytes per tile
    bpt = kv_bytes / max(int(tiles.sum()), 1)
    marks = np.stack([first, q1, q2, q3, np.maximum(last, q3)], axis=1)
    done = np.stack([np.minimum(1, tiles), np.maximum(1, tiles // 4), np.maximum(2, tiles // 2),
                     np.maximum(3, tiles * 3 // 4), tiles], axis=1).astype(np.float64)
    step = 10.0
    edges = np.arange(0.0, end.max() + step, step)
    prog = np.array([sum(np.interp(t, marks[i], done[i], left=0.0, right=float(tiles[i])) for i in range(n))
                     for t in edges])
    out += ["", f"Aggregate KV rate per {step:.0f} µs window (each wave's tiles interpolated between its stamps, "
            f"{bpt / 1024:.2f} KiB per tile on average), waves still running, and those of them that have consumed "
            f"their last tile (closing and merging their last state):", "",
            "| window (µs) | TB/s | waves running | of them past their last tile |", "|---|---|---|---|"]
    for a, b, pa, pb in zip(edges[:-1], edges[1:], prog[:-1], prog[1:]):
        running = int(((ent <= b) & (end > a)).sum())
        closing = int(((last <= a) & (end > a)).sum())
        out.append(f"| {a:.0f}–{b:.0f} | {(pb - pa) * bpt / (step * 1e-6) / 1e12:.2f} | {running} | {closing} |")
    return "\n".join(out) + "\n"


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed steps before the timed ones (default 100, about 15 ms of decode steps even "
                         "for the shortest workload, after which the clocks have settled; 30 with --prefill, whose "
                         "matrix-bound calls take about 20 back-to-back calls to reach their sustained speed)")
    ap.add_argument("--workload", default="gqa8b", choices=sorted(WORKLOAD_DESC))
    ap.add_argument("--partition-size", type=int, default=-1,
                    help="-1 = the workload's setting (0 = balanced split only)")
    ap.add_argument("--cpu-seqs", type=int, default=-1,
                    help="sequences in the CPU-oracle baseline and check (-1 = as many as fit about 4e9 "
                         "multiply-adds: every sequence of the decode workloads; 0 = skip)")
    ap.add_argument("--seed", type=int, default=None)
    ap.add_argument("--cascade", action="store_true",
                    help="decode with paged_attention_decode_cascade using the workload's sharing arrays")
    ap.add_argument("--no-read-ceiling", "--no-plain-read", dest="no_read_ceiling", action="store_true",
                    help="skip the plain streaming-read measurement reported beside the decode's bandwidth")
    ap.add_argument("--prefill", action="store_true",
                    help="several-token workloads: time paged_attention_prefill (32 query columns per wave) "
                         "instead of paged_attention_varlen")
    ap.add_argument("--flush-mall", choices=["read", "write"], default=None,
                    help="read (or overwrite) 512 MB before every step, outside the timed brackets, so the step's "
                         "KV reads cannot hit what the previous step left in the 256 MB infinity cache")
    ap.add_argument("--timeline", action="store_true",
                    help="run the instrumented library (python -m paged_kv_cache_369_amd.build --timeline) and "
                         "write a per-wave timeline summary of one decode call to --timeline-out")
    ap.add_argument("--timeline-out", default=None, help="where --timeline writes (default profiles/)")
    ap.add_argument("--read-probe", action="store_true",
                    help="time pkv_tile_read (gathered K/V tile reads) per tile size, V load width and depth, and "
                         "write profiles/read_probe_tiles.md")
    ap.add_argument("--read-probe-out", default=None, help="where --read-probe writes (default profiles/)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="instead of the decode step, run a plain device copy of known size (counter scale)")
    ap.add_argument("--summarize-trace", metavar="DIR", help="print a markdown summary of a rocprofv3 --stats run")
    ap.add_argument("--last", type=int, default=0,
                    help="with --summarize-trace: also the mean of each kernel's last N dispatches")
    ap.add_argument("--summarize-traffic", action="store_true", help="write profiles/ HBM traffic summary")
    ap.add_argument("--summarize-counters", action="store_true", help="write profiles/ SQ counter summary")
    ap.add_argument("--utilisation", action="store_true",
                    help="print KV utilisation, max-length reservation vs paging, per workload (host only)")
    ap.add_argument("--counters", action="append", dest="counter_dirs", default=[],
                    help="a rocprofv3 --pmc output directory (repeatable)")
    ap.add_argument("--out-dir", default=PROFILES, help="where --summarize-traffic writes")
    ap.add_argument("--copy-fetch"); ap.add_argument("--copy-write")
    ap.add_argument("--dec-fetch"); ap.add_argument("--dec-write")
    ap.add_argument("--command", action="append", dest="commands", default=[],
                    help="command line recorded in a summary (repeatable)")
    args = ap.parse_args()
    if args.warmup is None:
        args.warmup = 30 if args.prefill else 100

    if args.summarize_trace:
        return summarize_trace(args.summarize_trace, " && ".join(args.commands), args.last)
    if args.utilisation:
        return utilisation(args)
    if args.summarize_counters:
        return summarize_counters(args)
    if args.summarize_traffic:
        return summarize_traffic(args)

    if args.gpus != 1:
        print(f"bench.py measures one GPU: this library has no multi-GPU path (got --gpus {args.gpus}). "
              "How the decode would shard over several GPUs is described in the design notes.", file=sys.stderr)
        return 2

    import torch
    import paged_kv_cache_369_amd as pkv
    from paged_kv_cache_369_amd import workloads as W

    if args.timeline:
        from paged_kv_cache_369_amd import build as pkv_build
        if not os.path.exists(pkv_build.OUT_TIMELINE):
            print(f"{pkv_build.OUT_TIMELINE} is not built: python -m paged_kv_cache_369_amd.build --timeline",
                  file=sys.stderr)
            return 2
        pkv._LIB_PATH = pkv_build.OUT_TIMELINE

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2

    if args.copy_calibration:
        return copy_calibration(torch, args.steps)
    if args.read_probe:
        return read_probe(torch, pkv, args.read_probe_out or os.path.join(PROFILES, "read_probe_tiles.md"))

    t0 = time.perf_counter()
    w = W.make(args.workload, args.seed)
    log(f"workload {args.workload} generated in {time.perf_counter() - t0:.1f}s: B={w.num_seqs} "
        f"sum(L)={int(w.context_lens.sum())} blocks={w.layout.num_blocks}")
    part = w.partition_size if args.partition_size < 0 else args.partition_size
    layout = w.layout
    if args.cascade and w.prefix_leader is None:
        print(f"workload {args.workload} declares no shared prefixes", file=sys.stderr)
        return 2
    multi = w.cu_q is not None  # several new query tokens per sequence
    if args.prefill and not multi:
        print(f"workload {args.workload} has one query token per sequence; --prefill needs several", file=sys.stderr)
        return 2

    # device-resident inputs
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.uint8}[w.cache_dtype]
    kc = torch.zeros(pkv.k_cache_shape(layout.num_blocks, w.num_kv_heads, w.head_dim, w.cache_dtype),
                     dtype=tdt, device="cuda")
    vc = torch.zeros(pkv.v_cache_shape(layout.num_blocks, w.num_kv_heads, w.head_dim), dtype=tdt, device="cuda")
    for b in layout.history:
        pkv.paged_kv_write(_dev(b.k, w.in_dtype, torch), _dev(b.v, w.in_dtype, torch), kc, vc,
                           _dev(b.slots, "i32", torch), w.k_scale, w.v_scale)
    torch.cuda.synchronize()
    k_new = _dev(w.new_k, w.in_dtype, torch)
    v_new = _dev(w.new_v, w.in_dtype, torch)
    slots = _dev(layout.new_slots, "i32", torch)
    q = _dev(w.q, w.q_dtype, torch)
    out = torch.empty_like(q)
    bt = _dev(layout.block_table, "i32", torch)
    cl = _dev(w.context_lens, "i32", torch)
    ws_query = (pkv.paged_attention_cascade_workspace_bytes if args.cascade else
                pkv.paged_attention_varlen_workspace_bytes if multi else pkv.paged_attention_workspace_bytes)
    ws_bytes = ws_query(w.num_seqs, w.num_heads, w.num_kv_heads, w.head_dim, w.max_blocks_per_seq, W.BLOCK_SIZE,
                        part)
    if args.cascade:
        pl = _dev(w.prefix_leader, "i32", torch)
        pbl = _dev(w.prefix_blocks, "i32", torch)
    if multi:
        cuq = _dev(w.cu_q, "i32", torch)
        max_q = int(np.max(np.diff(w.cu_q)))
    ws = torch.zeros(max(ws_bytes, 16), dtype=torch.uint8, device="cuda")
    log(f"resident: pools {2 * kc.numel() * kc.element_size() / 1e9:.2f} GB, workspace {ws_bytes / 1e6:.1f} MB")

    # Each step's two launches are prepared once (arguments marshalled, C calls recorded), as a serving
    # loop would: the timed loop then costs the host a C call per launch, so the GPU does not wait on
    # Python between the write and the decode.
    write = pkv.prepare(pkv.paged_kv_write, k_new, v_new, kc, vc, slots, w.k_scale, w.v_scale)
    if args.cascade:
        decode = pkv.prepare(pkv.paged_attention_decode_cascade, out, q, kc, vc, bt, cl, pl, pbl, w.scale,
                             w.k_scale, w.v_scale, partition_size=part, workspace=ws)
    elif args.prefill:
        decode = pkv.prepare(pkv.paged_attention_prefill, out, q, cuq, kc, vc, bt, cl, w.scale, max_q,
                             w.k_scale, w.v_scale)
    elif multi:
        decode = pkv.prepare(pkv.paged_attention_varlen, out, q, cuq, kc, vc, bt, cl, w.scale, w.k_scale,
                             w.v_scale, partition_size=part, workspace=ws)
    else:
        decode = pkv.prepare(pkv.paged_attention_decode, out, q, kc, vc, bt, cl, w.scale, w.k_scale, w.v_scale,
                             partition_size=part, workspace=ws)

    for _ in range(args.warmup):
        write()
        decode()
    torch.cuda.synchronize()

    # Exactly K steps between two synchronisations; HIP events on the launch
    # stream (torch's current stream, which the binding passes to the library)
    # bracket the write and the decode call of every step.
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    # --flush-mall: before every step, outside the event brackets, stream a buffer of twice the
    # 256 MB infinity cache through it (reading, or writing), so the KV reads of the step cannot hit
    # data the previous step left there
    flush = torch.ones(128 << 20, dtype=torch.float32, device="cuda") if args.flush_mall else None
    flush_sink = torch.empty((), dtype=torch.float32, device="cuda") if args.flush_mall else None
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for e in ev:
        if flush is not None:
            if args.flush_mall == "read":
                torch.sum(flush, dim=0, out=flush_sink)
            else:
                flush.fill_(1.0)
        e[0].record()
        write()
        e[1].record()
        decode()
        e[2].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    if args.timeline:
        # one more step after the timed ones, its decode waves' stamps read back
        lib = pkv._load()
        lib.pkv_timeline_read.argtypes = [ctypes.c_void_p, ctypes.c_int]
        if lib.pkv_timeline_clear() != 0:
            raise RuntimeError("pkv_timeline_clear failed")
        write()
        decode()
        torch.cuda.synchronize()
        rows = np.zeros((4096, 8), dtype=np.uint64)
        if lib.pkv_timeline_read(rows.ctypes.data, 4096) != 0:
            raise RuntimeError("pkv_timeline_read failed")
        kvb = (cascade_read_bytes(w) if args.cascade else varlen_read_bytes(w) if multi else w.kv_bytes())
        argv, skip = [], False
        for a in sys.argv[1:]:  # the command as run, without where it wrote
            if skip or a.startswith("--timeline-out"):
                skip = a == "--timeline-out"
                continue
            argv.append(a)
        cmd = "python -m paged_kv_cache_369_amd.build --timeline && python3 bench.py " + " ".join(argv)
        text = timeline_summary(rows, kvb, WORKLOAD_DESC[args.workload] + (CASCADE_NOTE if args.cascade else ""),
                                cmd)
        path = args.timeline_out or os.path.join(PROFILES, f"paged_decode_{profile_key(args)}_timeline.md")
        with open(path, "w") as f:
            f.write(text)
        print(text)
        return 0
    if flush is not None:  # the flush is not part of the step: time the step from its events
        ms_per_step = float(np.mean([e[0].elapsed_time(e[2]) for e in ev]))
    t_write = np.array([e[0].elapsed_time(e[1]) for e in ev]) * 1e3
    t_dec = np.array([e[1].elapsed_time(e[2]) for e in ev]) * 1e3
    dec_us = float(np.mean(t_dec))
    kv_bytes = (cascade_read_bytes(w) if args.cascade else prefill_read_bytes(w) if args.prefill else
                varlen_read_bytes(w) if multi else w.kv_bytes())
    rows = int(q.shape[0])  # query tokens per step
    achieved = kv_bytes / (dec_us * 1e-6) / 1e9
    log(f"timed {args.steps} steps: {ms_per_step:.4f} ms/step; events: write {np.mean(t_write):.1f} us, "
        f"decode call {dec_us:.1f} us (p10 {np.percentile(t_dec, 10):.1f}, p90 {np.percentile(t_dec, 90):.1f}), "
        f"KV {kv_bytes / 1e9:.3f} GB -> {achieved:.0f} GB/s")

    traffic, traffic_src = load_traffic(profile_key(args))
    overhead = {"q_bytes": q.numel() * q.element_size(), "out_bytes": out.numel() * out.element_size(),
                "block_table_bytes": bt.numel() * 4, "context_lens_bytes": cl.numel() * 4}
    result = {
        "metric": "paged-attn decode tokens/s and achieved KV-read GB/s (% HBM peak), 1 GPU",
        "value": rows / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"f32": "f32", "bf16": "bf16", "fp8": "fp8-e4m3"}[w.cache_dtype],
        "data": "synthetic",
        "config": {"workload": WORKLOAD_DESC[args.workload], "name": args.workload, "batch": w.num_seqs,
                   "num_heads": w.num_heads, "num_kv_heads": w.num_kv_heads, "head_dim": w.head_dim,
                   "block_size": W.BLOCK_SIZE, "kv_dtype": w.cache_dtype, "q_dtype": w.q_dtype,
                   "sum_context": int(w.context_lens.sum()),
                   "partition_size": part, "kv_bytes": kv_bytes, "kv_unique_bytes": w.kv_unique_bytes(),
                   "kv_logical_bytes": w.kv_bytes(), "mall_flush": args.flush_mall, "query_rows": rows,
                   "decode": ("paged_attention_decode_cascade" if args.cascade else
                              "paged_attention_prefill" if args.prefill else
                              "paged_attention_varlen" if multi else "paged_attention_decode")},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS,
                     "traffic": traffic,
                     "traffic_source": traffic_src,
                     "kernel": (" + ".join(call_kernels(args)) + " (the whole call)"),
                     "avg_us": dec_us,
                     "p10_us": float(np.percentile(t_dec, 10)), "p90_us": float(np.percentile(t_dec, 90)),
                     "algorithmic_bytes_per_call": kv_bytes},
        "write_us": float(np.mean(t_write)),
        "attention_tokens_per_s": rows / (dec_us * 1e-6),
        "overhead_bytes": overhead,
        "cpu_baseline": None,
        "check": None,
    }

    if args.prefill:
        # a contraction over the visible positions: priced against the matrix cores' dense bf16 peak
        fl = prefill_flops(w)
        tf = fl / (dec_us * 1e-6) / 1e12
        result["roofline"] = {"bound": "mfma", "achieved": tf, "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                              "frac": tf / MFMA_BF16_PEAK_TFLOPS, "traffic": traffic, "traffic_source": traffic_src,
                              "kernel": ("paged_prefill_kernel" if w.cache_dtype == "f32" else "paged_prefill_lds_kernel") + " (the whole prefill call)", "avg_us": dec_us,
                              "algorithmic_flops_per_call": fl, "kv_read_bytes_bound": kv_bytes}
        log(f"prefill: {fl / 1e9:.1f} GFLOP per call -> {tf:.1f} TFLOP/s")

    if not args.no_read_ceiling and result["roofline"]["bound"] == "hbm":
        result["plain_read"] = plain_read(torch, pkv, kv_bytes)
        log(f"plain streaming read on this GPU: {result['plain_read']['GBps']:.0f} GB/s "
            f"(decode reaches {achieved / result['plain_read']['GBps']:.1%} of it)")

    if args.cpu_seqs != 0:
        n, nrows, dt, times, cores, err = oracle_baseline(w, out, w.q_dtype, args.cpu_seqs)
        tok = int(w.context_lens[:n].sum())
        sample_kv = tok * w.num_kv_heads * w.head_dim * 2 * w.kv_elt_bytes()  # each sampled context once
        result["cpu_baseline"] = {
            "value": nrows / dt, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"{n} of {w.num_seqs} sequences of this workload ({nrows} query tokens, all {w.num_heads} "
                      f"heads, {tok} context tokens, one step); median of {CPU_RUNS} timed runs after one "
                      f"warm-up, {dt:.2f} s each, on {cores} threads of {cpu_model()}",
            "GBps": sample_kv / dt / 1e9, "kv_bytes": sample_kv, "runs": CPU_RUNS, "warmup": 1,
            "run_s": [round(t, 4) for t in times], "median_s": dt, "cpu_model": cpu_model(),
        }
        result["check"] = {"max_abs_err_vs_oracle": err, "tolerance": TOL[w.cache_dtype], "seqs": n,
                           "pass": bool(err <= TOL[w.cache_dtype])}
        log(f"cpu oracle: {n} seqs in {dt:.2f}s on {cores} threads; max|gpu-oracle| = {err:.3e}")

    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
