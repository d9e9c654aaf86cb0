"""Benchmark: paged-attention decode on one MI355X.

One step = the whole hot path for one decode iteration of the batch: the
write of every sequence's new token into the paged pools (paged_kv_write),
then paged attention over every sequence's full context (the decode kernel,
plus the split-K merge kernel when a sequence spans several partitions).
Inputs are synthetic and already resident in HBM when timing starts.

Default workload: Llama-3-8B-shaped GQA decode -- 256 sequences, 32 query
heads sharing 8 KV heads, head_dim 128, bf16 pools in 16-token blocks,
context lengths log-uniform in [256, 8192], physical blocks shuffled.

Prints one JSON line.  `value` is decode tokens/s (sequences advanced by one
token per second).  `roofline` rates the decode call against MI355X HBM peak
using the algorithmic KV bytes (sum_s L_s * H_kv * D * 2 * elt) and the
decode call's average duration from HIP events on the launch stream.
`cpu_baseline` times the CPU oracle on a bounded sample of the same workload.

    python bench.py [--gpus 1] [--steps 50] [--warmup 10] [--workload gqa8b]
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
WORKLOAD_DESC = {
    "tiny": "tiny fp32 paged decode: lens {7,16,33,100}, 4/4 heads, D=64",
    "13b": "LLaMA-2-13B-shaped bf16 decode: B=64, 40/40 heads, D=128, lens U[128,2048]",
    "gqa8b": "Llama-3-8B-shaped GQA bf16 decode: B=256, 32 q / 8 kv heads, D=128, lens log-U[256,8192]",
    "prefix": "shared-prefix bf16 decode: 32 prompts x 8 samples, 32/8 heads, D=128, 1024-token aliased prefix",
    "longfp8": "long-context fp8-e4m3 KV decode: B=16, 64 q / 8 kv heads, D=128, lens U[16384,32768], 512-token partitions",
}


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


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


def cpu_baseline(w, host_pools, n_seqs, threads=0):
    """Time the CPU oracle (as it stands) on the first n_seqs sequences, all heads."""
    import oracle  # test infrastructure, used only for this reported baseline
    kp, vp = host_pools
    lo = slice(0, n_seqs)
    t0 = time.perf_counter()
    out = oracle.paged_attention(np.ascontiguousarray(w.q[lo]), w.q_dtype, kp, vp, w.cache_dtype,
                                 np.ascontiguousarray(w.layout.block_table[lo]),
                                 np.ascontiguousarray(w.context_lens[lo]), w.scale, w.k_scale, w.v_scale,
                                 threads=threads)
    dt = time.perf_counter() - t0
    return out, dt, oracle.num_threads(threads)


COPY_BYTES = 1 << 30


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


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="gqa8b", choices=sorted(WORKLOAD_DESC))
    ap.add_argument("--partition-size", type=int, default=-1, help="-1 = the workload's setting")
    ap.add_argument("--cpu-seqs", type=int, default=12, help="sequences in the CPU-oracle sample (0 = skip)")
    ap.add_argument("--seed", type=int, default=None)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="instead of the decode step, run a plain device copy of known size (HBM counter scale)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only (this build has no multi-GPU path); got --gpus {args.gpus}",
              file=sys.stderr)
        return 2

    import torch
    import paged_kv_cache_369_amd as pkv
    from paged_kv_cache_369_amd import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2

    if args.copy_calibration:
        return copy_calibration(torch, args.steps)

    t0 = time.perf_counter()
    w = W.make(args.workload, args.seed)
    log(f"workload {args.workload} generated in {time.perf_counter() - t0:.1f}s: B={w.num_seqs} "
        f"sum(L)={int(w.context_lens.sum())} blocks={w.layout.num_blocks}")
    part = w.partition_size if args.partition_size < 0 else args.partition_size
    layout = w.layout

    # device-resident inputs
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.uint8}[w.cache_dtype]
    shp = (layout.num_blocks, w.num_kv_heads, W.BLOCK_SIZE, w.head_dim)
    kc = torch.zeros(shp, dtype=tdt, device="cuda")
    vc = torch.zeros(shp, dtype=tdt, device="cuda")
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
    ws_bytes = pkv.paged_attention_workspace_bytes(w.num_seqs, w.num_heads, w.head_dim, w.max_blocks_per_seq,
                                                   W.BLOCK_SIZE, part)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device="cuda")
    log(f"resident: pools {2 * kc.numel() * kc.element_size() / 1e9:.2f} GB, workspace {ws_bytes / 1e6:.1f} MB")

    def step():
        pkv.paged_kv_write(k_new, v_new, kc, vc, slots, w.k_scale, w.v_scale)
        pkv.paged_attention_decode(out, q, kc, vc, bt, cl, w.scale, w.k_scale, w.v_scale, partition_size=part,
                                   workspace=ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # wall-clock over exactly K steps
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    log(f"timed {args.steps} steps: {ms_per_step:.4f} ms/step")

    # per-call durations from HIP events on the launch stream (torch's current stream)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    for e in ev:
        e[0].record()
        pkv.paged_kv_write(k_new, v_new, kc, vc, slots, w.k_scale, w.v_scale)
        e[1].record()
        pkv.paged_attention_decode(out, q, kc, vc, bt, cl, w.scale, w.k_scale, w.v_scale, partition_size=part,
                                   workspace=ws)
        e[2].record()
    torch.cuda.synchronize()
    t_write = np.array([e[0].elapsed_time(e[1]) for e in ev])
    t_dec = np.array([e[1].elapsed_time(e[2]) for e in ev])
    dec_ms = float(np.mean(t_dec))
    kv_bytes = w.kv_bytes()
    achieved = kv_bytes / (dec_ms * 1e-3) / 1e9
    log(f"events: write {np.mean(t_write) * 1e3:.1f} us, decode call {dec_ms * 1e3:.1f} us "
        f"(p10 {np.percentile(t_dec, 10) * 1e3:.1f}, p90 {np.percentile(t_dec, 90) * 1e3:.1f}), "
        f"KV {kv_bytes / 1e9:.3f} GB -> {achieved:.0f} GB/s")

    result = {
        "metric": "paged-attn decode tokens/s and achieved KV-read GB/s (% HBM peak), 1 GPU",
        "value": w.num_seqs / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"f32": "f32", "bf16": "bf16", "fp8": "fp8-e4m3 KV, bf16 q/out, f32 accumulate"}[w.cache_dtype],
        "data": "synthetic",
        "config": {"workload": WORKLOAD_DESC[args.workload], "name": args.workload, "batch": w.num_seqs,
                   "num_heads": w.num_heads, "num_kv_heads": w.num_kv_heads, "head_dim": w.head_dim,
                   "block_size": W.BLOCK_SIZE, "sum_context": int(w.context_lens.sum()),
                   "partition_size": part or pkv.DEFAULT_PARTITION, "kv_bytes": kv_bytes},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": None,
                     "kernel": "decode call (paged_decode_kernel + paged_reduce_kernel)",
                     "avg_us": dec_ms * 1e3},
        "write_us": float(np.mean(t_write) * 1e3),
        "attention_tokens_per_s": w.num_seqs / (dec_ms * 1e-3),
        "cpu_baseline": None,
    }

    if args.cpu_seqs > 0:
        import oracle
        t0 = time.perf_counter()
        npd = {"f32": np.float32, "bf16": np.uint16, "fp8": np.uint8}[w.cache_dtype]
        kp = np.zeros(shp, dtype=npd)
        vp = np.zeros(shp, dtype=npd)
        for b in layout.history:
            oracle.kv_write(b.k, b.v, w.in_dtype, kp, vp, w.cache_dtype, b.slots, k_scale=w.k_scale,
                            v_scale=w.v_scale)
        oracle.kv_write(w.new_k, w.new_v, w.in_dtype, kp, vp, w.cache_dtype, layout.new_slots,
                        k_scale=w.k_scale, v_scale=w.v_scale)
        log(f"oracle pools built in {time.perf_counter() - t0:.1f}s")
        n = min(args.cpu_seqs, w.num_seqs)
        ref, dt, cores = cpu_baseline(w, (kp, vp), n)
        got = out[:n].float().cpu().numpy().astype(np.float64)
        err = float(np.max(np.abs(got - ref)))
        tok = int(w.context_lens[:n].sum())
        result["cpu_baseline"] = {
            "value": n / dt, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"first {n} of {w.num_seqs} sequences (all {w.num_heads} heads, {tok} context tokens), "
                      f"{dt:.1f} s on {cpu_model()}",
        }
        result["check"] = {"max_abs_err_vs_oracle": err, "seqs": n}
        log(f"cpu oracle: {n} seqs in {dt:.2f}s on {cores} threads; max|gpu-oracle| on them = {err:.3e}")

    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
