"""Host-side accounting of bench.py: flops and bytes per call, and where counter summaries live.

Checked against brute-force counts on small workloads, so a wrong term in the closed forms bench.py uses
for the roofline fails here (CPU only)."""
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from paged_kv_cache_369_amd import workloads as W  # noqa: E402


def _multi():
    return W.make_multi("acct", 3, [40, 520, 33, 5, 16, 200], [40, 100, 3, 5, 0, 37], 32, 8, 64, "bf16", "bf16")


def test_prefill_flops_brute_force():
    w = _multi()
    vis = 0
    for s, L in enumerate(w.context_lens.tolist()):
        n = int(w.cu_q[s + 1] - w.cu_q[s])
        for i in range(n):
            vis += L - n + i + 1  # positions the i-th new token sees
    assert bench.prefill_flops(w) == 4 * w.head_dim * w.num_heads * vis


def test_prefill_and_varlen_read_bytes_brute_force():
    w = _multi()
    elt = w.kv_elt_bytes()
    row = w.num_kv_heads * w.head_dim * 2 * elt  # K and V of one position, all KV heads

    def per_group(tpw):
        tot = 0
        for s, L in enumerate(w.context_lens.tolist()):
            n = int(w.cu_q[s + 1] - w.cu_q[s])
            for t0 in range(0, n, tpw):
                tot += L - n + min(t0 + tpw, n)  # the group reads up to its last token
        return tot

    G = w.num_heads // w.num_kv_heads
    assert bench.prefill_read_bytes(w) == per_group(32 // G) * row
    rh = bench.run_heads(G)
    assert bench.varlen_read_bytes(w) == per_group(16 // rh) * (w.num_heads // rh) * w.head_dim * 2 * elt


def test_run_heads_matches_the_library_rule():
    # largest divisor of the group that is at most 16
    for g in range(1, 65):
        want = max(d for d in range(1, min(g, 16) + 1) if g % d == 0)
        assert bench.run_heads(g) == want


def test_cascade_read_bytes_on_the_prefix_workload():
    w = W.make_scaled("prefix", max_seqs=16)
    members = 16 // bench.run_heads(w.num_heads // w.num_kv_heads)
    tokens = 0
    for s, L in enumerate(w.context_lens.tolist()):
        pb = min(max(int(w.prefix_blocks[s]), 0), L // 16)
        if pb and (s - int(w.prefix_leader[s])) % members == 0:
            tokens += 16 * pb  # a chunk's first member reads the shared blocks for the chunk
        tokens += L - 16 * pb
    assert bench.cascade_read_bytes(w) == tokens * w.num_kv_heads * w.head_dim * 2 * w.kv_elt_bytes()
    assert bench.cascade_read_bytes(w) < w.kv_bytes()


def test_counter_summary_paths():
    assert bench.traffic_file("gqa8b").endswith("profiles/paged_decode_gqa8b_hbm_traffic.json")
    assert bench.traffic_file("prefix-cascade").endswith("profiles/paged_decode_prefix-cascade_hbm_traffic.json")
    assert bench.traffic_file("chunk512-prefill").endswith("profiles/paged_prefill_chunk512_hbm_traffic.json")



def test_timeline_summary_on_made_up_stamps():
    """Two slots of waves with known stamps: the per-slot medians, the close time after the last tile and the
    aggregate rate (all tiles of every wave, spread over its stamps) come out as constructed."""
    n, tiles, tb = 64, 96, 4096
    rows = np.zeros((4096, 8), dtype=np.uint64)
    t0 = 10 ** 9
    slot = np.arange(n) % 2
    first = t0 + 800 + 400 * slot                       # 8 / 12 us
    run = 10000 + 2000 * slot                           # 100 / 120 us of streaming
    rows[:n, 0] = t0
    rows[:n, 1] = first
    for k in (1, 2, 3):
        rows[:n, 1 + k] = first + run * k // 4
    last = first + run
    rows[:n, 5] = last + 300                            # 3 us closing the last state
    rows[:n, 6] = slot.astype(np.uint64) | (np.uint64(5) << np.uint64(32)) | (np.uint64(tiles) << np.uint64(40))
    rows[:n, 7] = last
    text = bench.timeline_summary(rows, n * tiles * tb, "made up", "cmd")
    lines = {ln.split("|")[1].strip(): ln for ln in text.splitlines() if ln.startswith("| 0 |") or ln.startswith("| 1 |")}
    cells0 = [c.strip() for c in lines["0"].split("|")[1:-1]]
    cells1 = [c.strip() for c in lines["1"].split("|")[1:-1]]
    assert cells0[1] == "32" and cells0[3] == "8.0" and cells0[7] == "108.0" and cells0[9] == "111.0"
    assert cells1[3] == "12.0" and cells1[7] == "132.0" and cells1[12] == "3.0 / 3.0 / 3.0"
    assert "Last wave ends at 135.0" in text
    # the rate windows add up to every tile once
    rates = [float(ln.split("|")[2]) for ln in text.splitlines() if "–" in ln and ln.startswith("| ")]
    total = sum(r * 1e12 * 10e-6 for r in rates)
    assert abs(total - n * tiles * tb) / (n * tiles * tb) < 0.02
