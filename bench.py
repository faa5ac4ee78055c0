"""Throughput of the MI355X ring-attention forward on one GPU.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-extras] [--no-cpu]

A step is one pass of the whole hot path over one batch of synthetic input:
the long-context GQA causal workload (batch 1, 524288 tokens, 32 query heads
over 8 key/value heads, d = 128, bf16, N(0,1)) processed as the 8-device
ZigZag ring schedule (16 chunks of 32768) of every device in one launch of
rattn_fwd_queued: every query tile walks its device's key/value chunks in ring
order, skips fully masked tiles, masks the diagonal ones, keeps the online
softmax in registers and merges the ring steps in place (one running max, sum
and accumulator per row), dividing by the sum once at the end; the query
tiles are handed to a persistent grid from per-XCD queues.  The same
workload through rattn_fwd (one workgroup per query tile) is an extra.

`value` is causal-adjusted TFLOP/s: 4*d FLOP per visible (query, key) pair
per query head (2d for QK^T, 2d for PV; exponentials and masked work are not
counted), pairs counted from the positions alone.  Timing uses HIP events on
the stream the kernels run on; inputs are resident in HBM before timing.

Also reported: the roofline entry of the dominant kernel (MFMA bound, against
the 2.5 PFLOP/s dense bf16 peak, and that peak restated from the device's CU
count and clock), the fp64 CPU oracle timed on a bounded sample of the same
workload, and other workloads timed the same way (extras), among them one
device's share of the 131072-token ZigZag ring run as 8 ring-step launches
with the log-sum-exp merge in their epilogues (with its own roofline entry).
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16/fp16 MFMA, published
MFMA_BF16_FLOP_PER_CLK_CU = 4096  # 4 SIMDs x one 32x32x16 bf16 MFMA (32768 FLOP) per 32 clocks
# the dominant kernel of the headline workload (d = 128, 16-bit, output in the input type)
HEADLINE_KERNEL = "rattn::fwd_mfma128_queue_kernel<rattn::Bf16, 128, false, true>"
# the ring-step kernel (d = 128, 16-bit, float32 partials merged in the epilogue)
STEP_KERNEL = "rattn::fwd_mfma128_kernel<rattn::Bf16, 128, true, true>"
# sources the d = 128 kernel is built from; a stored counter summary is valid
# only for the kernel it was measured on
KERNEL_SOURCES = ("fwd_mfma128.hip", "kcommon.h", "ring_sched.h", "launch.h", "lds_dma.h")
HEADLINE_COUNTERS = os.path.join(ROOT, "profiles",
                                 "fwd_mfma128_queue_gqa_causal_512k_bf16_hbm_counters.txt")
COUNTER_SUMMARY = os.path.join(ROOT, "profiles",
                               "fwd_mfma128_zigzag_rank2_131k_bf16_hbm_counters.txt")
HEADLINE_WORKLOAD = 5
METRIC = "attention fwd TFLOP/s (causal-adjusted) and % of bf16 MFMA peak, 1 MI355X"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--no-extras", action="store_true", help="skip the other workloads")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-rows", type=int, default=2048,
                    help="query rows of the workload the CPU oracle times")
    ap.add_argument("--kernel", default=None,
                    help="kernel the --summarize-counters / --summarize-mfma summaries are "
                         "about (default: the headline workload's kernel)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="first run one plain 1 GiB device-to-device copy, whose byte "
                         "counters calibrate the kernels' FETCH_SIZE/WRITE_SIZE readings")
    ap.add_argument("--small-d-only", action="store_true",
                    help="run only the small head-dim sweep (after --copy-probe, if given) "
                         "and print its JSON")
    ap.add_argument("--layouts-only", action="store_true",
                    help="run only the causal layout comparison and print its JSON")
    ap.add_argument("--bwd-only", action="store_true",
                    help="run only the backward measurements and print their JSON")
    ap.add_argument("--single-head-only", action="store_true",
                    help="only the single-head 4096-token workload through rattn_fwd "
                         "(the key-split kernel)")
    ap.add_argument("--ring-share-only", action="store_true",
                    help="run only the 131072-token ZigZag ring share (ring steps, fused) "
                         "and print its JSON")
    ap.add_argument("--summarize-stats", metavar="KERNEL_STATS_CSV",
                    help="print a summary of a rocprofv3 --stats kernel_stats.csv and exit")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="print the HBM traffic summary of two rocprofv3 --pmc runs "
                         "(FETCH_SIZE, then WRITE_SIZE; counter_collection.csv) and exit")
    ap.add_argument("--summarize-kernels", nargs=3, metavar=("FETCH_CSV", "WRITE_CSV", "SQ_CSV"),
                    help="print per-kernel HBM GB/s and MFMA busy from three rocprofv3 --pmc "
                         "runs (FETCH_SIZE, WRITE_SIZE, SQ counters) and exit")
    ap.add_argument("--summarize-waits", metavar="SQ_CSV",
                    help="wave time shares of every library kernel from an SQ wait-counter pass")
    ap.add_argument("--summarize-mfma", metavar="SQ_CSV",
                    help="print MFMA / VALU / LDS utilisation of the step kernel from a "
                         "rocprofv3 --pmc run of the SQ counters and GRBM_GUI_ACTIVE and exit")
    return ap.parse_args()


# ------------------------------------------------------------ profile summaries

def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "ring_attention_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def _short_name(name: str) -> str:
    name = name.replace("(anonymous namespace)::", "").replace("void ", "")
    return name.split("(")[0]


def summarize_stats(path: str) -> None:
    """Top kernels of a rocprofv3 --stats run: calls, average and total time."""
    rows = list(csv.DictReader(open(path)))
    print(f"{'kernel':60s} {'calls':>6s} {'avg_us':>10s} {'total_ms':>10s} {'pct':>6s}")
    for r in rows[:12]:
        print(f"{_short_name(r['Name'])[:60]:60s} {int(r['Calls']):6d} "
              f"{float(r['AverageNs']) / 1e3:10.1f} {float(r['TotalDurationNs']) / 1e6:10.3f} "
              f"{float(r['Percentage']):6.2f}")


def _counter_means(path: str, counter: str):
    per = {}
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter:
            continue
        per.setdefault(_short_name(r["Kernel_Name"]), []).append(float(r["Counter_Value"]))
    return per


def summarize_counters(fetch_csv: str, write_csv: str, kernel: str) -> None:
    """HBM bytes per launch of the step kernel from FETCH_SIZE / WRITE_SIZE (KiB per
    dispatch), each scaled by what the same counter reads for the 1 GiB copy of
    --copy-probe (the largest copy dispatch in the run)."""
    fetch = _counter_means(fetch_csv, "FETCH_SIZE")
    write = _counter_means(write_csv, "WRITE_SIZE")
    gib_kib = float(1 << 20)
    copy_f = max(v for n, vs in fetch.items() if "copy" in n for v in vs)
    copy_w = max(v for n, vs in write.items() if "copy" in n for v in vs)
    f_scale, w_scale = gib_kib / copy_f, gib_kib / copy_w
    kf, kw = fetch[kernel], write[kernel]
    fetch_b = sum(kf) / len(kf) * 1024 * f_scale
    write_b = sum(kw) / len(kw) * 1024 * w_scale
    print(f"kernel: {kernel}")
    print(f"kernel_source_sha256_16: {kernel_source_hash()}")
    print(f"copy_probe_fetch_kib: {copy_f:.0f}  (1 GiB copy; scale {f_scale:.4f})")
    print(f"copy_probe_write_kib: {copy_w:.0f}  (1 GiB copy; scale {w_scale:.4f})")
    print(f"kernel_dispatches: {len(kf)} {len(kw)}")
    print(f"kernel_fetch_kib_avg: {sum(kf) / len(kf):.1f}")
    print(f"kernel_write_kib_avg: {sum(kw) / len(kw):.1f}")
    print(f"kernel_hbm_read_bytes_per_launch: {fetch_b:.0f}")
    print(f"kernel_hbm_write_bytes_per_launch: {write_b:.0f}")
    print(f"kernel_hbm_bytes_per_launch: {fetch_b + write_b:.0f}")


def summarize_mfma(path: str, kernel: str) -> None:
    """Matrix-core utilisation of the step kernel: SQ_VALU_MFMA_BUSY_CYCLES over
    the SIMD-cycles of the dispatch (GRBM_GUI_ACTIVE is summed over the 8 XCDs,
    each with 32 CUs x 4 SIMDs), plus instruction counts per dispatch."""
    per, dur = {}, {}
    for r in csv.DictReader(open(path)):
        if _short_name(r["Kernel_Name"]) != kernel:
            continue
        key = r["Dispatch_Id"]
        per.setdefault(key, {})[r["Counter_Name"]] = float(r["Counter_Value"])
        dur[key] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9
    n = len(per)
    avg = {c: sum(d[c] for d in per.values()) / n for c in next(iter(per.values()))}
    t = sum(dur.values()) / n
    xcd_cycles = avg["GRBM_GUI_ACTIVE"] / 8
    simd_cycles = xcd_cycles * 8 * 32 * 4
    print(f"kernel: {kernel}")
    print(f"kernel_source_sha256_16: {kernel_source_hash()}")
    print(f"dispatches: {n}")
    print(f"avg_duration_us: {t * 1e6:.1f}")
    print(f"clock_ghz_from_grbm: {xcd_cycles / t / 1e9:.3f}")
    print(f"mfma_busy_fraction: {avg['SQ_VALU_MFMA_BUSY_CYCLES'] / simd_cycles:.4f}")
    print(f"mfma_issued_tflops: {avg['SQ_INSTS_MFMA'] * 32768 / t / 1e12:.1f}"
          "  (every v_mfma_f32_32x32x16 counted as 32768 FLOP, masked work included)")
    # SQ_ACTIVE_INST_VALU counts quad-cycles (4 clocks)
    print(f"valu_active_fraction: {4 * avg['SQ_ACTIVE_INST_VALU'] / simd_cycles:.4f}")
    print(f"lds_bank_conflict_cycles: {avg['SQ_LDS_BANK_CONFLICT']:.0f}")
    for c in sorted(avg):
        print(f"  {c}: {avg[c]:.6g}")


def summarize_waits(path: str) -> None:
    """Where the waves of each kernel of this library spend their time, from one
    SQ pass (SQ_WAVE_CYCLES, SQ_WAIT_ANY, SQ_WAIT_INST_ANY, SQ_ACTIVE_INST_ANY,
    SQ_ACTIVE_INST_VALU, SQ_ACTIVE_INST_LDS: quad-cycles summed over waves;
    GRBM_GUI_ACTIVE summed over the 8 XCDs).  Shares are of resident
    wave-time; valu_busy and lds_issue are per SIMD-cycle."""
    per, dur = {}, {}
    for r in csv.DictReader(open(path)):
        name = _short_name(r["Kernel_Name"])
        if not name.startswith("rattn::"):
            continue
        key = (name, r["Dispatch_Id"])
        per.setdefault(key, {})[r["Counter_Name"]] = float(r["Counter_Value"])
        dur[key] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9
    names = sorted({k[0] for k in per})
    print(f"{'kernel':56s} {'n':>5s} {'avg_us':>8s} {'GHz':>5s} {'waves/SIMD':>10s} "
          f"{'wait_any':>8s} {'wait_issue':>10s} {'active':>7s} {'valu_busy':>9s} "
          f"{'lds_issue':>9s}")
    for name in names:
        ks = [k for k in per if k[0] == name]
        n = len(ks)
        avg = {c: sum(per[k].get(c, 0.0) for k in ks) / n for c in per[ks[0]]}
        t = sum(dur[k] for k in ks) / n
        xcd_cycles = avg["GRBM_GUI_ACTIVE"] / 8
        simd_cycles = xcd_cycles * 8 * 32 * 4
        wc = avg["SQ_WAVE_CYCLES"]
        print(f"{name[:56]:56s} {n:5d} {t * 1e6:8.1f} {xcd_cycles / t / 1e9:5.2f} "
              f"{4 * wc / simd_cycles:10.2f} {avg['SQ_WAIT_ANY'] / wc:8.3f} "
              f"{avg['SQ_WAIT_INST_ANY'] / wc:10.3f} {avg['SQ_ACTIVE_INST_ANY'] / wc:7.3f} "
              f"{4 * avg['SQ_ACTIVE_INST_VALU'] / simd_cycles:9.3f} "
              f"{4 * avg['SQ_ACTIVE_INST_LDS'] / simd_cycles:9.3f}")


def summarize_kernels(fetch_csv: str, write_csv: str, sq_csv: str) -> None:
    """Per kernel instantiation of this library: dispatches, average duration,
    HBM bytes per dispatch (FETCH_SIZE + WRITE_SIZE, each scaled by the 1 GiB
    copy of --copy-probe in its run), achieved HBM GB/s, and the matrix-core
    busy fraction and VALU instructions from an SQ counter pass."""
    fetch = _counter_means(fetch_csv, "FETCH_SIZE")
    write = _counter_means(write_csv, "WRITE_SIZE")
    f_scale = float(1 << 20) / max(v for n, vs in fetch.items() if "copy" in n for v in vs)
    w_scale = float(1 << 20) / max(v for n, vs in write.items() if "copy" in n for v in vs)
    per, dur = {}, {}
    for r in csv.DictReader(open(sq_csv)):
        name = _short_name(r["Kernel_Name"])
        if not name.startswith("rattn::"):
            continue
        per.setdefault(name, {}).setdefault(r["Dispatch_Id"], {})[r["Counter_Name"]] = \
            float(r["Counter_Value"])
        dur.setdefault(name, {})[r["Dispatch_Id"]] = \
            (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9
    print(f"{'kernel':58s} {'n':>4s} {'avg_us':>9s} {'HBM_MB':>8s} {'GB/s':>8s} "
          f"{'mfma_busy':>9s} {'valu_instr/disp':>15s}")
    for name in sorted(per):
        d = per[name]
        n = len(d)
        t = sum(dur[name].values()) / n
        avg = {c: sum(x.get(c, 0.0) for x in d.values()) / n for c in next(iter(d.values()))}
        simd_cycles = avg["GRBM_GUI_ACTIVE"] / 8 * 1024
        hbm = None
        if name in fetch and name in write:
            hbm = (sum(fetch[name]) / len(fetch[name]) * f_scale +
                   sum(write[name]) / len(write[name]) * w_scale) * 1024
        print(f"{name[:58]:58s} {n:4d} {t * 1e6:9.1f} "
              f"{(hbm or 0) / 1e6:8.1f} {(hbm or 0) / t / 1e9:8.1f} "
              f"{avg['SQ_VALU_MFMA_BUSY_CYCLES'] / simd_cycles:9.4f} {avg['SQ_INSTS_VALU']:15.4g}")


def stored_traffic(path: str):
    """HBM bytes per launch of a kernel from a committed counter summary, or
    None when it is missing or was measured on other kernel sources."""
    try:
        kv = {}
        for line in open(path):
            if ":" in line and not line.startswith("#"):
                key, val = line.split(":", 1)
                kv[key.strip()] = val.split()[0] if val.split() else ""
        if kv.get("kernel_source_sha256_16") != kernel_source_hash():
            return None
        return int(kv["kernel_hbm_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


# ---------------------------------------------------------------- pair counts

def causal_pairs(q_pos, k_pos):
    """Visible (query, key) pairs: keys with position <= the query's."""
    k_sorted = np.sort(np.asarray(k_pos))
    return int(np.searchsorted(k_sorted, np.asarray(q_pos), side="right").sum())


def runs_positions(runs):
    return np.concatenate([np.arange(a, a + n) for a, n in runs]) if runs else np.zeros(0, int)


# ---------------------------------------------------------------- timing

class Timer:
    """Accumulates HIP-event durations of launches on the current stream."""

    def __init__(self, torch):
        self.torch = torch
        self.pairs = []

    def __call__(self, fn):
        t = self.torch
        a, b = t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True)
        a.record()
        r = fn()
        b.record()
        self.pairs.append((a, b))
        return r

    def total_ms(self):
        self.torch.cuda.synchronize()
        return sum(a.elapsed_time(b) for a, b in self.pairs)


def warm_up(torch, fn, calls, min_s=0.25):
    """Untimed calls before an extra's timing: at least `calls`, and at least
    `min_s` seconds of them, so that a short workload is timed at the clock
    the GPU reaches under load (after a pause it starts lower and ramps up)."""
    t0 = time.perf_counter()
    n = 0
    while n < calls or time.perf_counter() - t0 < min_s:
        fn()
        n += 1
        if n % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()


def loop_ms(torch, fn, reps):
    """Average milliseconds per call of `reps` back-to-back calls, timed by one
    pair of HIP events on the current stream.  Per-call event pairs would also
    count the host's launch overhead whenever the GPU waits for the next call,
    which inflates calls of a few hundred microseconds."""
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        fn()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps


def step_plan(N, W, rank, c):
    """The launches of one ZigZag ring device (as ring.ring_forward_steps runs
    them): per step the query runs, key runs and whether it is merged."""
    from ring_attention_amd import ring
    plan = []
    q_runs = ring.shard_rows(N, W, True, rank)
    for s in range(W):
        src = (rank - s) % W
        k_runs = ring.shard_rows(N, W, True, src)
        if s == 0:
            plan.append((q_runs, k_runs))
        elif s <= rank:
            plan.append((q_runs, k_runs[:1]))
        else:
            plan.append((q_runs[1:], k_runs))
    return plan


def device_peak(torch):
    """The dense bf16 MFMA peak restated from the device: CU count x peak
    engine clock x 4096 FLOP per clock per CU (four SIMDs, each finishing one
    32x32x16 bf16 MFMA of 32768 FLOP every 32 clocks).  The clock comes from
    hipDeviceGetAttribute of the HIP runtime this process already uses."""
    import ctypes
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    clk_khz = None
    try:
        hip = ctypes.CDLL("libamdhip64.so.7")
        val = ctypes.c_int(0)
        # hipDeviceAttributeClockRate = 5, hipDeviceAttributeMultiprocessorCount = 63
        if hip.hipDeviceGetAttribute(ctypes.byref(val), 5, 0) == 0 and 5e5 < val.value < 5e6:
            clk_khz = val.value
        cu = ctypes.c_int(0)
        if hip.hipDeviceGetAttribute(ctypes.byref(cu), 63, 0) != 0 or cu.value != cus:
            clk_khz = None
    except OSError:
        pass
    out = {"published_tflops": PEAK_BF16_TFLOPS, "compute_units": cus,
           "peak_clock_mhz": None if clk_khz is None else clk_khz / 1000,
           "flop_per_clock_per_cu": MFMA_BF16_FLOP_PER_CLK_CU, "from_cus_x_clock_tflops": None}
    if clk_khz is not None:
        out["from_cus_x_clock_tflops"] = round(
            cus * clk_khz * 1e3 * MFMA_BF16_FLOP_PER_CLK_CU / 1e12, 1)
    return out


def headline(torch, binding, workloads, dev, args):
    """The long-context GQA causal workload: one rattn_fwd_queued call per step
    (every device's ZigZag ring schedule), W warm-up steps, K timed steps."""
    w = workloads.workload(HEADLINE_WORKLOAD)
    need = 2 * (w.B * w.Nq * w.Hq * w.d) * 2 + 2 * (w.B * w.N * w.Hkv * w.d) * 2 \
        + w.B * w.Nq * w.Hq * 4
    free, _total = torch.cuda.mem_get_info(dev)
    if free < need * 1.05:
        print(f"bench.py: the {w.name} workload needs {need / 1e9:.1f} GB of device memory, "
              f"{free / 1e9:.1f} GB are free", file=sys.stderr)
        sys.exit(1)
    q, k, v = workloads.make_inputs(w, device=dev)
    queue_ws = binding.queue_workspace(dev)
    torch.cuda.synchronize()
    pairs = w.N * (w.N + 1) // 2  # per head: keys 0..i for query i
    flop = 4 * w.d * w.Hq * w.B * pairs

    def step():
        return binding.fwd_queued(q, k, v, causal=True, n_ring_steps=w.W, zigzag=True, rank=-1,
                                  queue_ws=queue_ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(args.steps):
        step()
    t1.record()
    torch.cuda.synchronize()
    ms_per_step = t0.elapsed_time(t1) / args.steps
    # per-launch HIP events around each call on the stream it runs on (torch's
    # current stream, which the binding passes): one launch of the dominant
    # kernel per step (after a one-wave kernel that zeroes its 8 queue counters)
    kern = Timer(torch)
    for _ in range(args.steps):
        kern(step)
    launch_ms = sorted(a.elapsed_time(b) for a, b in kern.pairs) if kern.total_ms() else []
    avg_launch = sum(launch_ms) / len(launch_ms)
    return w, (q, k, v), flop, pairs, ms_per_step, launch_ms, avg_launch


def ring_share_extra(torch, binding, ring, workloads, dev, args, peak):
    """One simulated device's share of the 8-way ZigZag causal ring over
    131072 tokens (chunks {2, 13}, 8 heads): the device's 8 ring-step launches
    in ring order, steps 2-8 merging into the running (out, lse) in their
    epilogue; the same ring with separate merge launches; the same share in
    one fused rattn_fwd launch.  Carries the step kernel's roofline entry."""
    w = workloads.workload(4)
    W, rank, N, d, Hq = w.W, w.rank, w.N, w.d, w.Hq
    c = N // (2 * W)
    q, k, v = workloads.make_inputs(w, device=dev)
    ks = [ring.shard(k, W, True, r) for r in range(W)]
    vs = [ring.shard(v, W, True, r) for r in range(W)]
    torch.cuda.synchronize()
    plan = step_plan(N, W, rank, c)
    pairs = sum(causal_pairs(runs_positions(qr), runs_positions(kr)) for qr, kr in plan)
    flop = 4 * d * Hq * w.B * pairs
    reps = max(10, 2 * args.steps)

    def one(hook=None, fused_merge=True):
        kw = {} if hook is None else {"hook": hook}
        return ring.ring_forward_steps(q, ks, vs, W, True, rank, causal=True,
                                       fused_merge=fused_merge, **kw)
    warm_up(torch, one, 3)
    ms = loop_ms(torch, one, reps)
    kern, merge_t = Timer(torch), Timer(torch)

    def hook(kind, fn):
        return (kern if kind == "step" else merge_t)(fn)
    for _ in range(reps):
        one(hook)
    kern_ms = kern.total_ms() / len(kern.pairs)
    flop_launch = flop / len(plan)
    achieved = flop_launch / (kern_ms * 1e-3) / 1e12
    warm_up(torch, lambda: one(fused_merge=False), 3)
    sep_ms = loop_ms(torch, lambda: one(fused_merge=False), reps)
    merge_t.pairs.clear()
    for _ in range(reps):
        one(hook, fused_merge=False)
    merge_ms = merge_t.total_ms() / max(1, len(merge_t.pairs))

    def fused():
        return binding.fwd(q, k, v, causal=True, n_ring_steps=W, zigzag=True, rank=rank)
    warm_up(torch, fused, 3)
    fused_ms = loop_ms(torch, fused, reps)
    res = {
        "ring_steps": {"ms": round(ms, 4), "tflops": round(flop / (ms * 1e-3) / 1e12, 2),
                       "pct_of_peak": round(100 * flop / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2),
                       "mode": "8 ring-step launches; steps 2-8 merge into the running "
                               "(out, lse) in the kernel epilogue"},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": stored_traffic(COUNTER_SUMMARY), "kernel": STEP_KERNEL,
                     "avg_launch_ms": round(kern_ms, 4), "launches": len(kern.pairs),
                     "flop_per_launch": flop_launch},
        "steps_separate_merge": {"ms": round(sep_ms, 4),
                                 "tflops": round(flop / (sep_ms * 1e-3) / 1e12, 2),
                                 "merge_avg_ms": round(merge_ms, 4)},
        "fused": {"ms": round(fused_ms, 4), "tflops": round(flop / (fused_ms * 1e-3) / 1e12, 2),
                  "pct_of_peak": round(100 * flop / (fused_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                                       2)},
        "visible_pairs_per_head": pairs, "flop": flop,
        "conventional_flop": 4 * d * Hq * w.B * w.Nq * N // 2,
    }
    del q, k, v, ks, vs
    torch.cuda.empty_cache()
    return {w.name: res}


def device_us(torch, fn, reps=21):
    """Median device time of one call in microseconds: the stream is first
    kept busy by a spin kernel, so the event pair around the call times the
    GPU work (and the gap between its launches), not the host's enqueueing."""
    times = []
    for _ in range(reps):
        torch.cuda._sleep(1_000_000)
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        torch.cuda.synchronize()
        times.append(a.elapsed_time(b) * 1e3)
    return sorted(times)[len(times) // 2]


def tiny_latency_extra(torch, binding, workloads, dev, args):
    """The 4-device x 8-token ring simulation (fp32, d = 16): latency of one
    rattn_fwd call in microseconds -- per call of back-to-back calls under one
    event pair (bounded by the host's Python and allocation overhead), and
    the device time of one call."""
    w = workloads.workload(1)
    q, k, v = workloads.make_inputs(w, device=dev)

    def run():
        return binding.fwd(q, k, v, causal=False, n_ring_steps=w.W, zigzag=False, rank=-1)
    warm_up(torch, run, 10)
    ms = loop_ms(torch, run, 200)
    return {w.name: {"us_per_call": round(ms * 1e3, 2),
                     "device_us": round(device_us(torch, run), 2),
                     "note": "latency bound: 32 query rows, one workgroup"}}


def page_benchmark_sweep(torch, binding, workloads, dev, args):
    """The shapes of the yz520gzy chapter's attention benchmark (B = 2,
    H = 32, D = 128, fp16, non-causal, N = 512 ... 8192; 10 warm-up calls,
    50 timed), through rattn_fwd (which picks its kernel by itself).  Only
    this library is timed: the page's own comparison is not reproduced."""
    out = {}
    for n in (512, 1024, 2048, 4096, 8192):
        q, k, v = workloads.make_qkv(2, n, n, 32, 32, 128, torch.float16, seed=n, device=dev)

        def run():
            return binding.fwd(q, k, v)
        warm_up(torch, run, 10)
        ms = loop_ms(torch, run, 50)
        flop = 4 * 128 * 32 * 2 * n * n
        out[f"page_bench_b2_h32_n{n}_d128_f16"] = {
            "ms": round(ms, 4), "tflops": round(flop / (ms * 1e-3) / 1e12, 2),
            "pct_of_peak": round(100 * flop / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2)}
        del q, k, v
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: --gpus {args.gpus} is not supported "
              "(there is no multi-GPU path)", file=sys.stderr)
        sys.exit(2)
    if args.summarize_stats:
        summarize_stats(args.summarize_stats)
        return
    if args.summarize_counters:
        summarize_counters(*args.summarize_counters, args.kernel or HEADLINE_KERNEL)
        return
    if args.summarize_mfma:
        summarize_mfma(args.summarize_mfma, args.kernel or HEADLINE_KERNEL)
        return
    if args.summarize_kernels:
        summarize_kernels(*args.summarize_kernels)
        return
    if args.summarize_waits:
        summarize_waits(args.summarize_waits)
        return

    import torch

    from ring_attention_amd import binding, ring, workloads

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    binding.load_library()
    dev = torch.device("cuda:0")
    if args.copy_probe:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)  # reads exactly 1 GiB, writes exactly 1 GiB
        torch.cuda.synchronize()
        del src, dst
    if args.small_d_only:
        print(json.dumps({"extras": small_d_sweep(torch, binding, workloads, dev, args)}),
              flush=True)
        return
    if args.layouts_only:
        print(json.dumps({"extras": layout_comparison(torch, binding, ring, workloads, dev,
                                                      args)}), flush=True)
        return
    if args.bwd_only:
        print(json.dumps({"extras": backward_extras(torch, binding, ring, workloads, dev, args)}),
              flush=True)
        return
    if args.ring_share_only:
        print(json.dumps({"extras": ring_share_extra(torch, binding, ring, workloads, dev, args,
                                                     None)}), flush=True)
        return
    if args.single_head_only:
        print(json.dumps({"extras": single_head_extra(torch, binding, workloads, dev, args)}),
              flush=True)
        return
    peak = device_peak(torch)
    w, inputs, flop, pairs, ms_per_step, launch_ms, avg_launch = headline(
        torch, binding, workloads, dev, args)
    value = flop / (ms_per_step * 1e-3) / 1e12
    achieved = flop / (avg_launch * 1e-3) / 1e12
    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "ms_per_step_median": round(launch_ms[len(launch_ms) // 2], 4),
        "ms_per_step_min": round(launch_ms[0], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: N(0,1) bf16 q/k/v from a seeded torch generator, resident in HBM",
        "config": {"workload": w.name, "B": w.B, "Nq": w.Nq, "N": w.N, "Hq": w.Hq,
                   "Hkv": w.Hkv, "d": w.d, "causal": True, "ring": w.W, "zigzag": True,
                   "rank": -1,
                   "mode": "one rattn_fwd_queued call per step: the ZigZag ring schedule of "
                           "all 8 simulated devices (16 chunks of 32768 tokens), ring steps "
                           "merged in place by the online softmax, query tiles handed out from "
                           "per-XCD queues to a persistent grid",
                   "visible_pairs_per_head": pairs,
                   "flop_per_step": flop,
                   # the usual causal estimate, half of all (query, key) pairs
                   "conventional_flop_per_step": 4 * w.d * w.Hq * w.B * w.Nq * w.N // 2},
        "pct_of_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": stored_traffic(HEADLINE_COUNTERS), "kernel": HEADLINE_KERNEL,
                     "avg_launch_ms": round(avg_launch, 4), "launches": len(launch_ms),
                     "flop_per_launch": flop},
        "peak_bf16": peak,
        # context only, not a target: the memory-wall figures of the
        # guijiagi.com ring-attention page (naive attention section) -- a full
        # fp16 score matrix at one million tokens against one GPU's HBM
        "page_context": {
            "score_matrix_1M_tokens_fp16_bytes": 10**6 * 10**6 * 2,
            "page_gpu_hbm_bytes": 80 * 10**9,
            "page_gpu": "unnamed 80 GB GPU",
            "this_gpu_hbm_bytes": 288 * 10**9,
            "score_matrix_bytes_this_workload_if_materialised":
                2 * w.B * w.Hq * w.Nq * w.N,
            "score_bytes_materialised_here": 0},
    }
    if not args.no_cpu:
        q, k, v = inputs
        result["cpu_baseline"] = cpu_baseline(w, q, k, v, args.cpu_rows)
    plain = None
    if not args.no_extras:
        # the same workload through rattn_fwd: one workgroup per query tile
        q, k, v = inputs

        def run_plain():
            return binding.fwd(q, k, v, causal=True, n_ring_steps=w.W, zigzag=True, rank=-1)
        run_plain()
        ms = loop_ms(torch, run_plain, 3)
        plain = {"ms": round(ms, 4), "tflops": round(flop / (ms * 1e-3) / 1e12, 2),
                 "pct_of_peak": round(100 * flop / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2),
                 "entry_point": "rattn_fwd"}
        del q, k, v
    del inputs
    torch.cuda.empty_cache()

    if not args.no_extras:
        extras = {w.name + "_rattn_fwd": plain}

        def workload_extra(idx):
            we = workloads.workload(idx)
            qe, ke, ve = workloads.make_inputs(we, device=dev)
            if we.causal:
                qpos = np.arange(we.Nq)
                pe = causal_pairs(qpos, np.arange(we.N))
            else:
                pe = we.Nq * we.N
            fe = 4 * we.d * we.Hq * we.B * pe
            reps = max(20, 2 * args.steps)

            def run():
                return binding.fwd(qe, ke, ve, causal=we.causal, n_ring_steps=we.W,
                                   zigzag=we.zigzag, rank=we.rank)
            warm_up(torch, run, 5)
            ms = loop_ms(torch, run, reps)
            extras[we.name] = {"ms": round(ms, 4), "tflops": round(fe / (ms * 1e-3) / 1e12, 2),
                               "pct_of_peak": round(100 * fe / (ms * 1e-3) / 1e12
                                                    / PEAK_BF16_TFLOPS, 2)}
            if idx == 2:  # latency-sized: the device time of one call as well
                extras[we.name]["device_us"] = round(device_us(torch, run), 2)
            ns = binding.split_hint(qe, ke, we.W, we.zigzag, we.rank)
            if ns > 1:  # too few query tiles for the GPU: the split-KV entry point
                ws = torch.empty(ns * qe.numel() // we.d * (we.d + 1), dtype=torch.float32,
                                 device=dev)

                def run_split():
                    return binding.fwd_split(qe, ke, ve, causal=we.causal, n_ring_steps=we.W,
                                             zigzag=we.zigzag, rank=we.rank, n_splits=ns, ws=ws)
                warm_up(torch, run_split, 5)
                ms = loop_ms(torch, run_split, reps)
                extras[we.name + "_splitkv"] = {
                    "ms": round(ms, 4), "tflops": round(fe / (ms * 1e-3) / 1e12, 2),
                    "pct_of_peak": round(100 * fe / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2),
                    "n_splits": ns}
                del ws
            del qe, ke, ve
            torch.cuda.empty_cache()

        extras.update(ring_share_extra(torch, binding, ring, workloads, dev, args, peak))
        for idx in (2, 3):
            workload_extra(idx)
        extras.update(tiny_latency_extra(torch, binding, workloads, dev, args))
        extras.update(page_benchmark_sweep(torch, binding, workloads, dev, args))
        extras.update(small_d_sweep(torch, binding, workloads, dev, args))
        extras.update(backward_extras(torch, binding, ring, workloads, dev, args))
        extras.update(layout_comparison(torch, binding, ring, workloads, dev, args))
        extras.update(varlen_extra(torch, binding, workloads, dev, args))
        result["extras"] = extras

    print(json.dumps(result), flush=True)


def backward_extras(torch, binding, ring, workloads, dev, args):
    """Backward (dQ, dK, dV) throughput of the batched causal workload and of
    the ZigZag ring share: whole-schedule calls (rattn_bwd) and, for the ring
    share, the device's W backward ring steps (rattn_bwd_delta + rattn_bwd_step).
    Algorithmic work: 10 d FLOP per visible pair per query head (dP = dO V^T,
    dV, dK, dQ and the recomputed S: five products of 2 d each); the kernels
    issue 14 d (the dQ kernel recomputes S and dP)."""
    res = {}
    for idx in (3, 4):
        w = workloads.workload(idx)
        q, k, v = workloads.make_inputs(w, device=dev)
        g = torch.Generator(device=dev).manual_seed(1000 + idx)
        do = workloads.randn(q.shape, q.dtype, g, dev)
        qpos = runs_positions(ring.shard_rows(w.N, w.W, w.zigzag, w.rank)) \
            if w.rank >= 0 else np.arange(w.N)
        pairs = causal_pairs(qpos, np.arange(w.N)) if w.causal else w.Nq * w.N
        flop = 10 * w.d * w.Hq * w.B * pairs
        out, lse = binding.fwd(q, k, v, causal=w.causal, n_ring_steps=w.W, zigzag=w.zigzag,
                               rank=w.rank)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        ws = torch.empty(lse.shape, dtype=torch.float32, device=dev)

        def run():
            return binding.bwd(q, k, v, out, lse, do, causal=w.causal, n_ring_steps=w.W,
                               zigzag=w.zigzag, rank=w.rank, dq=dq, dk=dk, dv=dv, delta_ws=ws)
        reps = max(3, args.steps // 2)
        warm_up(torch, run, max(1, args.warmup))
        ms = loop_ms(torch, run, reps)
        tf = flop / (ms * 1e-3) / 1e12
        res[w.name + "_bwd"] = {"ms": round(ms, 4), "tflops": round(tf, 2),
                                "pct_of_peak": round(100 * tf / PEAK_BF16_TFLOPS, 2),
                                "flop": flop, "flop_rule": "10 d per visible pair per head"}
        if idx == 4:
            ks = [ring.shard(k, w.W, True, r) for r in range(w.W)]
            vs = [ring.shard(v, w.W, True, r) for r in range(w.W)]

            def run_steps():
                return ring.ring_backward_steps(q, ks, vs, out, lse, do, w.W, True, w.rank,
                                                causal=True)
            warm_up(torch, run_steps, max(1, args.warmup))
            ms = loop_ms(torch, run_steps, reps)
            tf = flop / (ms * 1e-3) / 1e12
            res[w.name + "_bwd_ring_steps"] = {
                "ms": round(ms, 4), "tflops": round(tf, 2),
                "pct_of_peak": round(100 * tf / PEAK_BF16_TFLOPS, 2),
                "mode": "rattn_bwd_delta + 8 rattn_bwd_step launches into float32 "
                        "accumulators (zeroing included)"}
            del ks, vs
        del q, k, v, do, out, lse, dq, dk, dv, ws
        torch.cuda.empty_cache()
    return res


def tile_efficiency(steps, br=256, bc=64):
    """Visible pairs / pairs of the tiles a step kernel computes, for a list
    of (query positions, key positions) steps, each side ascending within
    its runs; a key tile is computed for a query tile iff its first key is
    not after the tile's last query."""
    vis = done = 0
    for qp, kp in steps:
        vis += causal_pairs(qp, kp)
        kfirst = np.asarray(kp)[::bc]
        krows = np.minimum(bc, len(kp) - np.arange(0, len(kp), bc))
        for i0 in range(0, len(qp), br):
            qt = np.asarray(qp[i0:i0 + br])
            done += len(qt) * int(krows[kfirst <= qt.max()].sum())
    return vis / done if done else 1.0


def layout_comparison(torch, binding, ring, workloads, dev, args):
    """Causal load balance of the ring layouts at the ZigZag ring share's
    shape (131072 tokens, 8 devices, 8 heads, d = 128, bf16): every device's
    W forward ring steps (merges in the step epilogue) timed on this GPU;
    the ring's step time is the slowest device's, and device_tflops is one
    device's share of the whole causal attention (4 d per visible pair) over
    that time.  Contiguous blocks, ZigZag chunk pairs (Twinkle page) and the
    Striped layout (ultralytics page)."""
    w = workloads.workload(4)
    W, N, d, H = w.W, w.N, w.d, w.Hq
    q, k, v = workloads.make_inputs(workloads.Workload(
        0, "layouts", 1, N, N, H, w.Hkv, d, w.dtype, True, W, False, -1, 0), device=dev)
    total_flop = 4 * d * H * (N * (N + 1) // 2)
    res = {}
    for layout in ("contiguous", "zigzag", "striped"):
        if layout == "striped":
            ks = [ring.stripe(k, W, r) for r in range(W)]
            vs = [ring.stripe(v, W, r) for r in range(W)]
            qs = [ring.stripe(q, W, r) for r in range(W)]

            def run(r):
                return ring.striped_forward_steps(qs[r], ks, vs, W, r)
            S = N // W
            steps = [(np.arange(S), np.arange(S) + ring.striped_key_offset(r, (r - s) % W))
                     for r in range(W) for s in range(W)]
        else:
            zz = layout == "zigzag"
            ks = [ring.shard(k, W, zz, r) for r in range(W)]
            vs = [ring.shard(v, W, zz, r) for r in range(W)]
            qs = [ring.shard(q, W, zz, r) for r in range(W)]

            def run(r, zz=zz):
                return ring.ring_forward_steps(qs[r], ks, vs, W, zz, r, causal=True)
            steps = []
            for r in range(W):
                qp = runs_positions(ring.shard_rows(N, W, zz, r))
                for s in range(W):
                    src = (r - s) % W
                    steps.append((qp, runs_positions(ring.shard_rows(N, W, zz, src))))
        warm_up(torch, lambda: [run(r) for r in range(W)], 1)  # every device's share
        ms = []
        for r in range(W):
            ms.append(loop_ms(torch, lambda: run(r), 3))
        ring_ms = max(ms)
        res["layout_" + layout] = {
            "device_ms": [round(x, 3) for x in ms], "ring_step_ms": round(ring_ms, 3),
            "imbalance_max_over_mean": round(ring_ms / (sum(ms) / W), 3),
            "device_tflops": round(total_flop / W / (ring_ms * 1e-3) / 1e12, 1),
            "tile_efficiency": round(tile_efficiency(steps), 4)}
        del ks, vs, qs
        torch.cuda.empty_cache()
    return res


def varlen_extra(torch, binding, workloads, dev, args):
    """A packed variable-length batch (rattn_fwd_varlen): 16 causal sequences
    with lengths drawn uniformly from [1024, 16384] (numpy seed 7), 32 query
    heads over 8 key/value heads, d = 128, bf16."""
    lens = [int(x) for x in np.random.default_rng(7).integers(1024, 16385, 16)]
    N = sum(lens)
    q, k, v = workloads.make_qkv(1, N, N, 32, 8, 128, torch.bfloat16, seed=7, device=dev)
    q, k, v = q[0], k[0], v[0]
    starts, ls = binding.varlen_from_cu_seqlens(np.concatenate([[0], np.cumsum(lens)]))
    flop = 4 * 128 * 32 * sum(n * (n + 1) // 2 for n in lens)

    def run():
        return binding.fwd_varlen(q, k, v, starts, ls, starts, ls, causal=True)
    warm_up(torch, run, max(1, args.warmup))
    reps = max(3, args.steps // 2)
    ms = loop_ms(torch, run, reps)
    tf = flop / (ms * 1e-3) / 1e12
    del q, k, v
    torch.cuda.empty_cache()
    return {"varlen_16seq_1k_16k_causal_h32kv8_d128_bf16": {
        "ms": round(ms, 4), "tflops": round(tf, 2),
        "pct_of_peak": round(100 * tf / PEAK_BF16_TFLOPS, 2), "tokens": N}}


def single_head_extra(torch, binding, workloads, dev, args):
    """The single-head workload (4096 queries and keys, d=128, bf16) through
    rattn_fwd, which runs it on the key-split kernel: 128 workgroups of 32
    query rows, each reading the head's whole K and V (2 MB) from L2 once.
    That read, over the compute units that do it, is what bounds the kernel
    (about 140 GB/s per compute unit from L2)."""
    w = workloads.workload(2)
    q, k, v = workloads.make_inputs(w, device=dev)
    flop = 4 * w.d * w.Hq * w.B * w.Nq * w.N

    def run():
        return binding.fwd(q, k, v)
    warm_up(torch, run, 5)
    ms = loop_ms(torch, run, max(50, 2 * args.steps))
    dev_us = device_us(torch, run)
    groups = w.B * w.Hq * ((w.Nq + 31) // 32)
    kv_bytes = 2 * w.N * w.Hkv * w.d * 2
    return {w.name: {"ms": round(ms, 4), "us": round(ms * 1e3, 2), "device_us": round(dev_us, 2),
                     "tflops": round(flop / (ms * 1e-3) / 1e12, 2),
                     "pct_of_peak": round(100 * flop / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2),
                     "kernel": "fwd_short_kernel (32 query rows per workgroup, key tiles split "
                               "among 8 waves)",
                     "workgroups": groups,
                     "l2_to_cu_bytes": groups * kv_bytes,
                     "l2_to_cu_GBps_per_busy_cu": round(kv_bytes / (ms * 1e-3) / 1e9, 1)}}


def small_d_sweep(torch, binding, workloads, dev, args):
    """Small head dims at the batched causal shape (B=2, 4096 tokens, 32 heads,
    fp16). Compulsory HBM bytes = q, k, v read + out written (input dtype) +
    lse written (fp32)."""
    out = {}
    w3 = workloads.workload(3)
    pe = causal_pairs(np.arange(w3.N), np.arange(w3.N))
    for dd in (16, 32, 64):
        qe, ke, ve = workloads.make_qkv(w3.B, w3.N, w3.N, w3.Hq, w3.Hkv, dd, torch.float16,
                                        seed=3, device=dev)
        fe = 4 * dd * w3.Hq * w3.B * pe
        comp = (qe.numel() + ke.numel() + ve.numel() + qe.numel()) * 2 + qe.numel() // dd * 4
        warm_up(torch, lambda: binding.fwd(qe, ke, ve, causal=True), args.warmup)
        ms = loop_ms(torch, lambda: binding.fwd(qe, ke, ve, causal=True), args.steps)
        out[f"mha_causal_b2_h32_4k_d{dd}_f16"] = {
            "ms": round(ms, 4), "tflops": round(fe / (ms * 1e-3) / 1e12, 2),
            "compulsory_bytes": comp, "compulsory_GBps": round(comp / (ms * 1e-3) / 1e9, 1)}
        del qe, ke, ve
        torch.cuda.empty_cache()
    return out


def cpu_baseline(w, q, k, v, n_rows):
    """The fp64 oracle, as it stands, on a bounded sample of the same workload."""
    import oracle
    from oracle import layouts

    rows = np.stack([np.zeros(n_rows, np.int64),
                     np.random.default_rng(7).choice(w.Nq, n_rows, replace=False),
                     np.random.default_rng(8).integers(0, w.Hq, n_rows)], axis=1)
    # every device's shard in one call (rank -1): q in natural order
    qpos = np.arange(w.Nq) if w.rank < 0 else layouts.zigzag_shard_positions(w.N, w.W, w.rank)
    qh, kh, vh = q.cpu(), k.cpu(), v.cpu()
    threads = oracle.default_threads()
    t = time.perf_counter()
    oracle.attention(qh, kh, vh, causal=True, q_pos=qpos, rows=rows, n_threads=threads)
    dt = time.perf_counter() - t
    pairs = int((qpos[rows[:, 1]] + 1).sum())  # keys 0..N-1, natural order
    flop = 4 * w.d * pairs
    all_pairs = int((qpos + 1).sum()) * w.Hq * w.B
    model = ""
    try:
        with open("/proc/cpuinfo") as fh:
            model = next((ln.split(":", 1)[1].strip() for ln in fh if ln.startswith("model name")),
                         "")
    except OSError:
        pass
    return {"value": round(flop / dt / 1e12, 6), "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{n_rows} seeded (row, head) query rows of the same workload, "
                      f"{pairs} visible pairs, {dt:.2f} s wall",
            "rows_per_s": round(n_rows / dt, 1),
            "full_workload_s_extrapolated": round(dt * all_pairs / pairs, 1),
            "cpu_model": model, "host_cpus": os.cpu_count()}


if __name__ == "__main__":
    main()
