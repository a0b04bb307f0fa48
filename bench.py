#!/usr/bin/env python3
"""Benchmark of MLA tree-verify attention on one MI355X.

Headline workload (one step = one call = split-KV kernel + combine kernel):
  binary16-ctx65536: batch 1, 16-node heap-binary tree, 8 heads, context 65536,
  pool of 262144 slots, fully scattered page_size=1 table, bf16 latents ~ N(0,1),
  scale 1/sqrt(192). Eight independently seeded input sets (pool, Q) rotate from
  call to call so that the 256 MB Infinity Cache cannot serve a repeat.
Metric: achieved GB/s = algorithmic bytes per call / time per call, where the
algorithmic bytes are every referenced 1152-byte row and its 4-byte index once,
Q, out, lse and the mask.

Also reported on the same line:
  roofline     the split-KV kernel's algorithmic bytes / its average launch
               duration (HIP events around each launch), against 8 TB/s;
  call_us      p10 / p50 / p90 of per-call durations (HIP events);
  context_sweep the 61-layer stacked chain8 sweep (own pool per layer, one page
               table per context): microseconds per layer and GB/s, with eager
               launches and as one HIP-graph-captured step;
  other_configs 64 nodes x 64 heads at context 131072 (MFMA-bound: TFLOP/s
               against 2.5 PFLOP/s dense bf16) and batch 8 with log-uniform
               contexts in both page layouts (GB/s each; outputs bitwise equal);
  cpu_baseline the CPU oracle on full calls of the headline workload.

Prints progress to stderr and one JSON line to stdout.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "achieved HBM GB/s (% of peak) for MLA tree-verify at 64k/185k ctx; µs/layer"
KERNEL_SOURCE = os.path.join(ROOT, "mla_tree_verify_02_amd", "csrc", "mtv_kernels.hip")
PROFILE_FILE = os.path.join(ROOT, "profiles", "binary16-ctx65536_counters.json")
PEAK_GBPS = 8000.0
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
MALL_BYTES = 256 << 20     # MI355X Infinity Cache
LAYERS = 61
C5_WARMUP = 100  # untimed calls per batch-8 layout before it is timed
SWEEP_CONTEXTS = "1024,11264,32768,65536,131072,189440"


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def split_kernel_bytes(seq_lens, n, h):
    """Algorithmic bytes the split-KV kernel must read: rows, indices, Q, mask."""
    from mla_tree_verify_02_amd import inputs as I
    w = I.mask_words(n)
    return sum(int(s) for s in seq_lens) * (I.ROW_BYTES + 4) + len(seq_lens) * (
        n * h * I.D_QK * 2 + n * w * 4)


def kernel_source_hash() -> str:
    import hashlib
    with open(KERNEL_SOURCE, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def measured_profile():
    """The committed rocprofv3 summary of the headline workload (kernel trace
    durations, HBM bytes from FETCH_SIZE/WRITE_SIZE, MFMA busy share), if it
    was taken on the current kernel source; else None."""
    try:
        with open(PROFILE_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha256") != kernel_source_hash():
        return None
    return t


SAMPLER_CHILD = r'''
import json, sys, time
import amdsmi
amdsmi.amdsmi_init()
h = amdsmi.amdsmi_get_processor_handles()[0]
period = float(sys.argv[1])
out = open(sys.argv[2], "w")
def get(fn):
    try:
        v = fn()
        return float(v) if isinstance(v, (int, float)) else None
    except Exception:
        return None
while True:
    act = {}
    try:
        act = amdsmi.amdsmi_get_gpu_activity(h)
    except Exception:
        pass
    rec = {"t": time.time(),
           "gfx_mhz": get(lambda: amdsmi.amdsmi_get_clock_info(h, amdsmi.AmdSmiClkType.GFX)["clk"]),
           "mem_mhz": get(lambda: amdsmi.amdsmi_get_clock_info(h, amdsmi.AmdSmiClkType.MEM)["clk"]),
           "power_w": get(lambda: amdsmi.amdsmi_get_power_info(h)["current_socket_power"]),
           "gfx_activity_pct": get(lambda: act["gfx_activity"]),
           "umc_activity_pct": get(lambda: act["umc_activity"])}
    out.write(json.dumps(rec) + "\n")
    out.flush()
    time.sleep(period)
'''


class ClockSampler:
    """Samples the GPU's graphics and memory clocks, socket power and engine
    activity (graphics, memory controller) through the amdsmi library, about
    every `period` seconds, in a child process (so that the bench's own
    launch loop cannot starve it), while the timed work runs. The analogue of
    an nvidia-smi probe beside a decode run. Reports None if the library or
    the device refuses. The summary covers all samples and, separately, the
    samples taken while the graphics engine was busy."""

    def __init__(self, period=0.05):
        self.period = period
        self.proc = None
        self.path = None

    def start(self):
        import subprocess
        import tempfile
        fd, self.path = tempfile.mkstemp(prefix="mtv_clocks_", suffix=".jsonl")
        os.close(fd)
        try:
            self.proc = subprocess.Popen([sys.executable, "-c", SAMPLER_CHILD, str(self.period), self.path],
                                         stdout=subprocess.DEVNULL, stderr=subprocess.DEVNULL)
        except OSError as e:
            log("clock sampling unavailable: %s" % e)
            self.proc = None
        return self

    def stop(self, window=None):
        """Stop sampling; summarise all samples, the samples with the
        graphics engine busy, and those inside `window` = (t0, t1, lag): the
        wall-clock span of a sustained load, less its first `lag` seconds (the
        driver's activity and clock readings trail the load by up to a second)."""
        if self.proc is None:
            return None
        self.proc.terminate()
        try:
            self.proc.wait(timeout=5)
        except Exception:
            self.proc.kill()
        recs = []
        try:
            with open(self.path) as f:
                for line in f:
                    try:
                        recs.append(json.loads(line))
                    except ValueError:
                        pass
            os.unlink(self.path)
        except OSError:
            pass
        if not recs:
            log("clock sampling returned no samples")
            return None

        def summary(rs):
            out = {"samples": len(rs)}
            for key in ("gfx_mhz", "mem_mhz", "power_w", "gfx_activity_pct", "umc_activity_pct"):
                v = sorted(r[key] for r in rs if r.get(key) is not None)
                if v:
                    out[key] = {"min": v[0], "p50": v[len(v) // 2], "max": v[-1]}
            return out

        busy = [r for r in recs if (r.get("gfx_activity_pct") or 0) >= 50]
        res = {"period_s": self.period, "all": summary(recs), "gfx_busy": summary(busy) if busy else None}
        if window is not None:
            t0, t1, lag = window
            load = [r for r in recs if t0 + lag <= r["t"] <= t1]
            res["under_load"] = summary(load) if load else None
        return res


def copy_calibration(mib, torch):
    """A plain copy of known size (reads and writes mib MiB each), run outside
    the timed region so that a counter pass can scale FETCH_SIZE/WRITE_SIZE."""
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    log("copy calibration: 3 x %d MiB read + %d MiB written" % (mib, mib))
    del src, dst


def sustain(calls, seconds, torch):
    """Back-to-back calls for about `seconds` of wall clock (chunks of 200,
    synchronised), so that a clock sampler sees a sustained load; returns the
    window (start, end) and the mean wall-clock microseconds per call."""
    torch.cuda.synchronize()
    t0 = time.time()
    n = 0
    while time.time() - t0 < seconds:
        for k in range(200):
            calls[k % len(calls)].run()
        torch.cuda.synchronize()
        n += 200
    t1 = time.time()
    return t0, t1, (t1 - t0) / n * 1e6


def time_calls(calls, steps, warmup, torch):
    """Wall-clock of `steps` calls (rotating), synchronised on both sides."""
    for k in range(warmup):
        calls[k % len(calls)].run()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(steps):
        calls[k % len(calls)].run()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / steps


def time_split_kernel(calls, steps, torch):
    """Average split-KV kernel duration from HIP events around each launch on
    the stream the library launches on (torch's current stream)."""
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    torch.cuda.synchronize()
    for k in range(steps):
        ev[k][0].record(stream)
        calls[k % len(calls)].splitkv()
        ev[k][1].record(stream)
    torch.cuda.synchronize()
    ms = [a.elapsed_time(b) for a, b in ev]
    ms.sort()
    return sum(ms) / len(ms), ms[len(ms) // 2]


def time_each_call(calls, steps, torch, fn="run"):
    """Per-call durations (us) from HIP events around each call on torch's
    current stream, rotating over `calls`; returns the sorted list."""
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    torch.cuda.synchronize()
    for k in range(steps):
        ev[k][0].record(stream)
        getattr(calls[k % len(calls)], fn)()
        ev[k][1].record(stream)
    torch.cuda.synchronize()
    return sorted(a.elapsed_time(b) * 1e3 for a, b in ev)


SPIN_CYCLES = 200_000  # torch.cuda._sleep cycles queued ahead of each timed small call


def time_each_call_gpu(fn, steps, torch, before=None):
    """Per-call GPU durations (us) of small calls: HIP events around each call
    on torch's current stream, with a short spin kernel queued ahead of the
    events so that the GPU is still busy while the host enqueues the events
    and the call (host time then stays outside the bracket). `before(k)`
    enqueues untimed work ahead of the spin. Returns the sorted list."""
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    torch.cuda.synchronize()
    for k in range(steps):
        if before is not None:
            before(k)
        torch.cuda._sleep(SPIN_CYCLES)
        ev[k][0].record(stream)
        fn(k)
        ev[k][1].record(stream)
    torch.cuda.synchronize()
    return sorted(a.elapsed_time(b) * 1e3 for a, b in ev)


def pct(sorted_us, q):
    return sorted_us[min(len(sorted_us) - 1, int(q * len(sorted_us)))]


def headline(args, torch, M, I):
    log("building headline inputs (binary16-ctx65536, %d rotated sets)" % args.rotate)
    wls = [I.config_workload(2, device="cuda", layer=r) for r in range(args.rotate)]
    ws = None
    calls = []
    for wl in wls:
        c = M.prepare_workload(wl, workspace=ws)
        ws = c.workspace
        calls.append(c)
    seq = wls[0].seq_lens_host()
    n, h = wls[0].num_nodes, wls[0].num_heads
    call_bytes = I.algorithmic_bytes(seq, n, h)
    log("timing %d steps after %d warmup" % (args.steps, args.warmup))
    sec = time_calls(calls, args.steps, args.warmup, torch)
    log("split-KV kernel events over %d launches" % args.steps)
    avg_ms, med_ms = time_split_kernel(calls, args.steps, torch)
    kbytes = split_kernel_bytes(seq, n, h)
    plan = M.plan_query(M.make_shape(1, n, h, wls[0].max_kv, wls[0].num_slots),
                        torch.cuda.get_device_properties(0).multi_processor_count)
    per_call = time_each_call(calls, args.steps, torch)
    return dict(wls=wls, calls=calls, sec=sec, call_bytes=call_bytes, split_avg_ms=avg_ms,
                split_med_ms=med_ms, split_bytes=kbytes, plan=plan,
                call_us={"p10": round(pct(per_call, 0.1), 3), "p50": round(pct(per_call, 0.5), 3),
                         "p90": round(pct(per_call, 0.9), 3)})


def other_configs(args, torch, M, I):
    """The all-heads configuration (64 nodes x 64 heads, MFMA-bound), the
    batch-8 mixed-length configuration in three page layouts (scattered,
    runs of 64, hybrid pages of 64), and the tree-mask build from parent
    arrays."""
    out = {}
    names = [c.strip() for c in args.configs.split(",") if c.strip()]
    if "c1" in names:
        # the tiny chain: 1.3 MB per call, served by the caches and bound by
        # launch and fixed per-call cost rather than by HBM
        log("building tiny-chain-ctx1024 (8 rotated sets)")
        wls = [I.config_workload(1, device="cuda", layer=r) for r in range(8)]
        ws = None
        calls = []
        for wl in wls:
            c = M.prepare_workload(wl, workspace=ws)
            ws = c.workspace
            calls.append(c)
        sec = time_calls(calls, args.steps, args.warmup, torch)
        us = time_each_call(calls, args.steps, torch)
        seq = wls[0].seq_lens_host()
        b = I.algorithmic_bytes(seq, wls[0].num_nodes, wls[0].num_heads)
        med = pct(us, 0.5)
        out["tiny-chain-ctx1024"] = {
            "us_per_call": {"p10": round(pct(us, 0.1), 2), "p50": round(med, 2), "p90": round(pct(us, 0.9), 2)},
            "wall_us_per_call": round(sec * 1e6, 2), "bytes_per_call": b,
            "gbps": round(b / (med * 1e-6) / 1e9, 1), "cache_resident": True}
        log("tiny-chain-ctx1024: %.2f us/call (events), %.2f us/call (wall)" % (med, sec * 1e6))
        del calls, wls, ws
    if "c4" in names:
        log("building random64-h64-ctx131072 (2 rotated sets)")
        wls = [I.config_workload(4, device="cuda", layer=r) for r in range(2)]
        ws = None
        calls = []
        for wl in wls:
            c = M.prepare_workload(wl, workspace=ws)
            ws = c.workspace
            calls.append(c)
        # about 20 ms of untimed calls first: the earliest calls after the
        # inputs are built run up to 10 % slower
        for k in range(20):
            calls[k % len(calls)].run()
        us = time_each_call(calls, args.big_steps, torch)
        sk = time_each_call(calls, args.big_steps, torch, "splitkv")
        seq = wls[0].seq_lens_host()
        n, h = wls[0].num_nodes, wls[0].num_heads
        flops = I.algorithmic_flops(seq, n, h)
        med = pct(us, 0.5)
        ksk = sum(sk) / len(sk)
        out["random64-h64-ctx131072"] = {
            "bound": "mfma", "calls": len(us),
            "us_per_call": {"p10": round(pct(us, 0.1), 2), "p50": round(med, 2), "p90": round(pct(us, 0.9), 2)},
            "tflops": round(flops / (med * 1e-6) / 1e12, 1),
            "split_kernel_avg_us": round(ksk, 2),
            "split_kernel_tflops": round(flops / (ksk * 1e-6) / 1e12, 1),
            "peak_tflops": PEAK_BF16_TFLOPS,
            "split_kernel_frac": round(flops / (ksk * 1e-6) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "gbps": round(I.algorithmic_bytes(seq, n, h) / (med * 1e-6) / 1e9, 1),
            "flops_per_call": flops,
            # SQ_VALU_MFMA_BUSY_CYCLES share of the split kernel in the committed
            # counter profile of the same kernel source (null if it differs)
            "split_mfma_busy_pct": (measured_profile() or {}).get("random64-h64-ctx131072_split_mfma_busy_pct")}
        log("random64-h64-ctx131072: %.1f us/call, %.1f TFLOP/s (split kernel %.1f us, %.1f TFLOP/s)"
            % (med, flops / (med * 1e-6) / 1e12, ksk, flops / (ksk * 1e-6) / 1e12))
        del calls, wls, ws
        torch.cuda.empty_cache()
    if "c5" in names:
        # The layouts are timed in alternating rounds (each one freshly built
        # layout runs slower for its first calls, and back-to-back phases drift
        # by 1-2 us on their own): the scattered per-token table, the same rows
        # relaid in runs of 64 slots, the hybrid layout (prefixes in pages of 64
        # slots, tree rows scattered) through mla_tree_verify_paged, and that
        # layout's pool through its expanded per-token table.
        base = I.config_workload(5, device="cuda", layout="scattered")
        runs = I.relayout(base, I.seed_for(5, 0, I.F_TABLE) + 1, "runs64")
        hl = I.hybrid_layout(base, 64, seed=64)
        w = hl.workload
        log("building batch8-loguniform (scattered, runs64, hybrid pages of 64)")
        calls = {"scattered": M.prepare_workload(base), "runs64": M.prepare_workload(runs),
                 "paged64": M.PreparedPagedCall(w.q, w.kv_pool, hl.prefix_pages, hl.tree_slots, w.seq_lens,
                                                w.tree_mask, w.scale, 64, w.max_kv),
                 "paged64_pool_per_token": M.prepare_workload(w)}
        torch.cuda.synchronize()
        outs = {k: (c.out.clone(), c.lse.clone()) for k, c in calls.items()}
        for c in calls.values():
            for _ in range(C5_WARMUP):
                c.run()
        us = {k: [] for k in calls}
        rounds = 5
        for _ in range(rounds):
            for k, c in calls.items():
                us[k] += time_each_call([c], max(1, args.steps // rounds), torch)
        seq = base.seq_lens_host()
        b = I.algorithmic_bytes(seq, base.num_nodes, base.num_heads)
        res = {}
        for k in calls:
            v = sorted(us[k])
            med = pct(v, 0.5)
            res[k] = {"us_per_call": {"p10": round(pct(v, 0.1), 2), "p50": round(med, 2),
                                      "p90": round(pct(v, 0.9), 2)},
                      "gbps": round(b / (med * 1e-6) / 1e9, 1),
                      "pct_of_peak": round(100 * b / (med * 1e-6) / 1e9 / PEAK_GBPS, 2),
                      "bytes_per_call": b}
            log("batch8-loguniform %s: %.2f us/call, %.0f GB/s" % (k, med, b / (med * 1e-6) / 1e9))
        res["seq_lens"] = [int(x) for x in seq]
        res["paged64"]["page_size"] = 64
        res["paged64"]["page_list_entries"] = int(hl.prefix_pages.numel())
        res["rounds"] = rounds

        def same(x, y):
            return bool(torch.equal(x[0].view(torch.int16), y[0].view(torch.int16))
                        and torch.equal(x[1].view(torch.int32), y[1].view(torch.int32)))
        res["bitwise_equal"] = all(same(outs["scattered"], o) for o in outs.values())
        out["batch8-loguniform"] = res
        del calls, base, runs, hl, w
        torch.cuda.empty_cache()
    if "mask" in names:
        # the tree-mask build before the verify step (parent array -> bitmask)
        import numpy as np
        res = {}
        for b, n in ((1, 64), (8, 8), (4096, 64)):
            parents = torch.from_numpy(np.stack([I.random_parents(n, 8, 70_000 + s) for s in range(b)])
                                       .astype(np.int32)).cuda()
            mask = M.tree_mask_build(parents)

            class _Call:
                def run(self):
                    M.tree_mask_build(parents, out=mask)
            us = time_each_call([_Call()], 200, torch)
            gus = time_each_call_gpu(lambda k: M.tree_mask_build(parents, out=mask), 200, torch)
            res["b%d_n%d" % (b, n)] = {"us_per_call": {"p10": round(pct(us, 0.1), 2),
                                                       "p50": round(pct(us, 0.5), 2),
                                                       "p90": round(pct(us, 0.9), 2)},
                                       "gpu_us": {"p10": round(pct(gus, 0.1), 2), "p50": round(pct(gus, 0.5), 2),
                                                  "p90": round(pct(gus, 0.9), 2)},
                                       "nodes_per_s": round(b * n / (pct(gus, 0.5) * 1e-6), 1)}
            log("tree mask build B=%d N=%d: %.2f us/call (%.2f us on the GPU)"
                % (b, n, pct(us, 0.5), pct(gus, 0.5)))
        out["tree_mask_build"] = res
        # the device input check on the headline's inputs (table, lengths, mask)
        wl = I.config_workload(2, device="cuda")
        counts = M.check_inputs(wl.page_table, wl.seq_lens, wl.tree_mask, wl.num_slots)
        gus = time_each_call_gpu(lambda k: M.check_inputs(wl.page_table, wl.seq_lens, wl.tree_mask,
                                                          wl.num_slots, counts=counts), 200, torch)
        out["input_check"] = {"workload": "binary16-ctx65536 (65,552 table positions)",
                              "counts": [int(x) for x in counts.cpu()],
                              "gpu_us": {"p10": round(pct(gus, 0.1), 2), "p50": round(pct(gus, 0.5), 2),
                                         "p90": round(pct(gus, 0.9), 2)}}
        log("input check binary16-ctx65536: %.2f us on the GPU, counts %s"
            % (pct(gus, 0.5), out["input_check"]["counts"]))
        del wl
    if "kv" in names:
        out["kv_moves"] = kv_moves(torch, M, I)
    return out


def kv_moves(torch, M, I):
    """Tier-0 moves after a verify step: a whole sequence gathered from
    scattered slots into a fresh contiguous run (HBM-bound copy, reported
    against 8 TB/s), and the accepted-path commit. The page table is restored
    before each call, outside the timed bracket; 4 source/destination sets
    rotate so that the Infinity Cache cannot serve repeats."""
    import numpy as np
    res = {}
    stream = torch.cuda.current_stream()
    for S in (65536, 189448):
        R = 4
        P = 2 * R * S
        pool = torch.empty((P, I.D_QK), dtype=torch.bfloat16, device="cuda")
        pool.view(torch.int16).random_()
        tables, bases = [], []
        for r in range(R):
            g = torch.Generator().manual_seed(4242 + r)
            src = (2 * r * S + torch.randperm(S, generator=g)).to(torch.int32)
            tables.append(src.view(1, S).cuda())
            bases.append(torch.tensor([2 * r * S + S], dtype=torch.int32, device="cuda"))
        seq = torch.tensor([S], dtype=torch.int32, device="cuda")
        work = torch.empty((1, S), dtype=torch.int32, device="cuda")
        ev = []
        for k in range(8 + 40):
            r = k % R
            work.copy_(tables[r])
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            M.kv_defrag(pool, work, seq, bases[r])
            e1.record(stream)
            if k >= 8:
                ev.append((e0, e1))
        torch.cuda.synchronize()
        us = sorted(a.elapsed_time(b) * 1e3 for a, b in ev)
        nbytes = S * (2 * I.ROW_BYTES + 8) + 8
        med = pct(us, 0.5)
        res["defrag_s%d" % S] = {"us_per_call": {"p10": round(pct(us, 0.1), 2), "p50": round(med, 2),
                                                 "p90": round(pct(us, 0.9), 2)},
                                 "bytes_per_call": nbytes, "gbps": round(nbytes / (med * 1e-6) / 1e9, 1),
                                 "frac_of_8tbs": round(nbytes / (med * 1e-6) / 1e9 / PEAK_GBPS, 4)}
        log("defrag of %d rows: %.2f us, %.0f GB/s" % (S, med, nbytes / (med * 1e-6) / 1e9))
        del pool, tables, work
        torch.cuda.empty_cache()
    # accepted-path commit: heap-binary 16-node tree, path 0-1-3-7-15 (L = 5);
    # and batch 8 of 8-node chains, 4 accepted each
    for B, N, path in ((1, 16, [0, 1, 3, 7, 15]), (8, 8, [0, 1, 2, 3])):
        S0 = 4096
        P = 2 * B * S0
        pool = torch.empty((P, I.D_QK), dtype=torch.bfloat16, device="cuda")
        pool.view(torch.int16).random_()
        g = torch.Generator().manual_seed(99)
        table0 = torch.randperm(B * S0, generator=g).to(torch.int32).view(B, S0).cuda()
        seq = torch.full((B,), S0, dtype=torch.int32, device="cuda")
        alen = torch.full((B,), len(path), dtype=torch.int32, device="cuda")
        apath = torch.zeros((B, N), dtype=torch.int32)
        apath[:, :len(path)] = torch.tensor(path, dtype=torch.int32)
        apath = apath.cuda()
        base = (B * S0 + S0 * torch.arange(B, dtype=torch.int32)).cuda()
        work = table0.clone()
        ev = []
        for k in range(20 + 200):
            work.copy_(table0)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            M.kv_commit(pool, work, seq, N, alen, apath, base)
            e1.record(stream)
            if k >= 20:
                ev.append((e0, e1))
        torch.cuda.synchronize()
        us = sorted(a.elapsed_time(b) * 1e3 for a, b in ev)
        gus = time_each_call_gpu(lambda k: M.kv_commit(pool, work, seq, N, alen, apath, base), 200, torch,
                                 before=lambda k: work.copy_(table0))
        res["commit_b%d_n%d_l%d" % (B, N, len(path))] = {
            "us_per_call": {"p10": round(pct(us, 0.1), 2), "p50": round(pct(us, 0.5), 2),
                            "p90": round(pct(us, 0.9), 2)},
            "gpu_us": {"p10": round(pct(gus, 0.1), 2), "p50": round(pct(gus, 0.5), 2),
                       "p90": round(pct(gus, 0.9), 2)},
            "rows_moved": B * len(path)}
        log("commit B=%d N=%d L=%d: %.2f us/call (%.2f us on the GPU)"
            % (B, N, len(path), pct(us, 0.5), pct(gus, 0.5)))
        del pool
    return res


def sweep(args, torch, M, I):
    ctxs = [int(c) for c in args.sweep.split(",") if c.strip()]
    if not ctxs:
        return []
    P = 262144
    log("building %d layer pools of %d slots for the sweep" % (LAYERS, P))
    pools = [I._randn_bf16((P, I.D_QK), I._gen(I.seed_for(3, l, I.F_KV), "cuda"), "cuda")
             for l in range(LAYERS)]
    qs = [I._randn_bf16((64, I.D_QK), I._gen(I.seed_for(3, l, I.F_Q), "cuda"), "cuda").view(1, 8, 8, I.D_QK)
          for l in range(LAYERS)]
    mask = torch.from_numpy(I.ancestor_bitmask(I.chain_parents(8)).view("int32").copy()).view(1, 8, 1).cuda()
    results = []
    ws = None
    for ctx in ctxs:
        S = ctx + 8
        rows, _ = I.scattered_table([S], P, I.seed_for(3, 0, I.F_TABLE) + ctx)
        table = torch.from_numpy(rows[0].reshape(1, S).copy()).cuda()
        seq = torch.tensor([S], dtype=torch.int32, device="cuda")
        calls = []
        for l in range(LAYERS):
            c = M.PreparedCall(qs[l], pools[l], table, seq, mask, I.DEFAULT_SCALE, workspace=ws)
            ws = c.workspace
            calls.append(c)
        steps = max(2, args.sweep_steps)
        for c in calls:  # warm-up step
            c.run()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            for c in calls:
                c.run()
        torch.cuda.synchronize()
        step_s = (time.perf_counter() - t0) / steps
        us_layer = step_s / LAYERS * 1e6
        b_layer = I.algorithmic_bytes([S], 8, 8)
        gbps = b_layer / (us_layer * 1e-6) / 1e9
        # the same 61-layer step captured once into a HIP graph and replayed
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for c in calls:
                c.run()
        torch.cuda.current_stream().wait_stream(side)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for c in calls:
                c.run()
        graph.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            graph.replay()
        torch.cuda.synchronize()
        gstep_s = (time.perf_counter() - t0) / steps
        # a whole step's rows fit in the 256 MB Infinity Cache only at the
        # shortest contexts; those figures are cache-served, not HBM-bound
        mall = LAYERS * b_layer <= MALL_BYTES
        results.append({"context": ctx, "layers": LAYERS, "us_per_layer": round(us_layer, 3),
                        "ms_per_step": round(step_s * 1e3, 4), "gbps": round(gbps, 1),
                        "pct_of_peak": round(100 * gbps / PEAK_GBPS, 2),
                        "bytes_per_layer": b_layer, "bytes_per_step": LAYERS * b_layer,
                        "mall_resident": mall,
                        "tokens_per_s_equiv": round(1.0 / step_s, 2),
                        "captured": {"us_per_layer": round(gstep_s / LAYERS * 1e6, 3),
                                     "ms_per_step": round(gstep_s * 1e3, 4),
                                     "gbps": round(b_layer * LAYERS / gstep_s / 1e9, 1),
                                     "pct_of_peak": round(100 * b_layer * LAYERS / gstep_s / 1e9 / PEAK_GBPS, 2),
                                     "tokens_per_s_equiv": round(1.0 / gstep_s, 2)}})
        log("sweep ctx %d: %.2f us/layer, %.0f GB/s (graph-captured step: %.2f us/layer)"
            % (ctx, us_layer, gbps, gstep_s / LAYERS * 1e6))
        del graph
        del calls
    return results


def cpu_per_config(I, threads):
    """The oracle's time per layer-step on the other configurations, with the
    same inputs as the GPU lines (built on the GPU, copied to the host):
    the tiny chain whole; one layer of the 61-layer sweep at 65536 and 189440
    (x61 extrapolated to a step); the 64 x 64-head call on 4 rows of every
    64-row group (extrapolated to its 4096 rows); the batch-8 call whole."""
    import numpy as np
    from oracle import oracle as O

    def timed(wl, rows=None, min_s=0.3):
        host = (wl.np_q(), wl.np_kv(), wl.np_page_table(), wl.np_seq_lens(), wl.np_mask())
        n, t = 0, 0.0
        while t < min_s or n == 0:
            t0 = time.perf_counter()
            O.run(*host, wl.scale, rows=rows, threads=threads)
            t += time.perf_counter() - t0
            n += 1
        return t / n

    res = {}
    wl = I.config_workload(1, device="cuda")
    s = timed(wl)
    res["tiny-chain-ctx1024"] = {"ms_per_layer_step": round(s * 1e3, 3), "rows": 64}
    for ctx in (65536, 189440):
        wl = I.config_workload(3, device="cuda", ctx=ctx, layer=0)
        s = timed(wl, min_s=0.0)
        res["chain8-ctx%d" % ctx] = {"ms_per_layer": round(s * 1e3, 2), "rows": 64,
                                     "ms_per_step_61_layers": round(61 * s * 1e3, 1),
                                     "extrapolated": "one layer timed, x61 for the step"}
        del wl
    wl = I.config_workload(4, device="cuda")
    rng = np.random.default_rng(4)
    rows = np.concatenate([g0 + rng.choice(64, size=4, replace=False) for g0 in range(0, 4096, 64)])
    s = timed(wl, rows=rows, min_s=0.0)
    res["random64-h64-ctx131072"] = {"ms_per_layer_step": round(s * 4096 / len(rows) * 1e3, 1),
                                     "rows_timed": int(len(rows)),
                                     "extrapolated": "%d of 4096 rows timed, x%.0f" % (len(rows), 4096 / len(rows))}
    del wl
    wl = I.config_workload(5, device="cuda")
    s = timed(wl, min_s=0.0)
    res["batch8-loguniform"] = {"ms_per_layer_step": round(s * 1e3, 2), "rows": 512}
    del wl
    for k, v in res.items():
        log("CPU oracle %s: %s" % (k, v))
    return res


def cpu_baseline(wls, call_bytes, I):
    """The CPU oracle, as it stands, on a bounded sample: full calls of the
    headline workload on the first input sets (about 10-30 s of CPU work)."""
    from oracle import oracle as O
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count() or 1
    threads = max(1, min(16, cores))
    # every rotated input set, three passes: about 10 s at 16 threads; stop
    # early past 25 s on a slower host
    hosts = [(wl.np_q(), wl.np_kv(), wl.np_page_table(), wl.np_seq_lens(), wl.np_mask())
             for wl in wls]
    log("CPU oracle on up to %d full calls with %d threads" % (3 * len(hosts), threads))
    total = 0.0
    calls = 0
    for _ in range(3):
        for host, wl in zip(hosts, wls):
            t0 = time.perf_counter()
            O.run(*host, wl.scale, threads=threads)
            total += time.perf_counter() - t0
            calls += 1
            if total > 25.0:
                break
        if total > 25.0:
            break
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    # the tree-mask oracle on the shapes the mask-build line times
    from oracle import tree_mask as TM
    import numpy as np
    mask_us = {}
    for b, n in ((1, 64), (8, 8), (4096, 64)):
        parents = np.stack([I.random_parents(n, 8, 70_000 + s) for s in range(b)]).astype(np.int32)
        reps = 20 if b < 100 else 1
        t0 = time.perf_counter()
        for _ in range(reps):
            TM.tree_mask(parents)
        mask_us["b%d_n%d" % (b, n)] = round((time.perf_counter() - t0) / reps * 1e6, 1)
    # the KV-move oracle: one accepted-path commit and a 65,536-row defrag
    from oracle import kv_move as KM
    pool = np.random.default_rng(1).integers(0, 1 << 16, size=(2 * 65536, 576), dtype=np.uint16)
    table = np.random.default_rng(2).permutation(65536).astype(np.int32).reshape(1, 65536)
    t0 = time.perf_counter()
    KM.kv_commit(pool, table, [65536], 16, [5], [[0, 1, 3, 7, 15] + [0] * 11], [65536])
    commit_us = (time.perf_counter() - t0) * 1e6
    t0 = time.perf_counter()
    KM.kv_defrag(pool, table, [65536], [65536])
    defrag_us = (time.perf_counter() - t0) * 1e6
    rows = wls[0].batch * wls[0].num_nodes * wls[0].num_heads
    per_config = cpu_per_config(I, threads)
    return {"value": round(calls * call_bytes / total / 1e9, 4), "unit": "GB/s",
            "per_config": per_config,
            "tree_mask_build_us": mask_us,
            "kv_commit_b1_n16_l5_us": round(commit_us, 1),
            "kv_defrag_s65536_us": round(defrag_us, 1),
            "cores": threads, "kind": "oracle", "seconds": round(total, 3),
            "cpu_model": model,
            "sample": "%d full calls (all %d rows each) of the binary16-ctx65536 workload, "
                      "cycling over its %d input sets" % (calls, rows, len(wls))}


def roofline_entry(hd, achieved, prof):
    """The dominant kernel against 8 TB/s: algorithmic bytes per launch over
    the average launch duration by HIP events in this run (achieved, frac);
    with the committed profile of the same kernel source, also over the
    kernel-trace average (achieved_trace, frac_trace), the HBM bytes the
    FETCH_SIZE/WRITE_SIZE counters saw per launch (traffic) and per call
    (call_traffic, against the call's algorithmic bytes), and the MFMA busy
    share."""
    r = {"bound": "hbm", "kernel": "split_ws_kernel",
         "achieved": round(achieved, 1), "peak": PEAK_GBPS, "unit": "GB/s",
         "frac": round(achieved / PEAK_GBPS, 4), "traffic": None,
         "avg_launch_us": round(hd["split_avg_ms"] * 1e3, 3),
         "bytes_per_launch": hd["split_bytes"], "call_bytes": hd["call_bytes"]}
    if prof is None:
        r["profile"] = None
        return r
    k = prof["kernels"]["split_ws_kernel"]
    r["profile"] = os.path.relpath(PROFILE_FILE, ROOT)
    r["traffic"] = k.get("hbm_bytes_per_dispatch")
    if r["traffic"]:
        r["traffic_ratio"] = round(r["traffic"] / hd["split_bytes"], 4)
    if k.get("trace_avg_us"):
        a = hd["split_bytes"] / (k["trace_avg_us"] * 1e-6) / 1e9
        r["trace_avg_us"] = k["trace_avg_us"]
        r["achieved_trace"] = round(a, 1)
        r["frac_trace"] = round(a / PEAK_GBPS, 4)
    call = sum(v.get("hbm_bytes_per_dispatch") or 0 for v in prof["kernels"].values())
    if call:
        r["call_traffic"] = call
        r["call_traffic_ratio"] = round(call / hd["call_bytes"], 4)
    r["mfma_busy_pct"] = k.get("mfma_busy_pct")
    return r


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=25000,
                    help="untimed calls first (about 1 s of work: the GPU's clocks ramp up from "
                         "idle over the first second of load)")
    ap.add_argument("--rotate", type=int, default=8, help="independent input sets cycled over")
    ap.add_argument("--sweep", default=SWEEP_CONTEXTS,
                    help="contexts of the 61-layer chain8 sweep ('' to skip)")
    ap.add_argument("--sweep-steps", type=int, default=5)
    ap.add_argument("--configs", default="c1,c4,c5,mask,kv",
                    help="other configurations to time: c1 (8-node chain, ctx 1024), "
                         "c4 (64 nodes x 64 heads, ctx 131072), "
                         "c5 (batch 8, mixed lengths, scattered and runs-of-64 layouts), "
                         "mask (the tree-mask build from parent arrays), "
                         "kv (Tier-0 defrag and accepted-path commit); '' for none")
    ap.add_argument("--big-steps", type=int, default=20, help="timed calls of the c4 configuration")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--clock-seconds", type=float, default=3.0,
                    help="seconds of back-to-back headline calls read by the clock sampler")
    ap.add_argument("--no-clocks", action="store_true",
                    help="skip the amdsmi clock/power sampler (e.g. under a profiler)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="also run a plain copy of MIB MiB (for counter calibration)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the verify attention here runs on a single device "
              "and there is no multi-GPU path to time (requested --gpus %d, WORLD_SIZE %d)"
              % (args.gpus, world), file=sys.stderr)
        return 2

    # started before this process touches the GPU; runs until the sweep ends
    sampler = ClockSampler() if not args.no_clocks else None
    if sampler is not None:
        sampler.start()

    import torch

    import mla_tree_verify_02_amd as M
    from mla_tree_verify_02_amd import inputs as I

    if not torch.cuda.is_available():
        if sampler is not None:
            sampler.stop()
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    M.load()
    props = torch.cuda.get_device_properties(0)
    log("device %s, %d CUs" % (props.name, props.multi_processor_count))

    if args.copy_calibration > 0:
        copy_calibration(args.copy_calibration, torch)
    hd = headline(args, torch, M, I)
    sec = hd["sec"]
    value = hd["call_bytes"] / sec / 1e9
    achieved = hd["split_bytes"] / (hd["split_avg_ms"] * 1e-3) / 1e9
    log("headline: %.2f us/call, %.0f GB/s; split kernel %.2f us avg (%.2f med), %.0f GB/s"
        % (sec * 1e6, value, hd["split_avg_ms"] * 1e3, hd["split_med_ms"] * 1e3, achieved))

    sw = sweep(args, torch, M, I)
    clocks = None
    if sampler is not None:
        # the timed work above takes about a second; the sampler needs a
        # sustained load of a few seconds to read the clocks under it
        t0, t1, us_sus = sustain(hd["calls"], args.clock_seconds, torch)
        clocks = sampler.stop(window=(t0, t1, 1.0))
        if clocks is not None:
            clocks["load"] = {"workload": "binary16-ctx65536 calls back to back",
                              "seconds": round(t1 - t0, 2), "us_per_call": round(us_sus, 2)}
        log("sustained headline calls for %.1f s: %.2f us/call" % (t1 - t0, us_sus))
    oc = other_configs(args, torch, M, I)
    cpu = None if args.no_cpu_baseline else cpu_baseline(hd["wls"], hd["call_bytes"], I)

    wl = hd["wls"][0]
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(sec * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: seeded N(0,1) bf16 latents and queries, scattered page_size=1 table, "
                "%d rotated input sets" % args.rotate,
        "config": {"workload": "binary16-ctx65536", "batch": 1, "num_nodes": wl.num_nodes,
                   "num_heads": wl.num_heads, "context": wl.prefix_lens[0],
                   "num_slots": wl.num_slots, "tree": "heap-binary depth 4",
                   "layout": "scattered page_size=1", "rotated_input_sets": args.rotate,
                   "plan": hd["plan"]},
        "us_per_layer": round(sec * 1e6, 3),
        "pct_of_peak": round(100 * value / PEAK_GBPS, 2),
        "roofline": roofline_entry(hd, achieved, measured_profile()),
        "call_us": hd["call_us"],
        "clocks": clocks,
        "context_sweep": sw,
        "other_configs": oc,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
