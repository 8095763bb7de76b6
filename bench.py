"""Frame-step throughput of the 24-block ViT-L-shaped stream on one MI355X.

One step = one new frame through all 24 blocks: per block, one
lbm_append_run (block 0 also reserves, plans -- one small table upload and
the row-table kernel -- and evicts): the append kernel (the block's K/V rows
into their pages), then paged attention (HIP, bf16 MFMA) and the split merge.
Shapes: 1369 patch + 6 special tokens per frame, 16 heads x 64,
scale_frames 8, sliding_window 64, bf16 unit-normal inputs.

Setup (untimed): the 8-frame first step and 64 single frames (F = 72, the
window full), then W warm-up steps; then K timed steps (the first window,
which gives value and roofline).  Inputs: 8 distinct seeded input sets per
block, drawn up front and resident in HBM, cycled over the steps.

The work per frame grows by 6 special keys a frame, so two more windows are
timed ('windows' in the line): the last 20 frames of the 1000-frame stream
(F = 981..1000), reached after the first window by appends and evictions
only, and the last 20 frames of the 10,000-frame 4-block stream (F =
9981..10000, 38% of the keys special), reached the same way.

Printed: one JSON line with frames/s (value), the attention kernel's roofline
(algorithmic FLOPs per call / call time from HIP events on the launch stream
around one lbm_append_run -- append, attention and merge -- against the bf16
dense MFMA peak), the windows, and the CPU oracle timed on a bounded sample of
the same step.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6      # MI355X dense bf16 MFMA
PEAK_FP16_TFLOPS = 2516.6      # MI355X dense fp16 MFMA
PEAK_FP32_TFLOPS = 157.3       # MI355X dense fp32 MFMA
PEAK_HBM_GBPS = 8000.0         # MI355X HBM3E
N_INPUT_SETS = 8


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target CPU time of the oracle sample")
    ap.add_argument("--splits", type=int, default=0, help="force the key-range split count")
    ap.add_argument("--variant-steps", type=int, default=100,
                    help="timed steps of the fp16 and the no-scale-frames variants of the workload "
                         "(reported under 'variants')")
    ap.add_argument("--no-variants", action="store_true")
    ap.add_argument("--end-steps", type=int, default=20,
                    help="timed frames at the end of the 1000-frame stream, reached after the "
                         "timed window by appends and evictions only (reported under 'windows')")
    ap.add_argument("--long-end-steps", type=int, default=20,
                    help="timed frames at the end of the 10,000-frame 4-block stream (reported "
                         "under 'windows')")
    ap.add_argument("--no-windows", action="store_true",
                    help="time the first window only (no end-of-stream windows)")
    ap.add_argument("--f32-steps", type=int, default=20,
                    help="timed steps of the fp32 (force_fp32) variant (reported under 'variants')")
    ap.add_argument("--graph-steps", type=int, default=100,
                    help="frame steps replayed as HIP graphs (reported under 'variants')")
    ap.add_argument("--batch-streams", type=int, default=4,
                    help="independent streams of the batched-launch variant")
    ap.add_argument("--batch-steps", type=int, default=30)
    ap.add_argument("--skip-steps", type=int, default=50,
                    help="skip-append frames timed after the run (reported under 'variants')")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="after the run, stream a 1 GiB buffer through a plain elementwise copy "
                         "three times (reference for the HBM byte counters)")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="summarise two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) of "
                         "'bench.py --calibrate-copy' into the traffic record and exit")
    return ap.parse_args()


# HBM traffic of one lbm_run, from rocprofv3 FETCH_SIZE / WRITE_SIZE scaled by
# what the same counters read for a copy of known size.  The record names the
# sources it was measured on; a changed kernel reports traffic null.
TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "traffic__attn_d64_kernel_bf16__vitl_24_block_frame_step.txt")
KERNEL_SOURCES = ["paged_kv_cache_312_amd/csrc/hip/attn16.hip",
                  "paged_kv_cache_312_amd/csrc/hip/attn_common.h",
                  "paged_kv_cache_312_amd/csrc/hip/merge.hip",
                  "paged_kv_cache_312_amd/csrc/hip/append.hip",
                  "paged_kv_cache_312_amd/csrc/hip/kernels.h",
                  "paged_kv_cache_312_amd/csrc/hip/api.hip"]
APPEND_SOURCES = ["paged_kv_cache_312_amd/csrc/hip/append.hip",
                  "paged_kv_cache_312_amd/csrc/hip/kernels.h"]
COPY_BYTES = 1 << 30


def kernel_source_hash(root: str = ROOT, sources=None) -> str:
    """Hash of the append, attention and merge sources (or of ``sources``) with
    comments and blank space removed (a comment edit does not change the
    kernel)."""
    import hashlib
    import re
    h = hashlib.sha256()
    for rel in (KERNEL_SOURCES if sources is None else sources):
        with open(os.path.join(root, rel)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        h.update("\n".join(" ".join(l.split()) for l in text.splitlines() if l.strip()).encode())
    return h.hexdigest()[:16]


def _traffic_record():
    try:
        with open(TRAFFIC_RECORD) as f:
            return json.loads(f.read().split("\n", 1)[1])
    except (OSError, ValueError, IndexError):
        return None


def recorded_traffic():
    """HBM bytes of one block's attention and merge (the roofline's kernels)
    from the traffic record, or None if it is missing or was measured on other
    kernel sources."""
    rec = _traffic_record()
    if rec is None or rec.get("kernel_source_hash") != kernel_source_hash():
        return None
    return rec.get("hbm_bytes_per_lbm_run")


def recorded_append_traffic():
    """HBM bytes of one single-frame append (K and V rows of one block) from
    the traffic record, or None if it is missing or was measured on other
    append sources."""
    rec = _traffic_record()
    if rec is None or rec.get("append_source_hash") != kernel_source_hash(sources=APPEND_SOURCES):
        return None
    return rec.get("hbm_bytes_per_append")


def bf16_kernel(name: str, base: str) -> bool:
    """Whether a profiler kernel name (demangled or mangled) is the bf16
    instance of the template ``base``."""
    return base in name and ("__bf16" in name or "DF16b" in name)


def pmc_summary(fetch_dir, write_dir):
    """Per-dispatch FETCH_SIZE / WRITE_SIZE (KiB) of the timed attention and
    merge launches and of the calibration copies -> traffic record."""
    import csv
    import glob
    import statistics

    def load(d, counter):
        paths = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
        if not paths:
            raise SystemExit(f"no counter_collection.csv under {d}")
        per = {}
        for path in paths:
            for r in csv.DictReader(open(path)):
                if r["Counter_Name"] != counter:
                    continue
                did = int(r["Dispatch_Id"])
                name = r["Kernel_Name"]
                per.setdefault(did, [name, 0.0])[1] += float(r["Counter_Value"])
        return per

    out = {}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        per = load(d, counter)
        ids = sorted(per)
        # steady state only: the two timed steps (48 calls at F = 73, 74:
        # append, attention, merge each), not the append-timing step after
        # them (24 appends, then 24 attention launches) nor the first step and
        # the fill steps (other shapes) (the counter runs time bf16 only, so
        # every attention instance is a bf16 one)
        attn = [per[i][1] for i in ids if "attn_d64_kernel" in per[i][0]][-72:-24]
        merge = [per[i][1] for i in ids if bf16_kernel(per[i][0], "merge_kernel")][-72:-24]
        apps = [per[i][1] for i in ids if "append_scatter_kernel" in per[i][0]]
        app_run = apps[-72:-24]
        # the single-frame appends of blocks 1..23 of the append-timing step
        app = apps[-23:]
        copy = [per[i][1] for i in ids if "elementwise" in per[i][0]][-3:]
        if not attn or len(copy) < 3:
            raise SystemExit(f"{counter}: attention or calibration dispatches missing")
        out[counter] = {"attn_kib": statistics.mean(attn),
                        "merge_kib": statistics.mean(merge) if merge else 0.0,
                        "merges_per_attn": len(merge) / len(attn),
                        "run_append_kib": statistics.mean(app_run) if app_run else 0.0,
                        "appends_per_attn": len(app_run) / len(attn),
                        "append_kib": statistics.mean(app) if app else None,
                        "copy_kib": statistics.mean(copy)}
    f, w = out["FETCH_SIZE"], out["WRITE_SIZE"]
    f_scale = COPY_BYTES / (f["copy_kib"] * 1024.0)
    w_scale = COPY_BYTES / (w["copy_kib"] * 1024.0)

    def run_kib(x):     # the roofline's kernels: attention and merge
        return x["attn_kib"] + x["merge_kib"] * x["merges_per_attn"]

    fetch_b = run_kib(f) * 1024.0 * f_scale
    write_b = run_kib(w) * 1024.0 * w_scale
    call_b = (fetch_b + write_b + f["run_append_kib"] * f["appends_per_attn"] * 1024.0 * f_scale
              + w["run_append_kib"] * w["appends_per_attn"] * 1024.0 * w_scale)
    rec = {"kernel_source_hash": kernel_source_hash(),
           "hbm_bytes_per_lbm_run": round(fetch_b + write_b),
           "fetch_bytes": round(fetch_b), "write_bytes": round(write_b),
           "hbm_bytes_per_append_run": round(call_b),
           "fetch_scale": round(f_scale, 4), "write_scale": round(w_scale, 4),
           "raw_kib": out, "copy_bytes": COPY_BYTES}
    if f["append_kib"] is not None and w["append_kib"] is not None:
        a_fetch = f["append_kib"] * 1024.0 * f_scale
        a_write = w["append_kib"] * 1024.0 * w_scale
        rec.update(append_source_hash=kernel_source_hash(sources=APPEND_SOURCES),
                   hbm_bytes_per_append=round(a_fetch + a_write),
                   append_fetch_bytes=round(a_fetch), append_write_bytes=round(a_write))
    os.makedirs(os.path.dirname(TRAFFIC_RECORD), exist_ok=True)
    with open(TRAFFIC_RECORD, "w") as fh:
        fh.write("HBM traffic of the attention and merge of one block's call (hbm_bytes_per_lbm_run), "
                 "of the whole lbm_append_run with its append (hbm_bytes_per_append_run) and of one "
                 "single-frame append, 24-block ViT-L step; written by "
                 "'bench.py --pmc-summary' from two rocprofv3 --pmc runs of 'bench.py --steps 2 "
                 "--warmup 0 --no-cpu-baseline --no-variants --no-windows --calibrate-copy' (FETCH_SIZE, "
                 "then WRITE_SIZE)\n")
        fh.write(json.dumps(rec, indent=1) + "\n")
    print(json.dumps(rec))



class Stream:
    """One synthetic stream of ``cfg`` in a live cache: the first step, then
    single frames drawn from N_INPUT_SETS seeded input sets per block (resident
    in HBM, cycled).  A frame step appends every block's rows, evicts and
    plans once (at block 0) and runs attention per block: with ``fused``, one
    lbm_append_run per block (append and attention in one call), else
    lbm_append_frame, lbm_evict_frames, lbm_plan and lbm_run.  A fast-forward
    step (``run=False``) appends and evicts only."""

    def __init__(self, cfg, dev, splits_req=0, fused=True):
        import torch

        import paged_kv_cache_312_amd as lbm
        import workloads

        self.cfg, self.dev = cfg, dev
        B, H, D, T = cfg.num_blocks, cfg.num_heads, cfg.head_dim, cfg.tokens_per_frame
        fields = workloads.lbm_config_fields(cfg, num_splits=splits_req)
        self.cache = lbm.PagedKVCache(lbm.make_config(**fields), dev)
        self.stream = torch.cuda.current_stream()
        self.init = [workloads.gen_step_qkv(cfg, b, 0, cfg.initial_frames, dev) for b in range(B)]
        self.sets = [[workloads.gen_step_qkv(cfg, b, 1 + i, 1, dev) for b in range(B)]
                     for i in range(N_INPUT_SETS)]
        self.outs = [torch.empty((T, H, D), dtype=self.cache.dtype, device=dev) for _ in range(B)]
        self.F = 0
        self.step_idx = 0
        self.fused = fused
        torch.cuda.synchronize()

    def frame_step(self, inputs, out_bufs, nq, ev=None, ev_block=-1, run=True):
        cache = self.cache
        if run and self.fused:
            for b in range(self.cfg.num_blocks):
                q, k, v = inputs[b]
                if b == ev_block:
                    ev[0].record(self.stream)
                cache.append_run(b, q, k, v, out_bufs[b])
                if b == ev_block:
                    ev[1].record(self.stream)
            return
        for b in range(self.cfg.num_blocks):
            q, k, v = inputs[b]
            cache.append_frame(b, k, v)
            if b == 0:
                cache.evict_frames()
                if run:
                    cache.plan(nq)
            if not run:
                continue
            if b == ev_block:
                ev[0].record(self.stream)
            cache.run(b, q, out_bufs[b])
            if b == ev_block:
                ev[1].record(self.stream)

    def first(self, run=True):
        """The first step (initial_frames frames)."""
        import torch
        cfg = self.cfg
        out_init = None
        if run:
            out_init = torch.empty((cfg.initial_frames * cfg.tokens_per_frame, cfg.num_heads,
                                    cfg.head_dim), dtype=self.cache.dtype, device=self.dev)
        self.frame_step(self.init, [out_init] * cfg.num_blocks,
                        cfg.initial_frames * cfg.tokens_per_frame, run=run)
        self.F = cfg.initial_frames

    def advance(self, n, run=True):
        """n single-frame steps (with attention, or appends and evictions only)."""
        T = self.cfg.tokens_per_frame
        for _ in range(n):
            self.frame_step(self.sets[self.step_idx % N_INPUT_SETS], self.outs, T, run=run)
            self.F += 1
            self.step_idx += 1

    def window(self, steps):
        """Time ``steps`` frame steps: wall clock over the whole steps, and HIP
        events on the launch stream around one call per step (lbm_append_run:
        append, attention, merge; separate calls: lbm_run's attention and
        merge) (block i mod B of step i, or 1 + i mod (B-1) with
        lbm_append_run, whose block 0 also plans: every block's launch has
        the same shape within a step, and an event pair at every launch would
        itself add ~6 us of queue work per event to the steps being timed)."""
        import statistics

        import torch
        cfg = self.cfg
        B, H, D, T = cfg.num_blocks, cfg.num_heads, cfg.head_dim, cfg.tokens_per_frame
        F_first = self.F + 1
        ev = [[torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)]
              for _ in range(steps)]
        kv_lens = []
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            # with fused calls block 0's call also plans (table upload, row
            # table kernel) before its launch: bracket the other blocks
            eb = 1 + i % (B - 1) if self.fused and B > 1 else i % B
            self.frame_step(self.sets[self.step_idx % N_INPUT_SETS], self.outs, T, ev[i], eb)
            self.F += 1
            self.step_idx += 1
            # past the window fill every frame adds special_per_frame keys
            kv_lens.append(self.cache.get_plan()[0] if i == 0
                           else kv_lens[-1] + cfg.special_per_frame)
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
        assert self.cache.stats()["frame_count"] == self.F
        launch_ms = [e0.elapsed_time(e1) for e0, e1 in ev]
        flops = sum(4.0 * T * kv * H * D for kv in kv_lens)
        attn_ms = sum(launch_ms)
        return {"fps": steps / elapsed, "ms_per_step": elapsed * 1e3 / steps,
                "tflops": flops / (attn_ms * 1e-3) / 1e12, "avg_launch_ms": attn_ms / steps,
                "median_launch_ms": statistics.median(launch_ms), "flops": flops,
                "n_launch": steps, "kv_lens": kv_lens, "splits": self.cache.num_splits(),
                "F_first": F_first, "F_last": self.F}

    def close(self):
        self.cache.close()


def window_record(w, peak, blocks):
    """The JSON form of one timed window."""
    return {"timed_frames": [w["F_first"], w["F_last"]], "kv_len": [w["kv_lens"][0], w["kv_lens"][-1]],
            "blocks": blocks, "value": round(w["fps"], 3), "unit": "frames/s",
            "ms_per_step": round(w["ms_per_step"], 4),
            "attention_tflops": round(w["tflops"], 2), "frac": round(w["tflops"] / peak, 4),
            "avg_launch_ms": round(w["avg_launch_ms"], 4),
            "median_launch_ms": round(w["median_launch_ms"], 4), "key_splits": w["splits"]}


def measure_end_window(cfg, dev, steps, splits_req=0, fused=True):
    """The last ``steps`` frames of ``cfg``'s stream: the frames before them
    only append and evict (no attention), then the timed window."""
    s = Stream(cfg, dev, splits_req, fused)
    try:
        s.first(run=False)
        s.advance(cfg.total_frames - steps - s.F, run=False)
        return s.window(steps)
    finally:
        s.close()


def measure_stream(cfg, dev, steps, warmup, splits_req=0, keep=False, skip_steps=0,
                   end_steps=0, fused=True):
    """Stream ``cfg`` through its first step and the window fill, ``warmup``
    more steps, then time ``steps`` frame steps (all blocks: append, evict and
    plan once, attention) and one event pair around the appends of blocks
    1 .. B-1 of one further step; then, with ``end_steps``, append and evict
    only up to the stream's last ``end_steps`` frames and time those; then
    ``skip_steps`` skip-append frames (each frame's queries over the visible
    set and its own rows, nothing stored).  Returns the figures (and, with
    ``keep``, the live cache and inputs for the CPU baseline)."""
    import torch

    B, H, D, T = cfg.num_blocks, cfg.num_heads, cfg.head_dim, cfg.tokens_per_frame
    st = Stream(cfg, dev, splits_req, fused)
    cache, stream, sets, outs = st.cache, st.stream, st.sets, st.outs
    st.first()
    st.advance(cfg.scale_frames + cfg.sliding_window - st.F)
    st.advance(warmup)
    torch.cuda.synchronize()
    w = st.window(steps)
    F, step_idx = st.F, st.step_idx

    # append bandwidth: one more full step whose appends of blocks 1 .. B-1 go
    # back to back between one event pair.  Block 0's append (which reserves
    # the step's pages), the plan (table upload, row table kernel) and block
    # 0's attention come first; the host queues the 23 appends while that
    # attention runs, so the pair times the appends on the device, not the
    # rate at which the host submits them.
    e_app = [torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)]
    inputs = sets[step_idx % N_INPUT_SETS]
    cache.append_frame(0, inputs[0][1], inputs[0][2])
    cache.evict_frames()
    cache.plan(T)
    cache.run(0, inputs[0][0], outs[0])
    e_app[0].record(stream)
    for b in range(1, B):
        cache.append_frame(b, inputs[b][1], inputs[b][2])
    e_app[1].record(stream)
    for b in range(1, B):
        cache.run(b, inputs[b][0], outs[b])
    torch.cuda.synchronize()
    st.F += 1
    st.step_idx += 1
    app_ms = e_app[0].elapsed_time(e_app[1]) / (B - 1)
    app_bytes = 2 * 2 * T * H * D * cache.dtype.itemsize  # K and V rows, read + write
    append_gbps = app_bytes / (app_ms * 1e-3) / 1e9

    # the stream's last end_steps frames, reached by appends and evictions only
    end = None
    if end_steps > 0 and st.F + end_steps <= cfg.total_frames:
        st.advance(cfg.total_frames - end_steps - st.F, run=False)
        end = st.window(end_steps)

    skip = None
    if skip_steps > 0:
        kv_cache = cache.get_plan()[0]
        F_skip = st.F
        ev_s = [[torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)]
                for _ in range(skip_steps)]
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        for i in range(skip_steps):
            inputs = sets[(st.step_idx + i) % N_INPUT_SETS]
            cache.plan_transient(T, T)
            for b in range(B):
                q, k, v = inputs[b]
                if b == i % B:
                    ev_s[i][0].record(stream)
                cache.run_transient(b, q, k, v, outs[b])
                if b == i % B:
                    ev_s[i][1].record(stream)
        torch.cuda.synchronize()
        el = time.perf_counter() - t1
        s_ms = sum(e0.elapsed_time(e1) for e0, e1 in ev_s)
        s_flops = skip_steps * 4.0 * T * (kv_cache + T) * H * D
        skip = {"fps": skip_steps / el, "tflops": s_flops / (s_ms * 1e-3) / 1e12,
                "avg_launch_ms": s_ms / skip_steps, "kv_len": kv_cache + T, "F": F_skip}
        assert cache.stats()["frame_count"] == F_skip   # nothing appended by the skip frames

    res = {"fps": w["fps"], "ms_per_step": w["ms_per_step"], "tflops": w["tflops"],
           "avg_launch_ms": w["avg_launch_ms"], "median_launch_ms": w["median_launch_ms"],
           "flops": w["flops"], "n_launch": w["n_launch"], "kv_lens": w["kv_lens"],
           "splits": w["splits"], "F_first": w["F_first"], "F_last": w["F_last"],
           "app_ms": app_ms, "app_bytes": app_bytes, "append_gbps": append_gbps, "skip": skip,
           "end": end}
    if keep:
        res.update(_cache=cache, _init=st.init, _sets=sets, _F=F)
    else:
        cache.close()
    return res


def measure_batch(cfg, dev, n_streams, steps, splits_req=0, n_sets=2):
    """n_streams independent streams of ``cfg`` (distinct seeds), each filled
    to a full window, then ``steps`` frame steps in which every block runs as
    one batched launch over all streams (lbm_run_batch).  Returns aggregate
    frames/s and the attention TFLOP/s of the batched launches."""
    import torch

    import paged_kv_cache_312_amd as lbm
    import workloads

    B, H, D, T = cfg.num_blocks, cfg.num_heads, cfg.head_dim, cfg.tokens_per_frame
    cfgs = [cfg.replace(base_seed=100 + i) for i in range(n_streams)]
    caches = [lbm.PagedKVCache(lbm.make_config(**workloads.lbm_config_fields(c, num_splits=splits_req)), dev)
              for c in cfgs]
    init = [[workloads.gen_step_qkv(c, b, 0, c.initial_frames, dev) for b in range(B)] for c in cfgs]
    sets = [[[workloads.gen_step_qkv(c, b, 1 + i, 1, dev) for b in range(B)] for i in range(n_sets)]
            for c in cfgs]
    outs = [[torch.empty((T, H, D), dtype=caches[0].dtype, device=dev) for _ in range(B)]
            for _ in range(n_streams)]
    stream = torch.cuda.current_stream()

    def append_all(si, inputs, nq):
        for b in range(B):
            caches[si].append_frame(b, inputs[b][1], inputs[b][2])
            if b == 0:
                caches[si].evict_frames()
                caches[si].plan(nq)

    for si in range(n_streams):                       # fill: appends only
        append_all(si, init[si], cfg.initial_frames * T)
        for f in range(cfg.scale_frames + cfg.sliding_window - cfg.initial_frames):
            append_all(si, sets[si][f % n_sets], T)
    torch.cuda.synchronize()
    # one batched launch per step bracketed by events (block i mod B of step i)
    ev = [[torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)]
          for _ in range(steps)]
    flops = 0.0
    t0 = time.perf_counter()
    for i in range(steps):
        for b in range(B):
            for si in range(n_streams):
                x = sets[si][i % n_sets][b]
                caches[si].append_frame(b, x[1], x[2])
                if b == 0:
                    caches[si].evict_frames()
                    caches[si].plan(T)
            if b == i % B:
                ev[i][0].record(stream)
            lbm.PagedKVCache.run_batch(caches, b, [sets[si][i % n_sets][b][0]
                                                   for si in range(n_streams)],
                                       [outs[si][b] for si in range(n_streams)])
            if b == i % B:
                ev[i][1].record(stream)
        flops += sum(4.0 * T * c.get_plan()[0] * H * D for c in caches)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    attn_ms = sum(e0.elapsed_time(e1) for e0, e1 in ev)
    F = caches[0].stats()["frame_count"]
    for c in caches:
        c.close()
    return {"fps": n_streams * steps / elapsed, "tflops": flops / (attn_ms * 1e-3) / 1e12,
            "avg_launch_ms": attn_ms / steps, "F_last": F}


def measure_graph(cfg, dev, steps, n_sets=N_INPUT_SETS):
    """The stream of ``cfg`` filled to a full window with the individual
    calls, then ``steps`` frame steps each replayed as one HIP graph (one graph
    per resident input set, its outputs in fixed buffers).  Returns frames/s
    and the host time to submit one step: through the graph, and through the
    individual calls (append, evict, plan, run per block) for comparison."""
    import statistics

    import torch

    import paged_kv_cache_312_amd as lbm
    import workloads

    B, H, D, T = cfg.num_blocks, cfg.num_heads, cfg.head_dim, cfg.tokens_per_frame
    cache = lbm.PagedKVCache(lbm.make_config(**workloads.lbm_config_fields(cfg)), dev)
    init = [workloads.gen_step_qkv(cfg, b, 0, cfg.initial_frames, dev) for b in range(B)]
    sets = [[workloads.gen_step_qkv(cfg, b, 1 + i, 1, dev) for b in range(B)] for i in range(n_sets)]
    outs = [torch.empty((T, H, D), dtype=cache.dtype, device=dev) for _ in range(B)]
    out_init = torch.empty((cfg.initial_frames * T, H, D), dtype=cache.dtype, device=dev)

    def calls(inputs, nq, out_bufs):
        for b in range(B):
            q, k, v = inputs[b]
            cache.append_frame(b, k, v)
            if b == 0:
                cache.evict_frames()
                cache.plan(nq)
            cache.run(b, q, out_bufs[b])

    calls(init, cfg.initial_frames * T, [out_init] * B)
    for f in range(cfg.scale_frames + cfg.sliding_window - cfg.initial_frames):
        calls(sets[f % n_sets], T, outs)
    graphs = [cache.capture_step(1, [x[1] for x in st], [x[2] for x in st], [x[0] for x in st],
                                 outs) for st in sets]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        graphs[i % n_sets].launch()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    host_graph, host_calls = [], []
    for i in range(5):
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        graphs[i % n_sets].launch()
        host_graph.append(time.perf_counter() - t1)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        calls(sets[i % n_sets], T, outs)
        host_calls.append(time.perf_counter() - t1)
    torch.cuda.synchronize()
    ns = graphs[0].num_splits()
    for g in graphs:
        g.close()
    cache.close()
    return {"fps": steps / elapsed, "ms_per_step": elapsed * 1e3 / steps,
            "host_submit_ms_graph": statistics.median(host_graph) * 1e3,
            "host_submit_ms_calls": statistics.median(host_calls) * 1e3, "splits": ns}


def main():
    args = parse()
    if args.pmc_summary:
        pmc_summary(*args.pmc_summary)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path (independent "
              "streams would take one cache per GPU; one stream would shard its heads across "
              "GPUs with replicated page bookkeeping).", file=sys.stderr)
        sys.exit(2)

    import torch

    import workloads

    cfg = workloads.get_config("vitl_24_block_frame_step")
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    m = measure_stream(cfg, dev, args.steps, args.warmup, args.splits, keep=True,
                       skip_steps=0 if args.no_variants else args.skip_steps,
                       end_steps=0 if args.no_windows else args.end_steps)
    B, H, D, T = cfg.num_blocks, cfg.num_heads, cfg.head_dim, cfg.tokens_per_frame
    cache, init, sets, F = m.pop("_cache"), m.pop("_init"), m.pop("_sets"), m.pop("_F")
    kv_lens, splits = m["kv_lens"], m["splits"]
    fps, ms_per_step, achieved_tflops = m["fps"], m["ms_per_step"], m["tflops"]
    avg_launch_ms, flops, n_launch = m["avg_launch_ms"], m["flops"], m["n_launch"]
    F_first = m["F_first"]
    app_ms, app_bytes, append_gbps = m["app_ms"], m["app_bytes"], m["append_gbps"]

    result = {
        "metric": "frames/sec per 24-block step at window 64 + attention MFMA util vs bf16 peak",
        "value": round(fps, 3),
        "unit": "frames/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": cfg.name, "blocks": B, "heads": H, "head_dim": D,
                   "patches_per_frame": cfg.patches_per_frame,
                   "special_per_frame": cfg.special_per_frame, "scale_frames": cfg.scale_frames,
                   "sliding_window": cfg.sliding_window, "timed_frames": [F_first, F],
                   "kv_len": [kv_lens[0], kv_lens[-1]], "query_tokens": T,
                   "key_splits": splits},
        "roofline": {"bound": "mfma", "achieved": round(achieved_tflops, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved_tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": recorded_traffic(),
                     "kernel": "attn_d64_kernel<__bf16> (+ merge_kernel, after the block's "
                               "append_scatter_kernel): one lbm_append_run",
                     "avg_launch_ms": round(avg_launch_ms, 4),
                     "flops_per_launch_avg": flops / n_launch},
        # each timed call runs the block's append kernel before its attention
        # (lbm_append_run); the append kernel's rate is timed on one more step,
        # its 23 appends back to back between one event pair, and the whole
        # step made of separate calls is a variant below
        "append": {"mode": "append kernel before the attention launch, in the same call",
                   "kernel": {
                       "bound": "hbm", "achieved": round(append_gbps, 1), "peak": PEAK_HBM_GBPS,
                       "unit": "GB/s", "frac": round(append_gbps / PEAK_HBM_GBPS, 4),
                       "traffic": recorded_append_traffic(),
                       "avg_launch_ms": round(app_ms, 5), "bytes_per_launch": app_bytes}},
    }

    cache.close()
    if m["skip"] is not None:
        sk = m["skip"]
        result["variants"] = {"skip_append_bf16": {
            "value": round(sk["fps"], 3), "unit": "frames/s", "steps": args.skip_steps,
            "kv_len": sk["kv_len"], "attention_tflops": round(sk["tflops"], 2),
            "frac": round(sk["tflops"] / PEAK_BF16_TFLOPS, 4), "peak": PEAK_BF16_TFLOPS,
            "avg_launch_ms": round(sk["avg_launch_ms"], 4)}}
    if not args.no_variants:
        # the same stream made of separate calls per block (lbm_append_frame,
        # then lbm_run; evict and plan once): the same kernels, and the events
        # bracket lbm_run alone (attention and merge, not the append)
        v = measure_stream(cfg, dev, args.variant_steps, args.warmup, args.splits, fused=False)
        result.setdefault("variants", {})["separate_calls_bf16"] = {
            "value": round(v["fps"], 3), "unit": "frames/s", "steps": args.variant_steps,
            "ms_per_step": round(v["ms_per_step"], 4),
            "timed_frames": [v["F_first"], v["F_last"]],
            "attention_tflops": round(v["tflops"], 2),
            "frac": round(v["tflops"] / PEAK_BF16_TFLOPS, 4), "peak": PEAK_BF16_TFLOPS,
            "avg_launch_ms": round(v["avg_launch_ms"], 4), "key_splits": v["splits"]}
        # the same 24-block stream with fp16 storage and MFMA (the pages' other
        # 16-bit type); a shorter timed run after the same fill
        v = measure_stream(cfg.replace(dtype="f16"), dev, args.variant_steps, args.warmup,
                           args.splits)
        result.setdefault("variants", {})["fp16"] = {
            "value": round(v["fps"], 3), "unit": "frames/s", "steps": args.variant_steps,
            "timed_frames": [v["F_first"], v["F_last"]],
            "attention_tflops": round(v["tflops"], 2),
            "frac": round(v["tflops"] / PEAK_FP16_TFLOPS, 4), "peak": PEAK_FP16_TFLOPS,
            "avg_launch_ms": round(v["avg_launch_ms"], 4), "key_splits": v["splits"]}
        # the eviction call's include_scale_frames=False: no frame kept beyond
        # the window, so 8 fewer patch pages in the visible set
        v = measure_stream(cfg.replace(scale_frames=0), dev, args.variant_steps, args.warmup,
                           args.splits)
        result["variants"]["no_scale_frames_bf16"] = {
            "value": round(v["fps"], 3), "unit": "frames/s", "steps": args.variant_steps,
            "timed_frames": [v["F_first"], v["F_last"]],
            "kv_len": [v["kv_lens"][0], v["kv_lens"][-1]],
            "attention_tflops": round(v["tflops"], 2),
            "frac": round(v["tflops"] / PEAK_BF16_TFLOPS, 4), "peak": PEAK_BF16_TFLOPS,
            "avg_launch_ms": round(v["avg_launch_ms"], 4), "key_splits": v["splits"]}

        # the force_fp32 path (fp32 storage, fp32 MFMA products and softmax)
        # against the fp32 dense MFMA peak; a short timed run
        if args.f32_steps > 0:
            v = measure_stream(cfg.replace(dtype="f32"), dev, args.f32_steps, args.warmup,
                               args.splits)
            result["variants"]["fp32"] = {
                "value": round(v["fps"], 3), "unit": "frames/s", "steps": args.f32_steps,
                "timed_frames": [v["F_first"], v["F_last"]],
                "attention_tflops": round(v["tflops"], 2),
                "frac": round(v["tflops"] / PEAK_FP32_TFLOPS, 4), "peak": PEAK_FP32_TFLOPS,
                "avg_launch_ms": round(v["avg_launch_ms"], 4), "key_splits": v["splits"],
                "append_gbps": round(v["append_gbps"], 1)}

    if not args.no_variants and args.graph_steps > 0:
        gr = measure_graph(cfg, dev, args.graph_steps)
        result.setdefault("variants", {})["graph_bf16"] = {
            "value": round(gr["fps"], 3), "unit": "frames/s", "steps": args.graph_steps,
            "ms_per_step": round(gr["ms_per_step"], 4), "key_splits": gr["splits"],
            "host_submit_ms_graph": round(gr["host_submit_ms_graph"], 3),
            "host_submit_ms_calls": round(gr["host_submit_ms_calls"], 3)}

    if not args.no_variants and args.batch_streams > 1:
        bt = measure_batch(cfg, dev, args.batch_streams, args.batch_steps, args.splits)
        result.setdefault("variants", {})[f"batch{args.batch_streams}_bf16"] = {
            "value": round(bt["fps"], 3), "unit": "frames/s (all streams)",
            "streams": args.batch_streams, "steps": args.batch_steps,
            "attention_tflops": round(bt["tflops"], 2),
            "frac": round(bt["tflops"] / PEAK_BF16_TFLOPS, 4), "peak": PEAK_BF16_TFLOPS,
            "avg_launch_ms": round(bt["avg_launch_ms"], 4)}

    if not args.no_windows:
        # the work per frame grows with the special stream (6 keys a frame):
        # the first window, the 1000-frame stream's last frames, and the last
        # frames of the 10,000-frame stream (4 blocks, 38% of its keys special)
        import statistics
        wins = {"first": window_record(m, PEAK_BF16_TFLOPS, B)}
        if m["end"] is not None:
            wins["stream_end"] = window_record(m["end"], PEAK_BF16_TFLOPS, B)
        if args.long_end_steps > 0:
            lcfg = workloads.get_config("vitl_long_stream")
            lw = measure_end_window(lcfg, dev, args.long_end_steps, args.splits)
            wins["long_stream_end"] = dict(window_record(lw, PEAK_BF16_TFLOPS, lcfg.num_blocks),
                                           workload=lcfg.name)
        fr = [w["frac"] for w in wins.values()]
        result["windows"] = dict(wins, frac_median=round(statistics.median(fr), 4),
                                 frac_min=min(fr), frac_max=max(fr))

    if args.calibrate_copy:
        src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        del src, dst

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(cfg, init, sets, F, args.cpu_seconds)
    print(json.dumps(result), flush=True)


def host_identity():
    """The host CPU's model name (/proc/cpuinfo), the CPUs this process may
    run on, and the BLAS library numpy calls (threadpoolctl: library, version,
    threads, file)."""
    import numpy  # noqa: F401  (loads the BLAS that threadpoolctl inspects)
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = None
    try:
        from threadpoolctl import threadpool_info
        infos = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if infos:
            i = infos[0]
            blas = {"library": i.get("internal_api"), "version": i.get("version"),
                    "threads": i.get("num_threads"),
                    "file": os.path.basename(i.get("filepath") or "")}
    except Exception:
        pass
    try:
        cpus = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        cpus = os.cpu_count()
    return {"cpu_model": model, "blas": blas, "host_cpus": cpus}


def cpu_baseline(cfg, init, sets, F_now, budget_s):
    """The oracle as it stands, timed on this host on a bounded sample of one
    steady-state frame step: block 0, the step's 1375 query rows, h heads,
    against the full visible set at the current frame count; scaled to the
    whole 24-block, 16-head step."""
    import numpy as np
    import torch
    from oracle import StreamOracle
    ident = host_identity()
    threads = (ident["blas"] or {}).get("threads") or os.cpu_count() or 1

    B, H, T = cfg.num_blocks, cfg.num_heads, cfg.tokens_per_frame

    n0 = cfg.initial_frames

    class CycledHistory:
        """The bytes the bench appended: frames of the first step from its
        tensors, frame f >= n0 from input set (f - n0) mod n."""
        def __init__(self):
            self.cache = {}

        def rows(self, block, frame, lo, hi, heads=None):
            key = ("i", block) if frame < n0 else ((frame - n0) % len(sets), block)
            if key not in self.cache:
                _, k, v = init[block] if frame < n0 else sets[key[0]][block]
                self.cache[key] = (k.double().cpu().numpy(), v.double().cpu().numpy())
            k, v = self.cache[key]
            if frame < n0:
                k, v = k[frame * T:(frame + 1) * T], v[frame * T:(frame + 1) * T]
            k, v = k[lo:hi], v[lo:hi]
            if heads is not None:
                k, v = k[:, heads], v[:, heads]
            return k, v

    orc = StreamOracle(cfg.patches_per_frame, cfg.special_per_frame, cfg.scale_frames,
                       cfg.sliding_window, history=CycledHistory())
    orc.F = F_now
    q, k, v = (t.double().cpu().numpy() for t in sets[(F_now - n0) % len(sets)][0])
    t0 = time.perf_counter()
    orc.step_outputs(0, q, k, v, heads=[0])
    t1 = time.perf_counter() - t0
    n_heads = int(max(1, min(H, budget_s // max(t1, 1e-3))))
    t0 = time.perf_counter()
    if n_heads > 1:
        orc.step_outputs(0, q, k, v, heads=list(range(1, n_heads)))
    t_rest = time.perf_counter() - t0
    per_head = (t1 + t_rest) / n_heads
    step_s = per_head * H * B
    return {"value": round(1.0 / step_s, 6), "unit": "frames/s", "cores": threads,
            "kind": "oracle", "cpu_model": ident["cpu_model"], "blas": ident["blas"],
            "host_cpus": ident["host_cpus"],
            "sample": (f"block 0, {n_heads} of {H} heads, all {T} query rows of one frame step "
                       f"at F={F_now + 1} (kv_len {98568 + 6 * (F_now + 1)}), fp64 numpy; "
                       f"{t1 + t_rest:.1f} s measured, scaled x{H * B / n_heads:.0f} to the "
                       f"24-block step ({step_s:.1f} s/frame)")}


if __name__ == "__main__":
    main()
