"""Helpers of the GPU tests: drive a stream through the C ABI and check it
against the CPU oracle.

Inputs are drawn on the device by the shared seeded generators; the oracle
receives exactly those values (copied to the host, widened to fp64) and its
own visible-set rules.  Nothing here feeds a value produced by the library's
kernels into the oracle.
"""
from __future__ import annotations

import sys
from typing import Dict, Iterable, List, Optional, Sequence

import numpy as np
import torch

import paged_kv_cache_312_amd as lbm
import workloads
from oracle import RefAllocator, StreamOracle

DEV = "cuda"

BF16_MAX_ABS = 2e-2      # stated tolerance for bf16
BF16_REL_L2 = 1e-2       # self-gate (catches a dropped page the max-abs bound misses)
F32_MAX_ABS = 1e-5       # stated tolerance for fp32
F32_REL_L2 = 1e-5
# fp16: the bf16 bounds scaled by the ratio of unit roundoffs, 2^-12 / 2^-9
# (P, q*log2(e)/sqrt(D) and the output are rounded to fp16 instead of bf16)
F16_MAX_ABS = BF16_MAX_ABS / 8
F16_REL_L2 = BF16_REL_L2 / 8
TOLERANCES = {"bf16": (BF16_MAX_ABS, BF16_REL_L2), "f16": (F16_MAX_ABS, F16_REL_L2),
              "f32": (F32_MAX_ABS, F32_REL_L2)}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


class SeededHistory:
    """Oracle history that regenerates an accepted frame's K/V from its seed."""

    def __init__(self, cfg: workloads.StreamConfig, device=DEV):
        self.cfg = cfg
        self.device = device
        self.sched = workloads.step_schedule(cfg)
        self.frames: List[tuple] = []          # frame -> (step, index in step)
        self._cache: Dict[tuple, tuple] = {}

    def accept(self, step: int) -> None:
        for i in range(self.sched[step]):
            self.frames.append((step, i))

    def clear_cache(self):
        self._cache.clear()

    def _kv(self, block, step):
        key = (block, step)
        if key not in self._cache:
            if len(self._cache) > 64:
                self._cache.clear()
            k, v = workloads.gen_step_qkv(self.cfg, block, step, self.sched[step], self.device,
                                          tensors=("k", "v"))
            self._cache[key] = (k, v)
        return self._cache[key]

    def rows(self, block, frame, lo, hi, heads=None):
        step, i = self.frames[frame]
        k, v = self._kv(block, step)
        T = self.cfg.tokens_per_frame
        kk, vv = k[i * T + lo:i * T + hi], v[i * T + lo:i * T + hi]
        if heads is not None:
            kk, vv = kk[:, heads], vv[:, heads]
        return kk.double().cpu().numpy(), vv.double().cpu().numpy()


def make_cache(cfg: workloads.StreamConfig, num_splits=0, max_q_tokens=None, frames=None):
    fields = workloads.lbm_config_fields(cfg, max_q_tokens=max_q_tokens, num_splits=num_splits,
                                         frames=frames)
    return lbm.PagedKVCache(lbm.make_config(**fields), DEV), fields


def ref_allocator(cfg, fields):
    return RefAllocator(cfg.patches_per_frame, cfg.special_per_frame, cfg.special_page_size,
                        cfg.scale_frames, cfg.sliding_window, fields["max_patch_pages"],
                        fields["max_special_pages"], fields["max_frames_per_step"])


def compare(out_gpu: np.ndarray, ref: np.ndarray, dtype: str, what: str) -> dict:
    err = np.abs(out_gpu - ref)
    max_abs = float(err.max())
    rel = float(np.linalg.norm(out_gpu - ref) / max(np.linalg.norm(ref), 1e-300))
    lim_abs, lim_rel = TOLERANCES[dtype]
    assert np.isfinite(out_gpu).all(), f"{what}: non-finite output"
    assert max_abs <= lim_abs, f"{what}: max-abs {max_abs:.3e} > {lim_abs}"
    assert rel <= lim_rel, f"{what}: rel-L2 {rel:.3e} > {lim_rel}"
    return {"max_abs": max_abs, "rel_l2": rel}


def sample_rows(n_rows: int, k: int, step: int) -> np.ndarray:
    """k query rows spread over [0, n_rows), always including the first and the
    last (ragged-tail) rows, rotating with the step."""
    if k >= n_rows:
        return np.arange(n_rows)
    rng = np.random.default_rng(1000 + step)
    picks = set(rng.choice(n_rows, size=k - 2, replace=False).tolist())
    picks |= {0, n_rows - 1}
    return np.array(sorted(picks))[:k]


def run_stream(cfg: workloads.StreamConfig, check_steps: Optional[Iterable[int]] = None,
               rows_per_check: Optional[int] = None, heads: Optional[Sequence[int]] = None,
               blocks: Optional[Sequence[int]] = None, num_splits: int = 0,
               deferred: bool = False, accept: Optional[List[bool]] = None,
               dump_every: int = 1, q_scale: float = 1.0, run_every_step: bool = False,
               skip_steps: Iterable[int] = (), fused_steps: Iterable[int] = (),
               label: str = "") -> dict:
    """Drive the whole schedule of ``cfg`` through the library; check the
    bookkeeping against the reference allocator and, at the checked steps, the
    attention outputs against the oracle.  Steps in ``skip_steps`` (single
    frames) are skip-append frames: planned and run with the frame's own rows,
    never appended; the bookkeeping must not move.  Steps in ``fused_steps``
    go through lbm_append_run (append, plan, evict and attention of each block
    in one call).  Returns error statistics."""
    skip = set(skip_steps)
    fused = set(fused_steps)
    sched = workloads.step_schedule(cfg)
    accept = accept or [True] * len(sched)
    check = set(range(len(sched))) if check_steps is None else set(check_steps)
    blocks = list(range(cfg.num_blocks)) if blocks is None else list(blocks)
    cache, fields = make_cache(cfg, num_splits=num_splits)
    ref = ref_allocator(cfg, fields)
    hist = SeededHistory(cfg)
    orc = StreamOracle(cfg.patches_per_frame, cfg.special_per_frame, cfg.scale_frames,
                       cfg.sliding_window, history=hist)
    T = cfg.tokens_per_frame
    worst = {"max_abs": 0.0, "rel_l2": 0.0, "checks": 0, "splits": set()}
    stream = torch.cuda.current_stream()
    for s, nf in enumerate(sched):
        do_check = s in check
        do_run = do_check or run_every_step
        step_in = {}
        for b in range(cfg.num_blocks):
            q, k, v = workloads.gen_step_qkv(cfg, b, s, nf, DEV, q_scale=q_scale)
            step_in[b] = (q, k, v)
        if s in skip:
            assert nf == 1 and s > 0
            before, stats_before = cache.dump_state(), cache.stats()
            cache.plan_transient(T, T)
            worst["splits"].add(cache.num_splits())
            outs = {b: cache.run_transient(b, *step_in[b]) for b in blocks}
            assert cache.dump_state() == before and cache.stats() == stats_before, \
                f"{label} step {s}: skip-append moved the bookkeeping"
            assert ref.dump() == before
            if do_check:
                torch.cuda.synchronize()
                rows = None if rows_per_check is None else sample_rows(T, rows_per_check, s)
                hs = None if heads is None else list(heads)
                for b in blocks:
                    q, k, v = [t.double().cpu().numpy() for t in step_in[b]]
                    ref_out = orc.skip_append_outputs(b, q, k, v, rows=rows, heads=hs)
                    g = outs[b].double()
                    if rows is not None:
                        g = g[torch.as_tensor(rows, device=g.device)]
                    if hs is not None:
                        g = g[:, hs]
                    st = compare(g.cpu().numpy(), ref_out, cfg.dtype,
                                 f"{label} skip step {s} block {b}")
                    worst["max_abs"] = max(worst["max_abs"], st["max_abs"])
                    worst["rel_l2"] = max(worst["rel_l2"], st["rel_l2"])
                    worst["checks"] += 1
                hist.clear_cache()
                say(f"{label}: skip-append step {s} at F={orc.F} checked, worst so far "
                    f"max_abs={worst['max_abs']:.3e} rel_l2={worst['rel_l2']:.3e}")
            continue
        before = ref.dump() if not accept[s] else None
        # protocol: append(0), [evict], plan, run(0), then append(b), run(b);
        # fused: append_run(b) for every block (block 0 reserves, plans, evicts)
        outs = {}
        for b in range(cfg.num_blocks):
            q, k, v = step_in[b]
            if s in fused:
                assert accept[s] and not deferred
                if b == 0:
                    ref.append(nf)
                    ref.evict()
                o = cache.append_run(b, q, k, v)
                if b == 0:
                    worst["splits"].add(cache.num_splits())
                if b in blocks:
                    outs[b] = o
                continue
            cache.append_frame(b, k, v)
            if b == 0:
                ref.append(nf)
                if not deferred:
                    assert cache.evict_frames() == ref.evict()
                cache.plan(nf * T)
                worst["splits"].add(cache.num_splits())
            if do_run and (b in blocks):
                outs[b] = cache.run(b, q)
        if deferred:
            if accept[s]:
                assert cache.evict_frames() == ref.evict()
            else:
                cache.rollback_last_frame()
                ref.rollback()
                assert ref.dump() == before
        if s % dump_every == 0 or not accept[s] or s == len(sched) - 1:
            assert cache.dump_state() == ref.dump(), f"{label} step {s}: state"
            assert cache.get_plan() == ref.plan(), f"{label} step {s}: table"
        if do_check:
            torch.cuda.synchronize()
            rows = None if rows_per_check is None else sample_rows(nf * T, rows_per_check, s)
            hs = None if heads is None else list(heads)
            for b in blocks:
                q, k, v = step_in[b]
                ref_out = orc.step_outputs(b, q.double().cpu().numpy(), k.double().cpu().numpy(),
                                           v.double().cpu().numpy(), rows=rows, heads=hs)
                g = outs[b].double()
                if rows is not None:
                    g = g[torch.as_tensor(rows, device=g.device)]
                if hs is not None:
                    g = g[:, hs]
                st = compare(g.cpu().numpy(), ref_out, cfg.dtype, f"{label} step {s} block {b}")
                worst["max_abs"] = max(worst["max_abs"], st["max_abs"])
                worst["rel_l2"] = max(worst["rel_l2"], st["rel_l2"])
                worst["checks"] += 1
            hist.clear_cache()
            say(f"{label}: step {s} F={orc.F + nf} checked, worst so far "
                f"max_abs={worst['max_abs']:.3e} rel_l2={worst['rel_l2']:.3e}")
        if accept[s]:
            hist.accept(s)
            orc.commit_count(nf)
    cache.close()
    return worst
