"""Several independent streams in one batched launch (lbm_run_batch): each
stream's output must equal its own lbm_run bit for bit when both use the same
split count, and the oracle within the usual tolerance."""
import numpy as np
import pytest
import torch

import paged_kv_cache_312_amd as lbm
import workloads
from gpu_helpers import (DEV, SeededHistory, compare, make_cache, ref_allocator, sample_rows,
                         say)
from oracle import StreamOracle
from test_gpu_parity import ODD_BF16, ODD_F16, ODD_F32

pytestmark = pytest.mark.gpu


class Stream:
    """One stream (cache + oracle) driven step by step."""

    def __init__(self, cfg, splits=0):
        self.cfg = cfg
        self.cache, fields = make_cache(cfg, num_splits=splits)
        self.ref = ref_allocator(cfg, fields)
        self.hist = SeededHistory(cfg)
        self.orc = StreamOracle(cfg.patches_per_frame, cfg.special_per_frame, cfg.scale_frames,
                                cfg.sliding_window, history=self.hist)
        self.sched = workloads.step_schedule(cfg)
        self.s = 0

    def inputs(self, b):
        return workloads.gen_step_qkv(self.cfg, b, self.s, self.sched[self.s], DEV)

    def append_block(self, b, k, v):
        self.cache.append_frame(b, k, v)
        if b == 0:
            nf = self.sched[self.s]
            self.ref.append(nf)
            assert self.cache.evict_frames() == self.ref.evict()
            self.cache.plan(nf * self.cfg.tokens_per_frame)

    def expected(self, b, q, k, v, rows=None):
        return self.orc.step_outputs(b, *[t.double().cpu().numpy() for t in (q, k, v)], rows=rows)

    def finish_step(self):
        assert self.cache.dump_state() == self.ref.dump()
        self.hist.accept(self.s)
        self.orc.commit_count(self.sched[self.s])
        self.hist.clear_cache()
        self.s += 1


def _lockstep(streams, steps, check_rows=None, bitwise=True):
    worst = 0.0
    for _ in range(steps):
        for b in range(streams[0].cfg.num_blocks):
            ins = [st.inputs(b) for st in streams]
            for st, (q, k, v) in zip(streams, ins):
                st.append_block(b, k, v)
            qs = [q for q, _, _ in ins]
            outs = lbm.PagedKVCache.run_batch([st.cache for st in streams], b, qs)
            if bitwise:
                for st, q, o in zip(streams, qs, outs):
                    assert torch.equal(st.cache.run(b, q), o), f"stream {st.cfg.name} step {st.s}"
            torch.cuda.synchronize()
            for st, (q, k, v), o in zip(streams, ins, outs):
                rows = None if check_rows is None else sample_rows(q.shape[0], check_rows, st.s)
                ref = st.expected(b, q, k, v, rows)
                g = o.double()
                if rows is not None:
                    g = g[torch.as_tensor(rows, device=g.device)]
                worst = max(worst, compare(g.cpu().numpy(), ref, st.cfg.dtype,
                                           f"{st.cfg.name} step {st.s} block {b}")["max_abs"])
        for st in streams:
            st.finish_step()
    return worst


@pytest.mark.parametrize("base", [ODD_BF16, ODD_F16, ODD_F32], ids=lambda c: c.name)
def test_three_small_streams_bitwise_and_oracle(base):
    """Three streams of different lengths and seeds, split count forced to 3:
    the batched launch equals each stream's own launch bit for bit."""
    cfgs = [base.replace(name=f"{base.name}_s{i}", base_seed=7 + i, total_frames=10 + 3 * i)
            for i in range(3)]
    streams = [Stream(c, splits=3) for c in cfgs]
    # advance the longer streams first so that key lengths differ
    for st, lead in zip(streams, (0, 2, 4)):
        for _ in range(lead):
            for b in range(st.cfg.num_blocks):
                q, k, v = st.inputs(b)
                st.append_block(b, k, v)
            st.finish_step()
    w = _lockstep(streams, 6)
    say(base.name, "worst", w)
    for st in streams:
        st.cache.close()


def test_two_vitl_streams():
    """Two ViT-L single-block streams at different lengths, planner-chosen
    splits for the combined work; oracle on sampled rows."""
    base = workloads.get_config(1)
    streams = [Stream(base.replace(name="vitl_a", base_seed=3, total_frames=90)),
               Stream(base.replace(name="vitl_b", base_seed=4, total_frames=90))]
    for _ in range(70):                      # stream a ahead: F = 77 vs 8 + ...
        st = streams[0]
        q, k, v = st.inputs(0)
        st.append_block(0, k, v)
        st.finish_step()
    for _ in range(3):
        st = streams[1]
        q, k, v = st.inputs(0)
        st.append_block(0, k, v)
        st.finish_step()
    w = _lockstep(streams, 2, check_rows=48, bitwise=False)
    say("vitl batch worst", w)
    for st in streams:
        st.cache.close()


def test_batch_errors():
    a = Stream(ODD_BF16.replace(name="e_a"))
    f = Stream(ODD_F32.replace(name="e_f"))
    for st in (a, f):
        q, k, v = st.inputs(0)
        for b in range(st.cfg.num_blocks):
            st.append_block(b, *st.inputs(b)[1:])
    q = a.inputs(0)[0]
    with pytest.raises(lbm.LbmError) as e:
        lbm.lbm_run_batch([], 0, [], [], 0)
    assert e.value.name == "LBM_ERR_INVALID_ARG"
    with pytest.raises(lbm.LbmError) as e:
        lbm.PagedKVCache.run_batch([a.cache] * 9, 0, [q] * 9)
    assert e.value.name == "LBM_ERR_INVALID_ARG"
    with pytest.raises(lbm.LbmError) as e:                 # mixed dtypes
        lbm.lbm_run_batch([a.cache.handle, f.cache.handle], 0, [q.data_ptr(), q.data_ptr()],
                          [q.data_ptr(), q.data_ptr()], 0)
    assert e.value.name == "LBM_ERR_INVALID_ARG"
    T = a.cfg.tokens_per_frame
    nq = a.sched[0] * T
    a.cache.plan_transient(nq, T)                          # a skip-append plan
    with pytest.raises(lbm.LbmError) as e:
        lbm.PagedKVCache.run_batch([a.cache], 0, [q])
    assert e.value.name == "LBM_ERR_BAD_STATE"
    a.cache.plan(nq)
    with pytest.raises(lbm.LbmError) as e:                 # the same cache twice
        lbm.PagedKVCache.run_batch([a.cache, a.cache], 1, [q, q])
    assert e.value.name == "LBM_ERR_INVALID_ARG"
    out = lbm.PagedKVCache.run_batch([a.cache], 1, [q])
    torch.cuda.synchronize()
    assert torch.equal(out[0], a.cache.run(1, q))
    for st in (a, f):
        st.cache.close()
