"""The library's host bookkeeping (liblbm_core, the same C++ that runs inside
liblbm) against the oracle's reference allocator: bit-exact state and table
records after every operation of every workload's schedule."""
import random

import pytest

import workloads
from oracle.allocator import AllocatorError, RefAllocator
from paged_kv_cache_312_amd import CoreBookkeeping, LbmError, make_config


def _pair(cfg, **kw):
    fields = workloads.lbm_config_fields(cfg)
    core = CoreBookkeeping(make_config(**fields))
    ref = RefAllocator(cfg.patches_per_frame, cfg.special_per_frame, cfg.special_page_size,
                       cfg.scale_frames, cfg.sliding_window, cfg.max_patch_pages,
                       fields["max_special_pages"], fields["max_frames_per_step"], **kw)
    return core, ref


def _ref_write_map(ref, wm, nf, st0, sps):
    """The reference write map in the library's record format."""
    toks = [s for slots in wm["special_slots"] for s in slots]
    pages = []
    for p, _slot in toks:
        if not pages or pages[-1] != p:
            pages.append(p)
    return [nf] + wm["patch_pages"] + [st0, st0 // sps, len(pages)] + pages


def _lockstep(cfg, accept=None, check_every=1):
    core, ref = _pair(cfg)
    sched = workloads.step_schedule(cfg)
    accept = accept or [True] * len(sched)
    for s, (nf, ok) in enumerate(zip(sched, accept)):
        st0 = ref.special_tokens
        wm = ref.append(nf)
        core.append(nf)
        assert core.write_map() == _ref_write_map(ref, wm, nf, st0, cfg.special_page_size)
        if s % check_every == 0 or not ok:
            assert core.dump() == ref.dump()
            assert core.plan() == ref.plan()
        if ok:
            assert core.evict() == ref.evict()
        else:
            core.rollback()
            ref.rollback()
        if s % check_every == 0 or not ok:
            assert core.dump() == ref.dump()
            assert core.plan() == ref.plan()
            assert core.stats() == ref.stats()
    assert core.dump() == ref.dump()
    assert core.plan() == ref.plan()
    return core, ref


@pytest.mark.parametrize("cid", [0, 1, 2])
def test_core_matches_reference_allocator(cid):
    _lockstep(workloads.get_config(cid))


def test_core_matches_reference_no_scale_frames():
    """include_scale_frames=False of the pages' eviction call (scale_frames = 0):
    every frame ages out of the window."""
    core, ref = _lockstep(workloads.get_config(1).replace(scale_frames=0, total_frames=150))
    st = core.stats()
    assert st["scale_pages"] == 0 and st["live_pages"] == 64


@pytest.mark.parametrize("kw", [dict(special_per_frame=0), dict(sliding_window=0),
                                dict(scale_frames=0, sliding_window=1, initial_frames=1)],
                         ids=["no_special", "no_window", "window1_no_scale"])
def test_core_matches_reference_degenerate_configs(kw):
    """No special tokens, no window, a one-frame window without scale frames;
    with rejected frames rolled back."""
    cfg = workloads.get_config(0).replace(total_frames=40, reject_prob=0.3, **kw)
    acc = workloads.accept_draws(cfg)
    assert not all(acc)
    _lockstep(cfg, accept=acc)


def test_core_matches_reference_long_stream():
    """10,000 frames: ~9,900 evictions and 3,750 special pages."""
    core, ref = _lockstep(workloads.get_config(3), check_every=61)
    assert core.stats()["special_tokens"] == 60000
    assert core.plan()[2] == 3750


def test_core_matches_reference_with_rollbacks():
    cfg = workloads.get_config(4)
    acc = workloads.accept_draws(cfg)
    assert acc.count(False) > 100
    _lockstep(cfg, accept=acc)


def test_core_rollback_restores_snapshot():
    cfg = workloads.get_config(4)
    core, _ = _pair(cfg)
    for nf, ok in zip(workloads.step_schedule(cfg), workloads.accept_draws(cfg)):
        before = core.dump()
        core.append(nf)
        if ok:
            core.evict()
        else:
            core.rollback()
            assert core.dump() == before


def test_core_permuted_free_lists():
    cfg = workloads.get_config(0).replace(total_frames=30)
    rng = random.Random(5)
    fields = workloads.lbm_config_fields(cfg)
    po = list(range(cfg.max_patch_pages)); rng.shuffle(po)
    so = list(range(fields["max_special_pages"])); rng.shuffle(so)
    core, ref = _pair(cfg, patch_order=po, special_order=so)
    core.seed_free_lists(po, so)
    assert core.dump() == ref.dump()
    for nf in workloads.step_schedule(cfg):
        ref.append(nf); core.append(nf)
        assert core.evict() == ref.evict()
        assert core.plan() == ref.plan()
    core.reset(); ref.reset()
    assert core.dump() == ref.dump()


def test_stats_worked_example_through_core():
    """The pages' stats record through the library's bookkeeping."""
    cfg = make_config(num_blocks=12, num_heads=8, head_dim=64, patches_per_frame=256,
                      special_per_frame=6, special_page_size=16, scale_frames=8,
                      sliding_window=64, max_patch_pages=88, max_special_pages=64,
                      max_frames_per_step=5, max_q_tokens=1310, dtype=0)
    core = CoreBookkeeping(cfg)
    core.append(5); core.evict()
    for _ in range(37):
        core.append(1); core.evict()
    assert core.stats() == {"frame_count": 42, "scale_pages": 8, "live_pages": 34,
                            "free_pages": 46, "special_tokens": 252}


def test_core_errors():
    cfg = make_config(num_blocks=1, num_heads=1, head_dim=64, patches_per_frame=4,
                      special_per_frame=2, special_page_size=4, scale_frames=1,
                      sliding_window=2, max_patch_pages=4, max_special_pages=8,
                      max_frames_per_step=4, max_q_tokens=16, dtype=0)
    core = CoreBookkeeping(cfg)
    with pytest.raises(LbmError) as e:
        core.rollback()
    assert e.value.name == "LBM_ERR_BAD_STATE"
    core.append(3)
    with pytest.raises(LbmError) as e:
        core.rollback()
    assert e.value.name == "LBM_ERR_BAD_STATE"
    core.evict()
    core.append(1)
    core.evict()
    with pytest.raises(LbmError):
        core.rollback()
    before = core.dump()
    with pytest.raises(LbmError) as e:
        core.append(3)
    assert e.value.name == "LBM_ERR_OUT_OF_PAGES"
    assert core.dump() == before
    with pytest.raises(LbmError) as e:
        core.append(0)
    assert e.value.name == "LBM_ERR_INVALID_ARG"
    with pytest.raises(LbmError) as e:
        core.append(5)
    assert e.value.name == "LBM_ERR_INVALID_ARG"
    # special pool exhaustion
    cfg2 = make_config(num_blocks=1, num_heads=1, head_dim=64, patches_per_frame=4,
                       special_per_frame=8, special_page_size=4, scale_frames=1,
                       sliding_window=2, max_patch_pages=8, max_special_pages=2,
                       max_frames_per_step=4, max_q_tokens=16, dtype=0)
    c2 = CoreBookkeeping(cfg2)
    c2.append(1)
    with pytest.raises(LbmError) as e:
        c2.append(1)
    assert e.value.name == "LBM_ERR_OUT_OF_PAGES"
    # seeding after the first append is refused
    with pytest.raises(LbmError) as e:
        c2.seed_free_lists(list(range(8)), [0, 1])
    assert e.value.name == "LBM_ERR_BAD_STATE"


@pytest.mark.parametrize("bad", [
    dict(num_blocks=0), dict(num_heads=0), dict(patches_per_frame=0), dict(special_page_size=0),
    dict(max_frames_per_step=0), dict(max_frames_per_step=129), dict(dtype=7),
    dict(scale_frames=-1), dict(num_splits=-2), dict(max_q_tokens=0),
])
def test_core_rejects_bad_config(bad):
    f = dict(num_blocks=1, num_heads=2, head_dim=32, patches_per_frame=16, special_per_frame=6,
             special_page_size=16, scale_frames=2, sliding_window=4, max_patch_pages=7,
             max_special_pages=8, max_frames_per_step=3, max_q_tokens=66, dtype=1)
    f.update(bad)
    with pytest.raises(LbmError) as e:
        CoreBookkeeping(make_config(**f))
    assert e.value.name == "LBM_ERR_INVALID_ARG"


def test_choose_splits():
    cs = CoreBookkeeping.choose_splits
    # the 24-block ViT-L step: 6 query groups x 16 heads, ~1.55k tiles
    ns = cs(1375, 99006, 16, 256, 2, 16)
    assert 4 <= ns <= 12
    # the 8-frame first step fills the chip without splitting
    assert cs(11000, 11000, 16, 256, 3, 2) == 1
    # forced counts are honoured and capped; no empty split
    assert cs(1375, 99006, 16, 256, 3, 16, 4) == 4
    assert cs(1375, 99006, 16, 256, 3, 16, 99) == 16
    assert cs(22, 66, 2, 256, 3, 16, 8) == 2          # two tiles only
    assert cs(22, 66, 2, 256, 3, 16) >= 1
    assert cs(0, 66, 2, 256, 3, 16) < 0
    # measured on MI355X at the ViT-L steady state (kv_len 99,054): 8 splits is
    # the 16-bit kernel's best (256-row workgroups, two per CU), and the fp32
    # kernel (128-row workgroups, two per CU) runs best at 10-16 against 8;
    # the model, counting each kernel's own workgroups, picks 8 and 10
    assert cs(1375, 99054, 16, 256, 2, 16) == 8
    assert cs(1375, 99054, 16, 256, 2, 16, 0, 256) == 8
    assert cs(1375, 99054, 16, 256, 2, 16, 0, 128) == 10
    assert cs(1375, 99054, 16, 256, 2, 16, 0, -1) == 8   # non-positive: the 256-row default
    # the 16-bit kernel with 512-row workgroups, one per CU: 5 key ranges (one
    # dispatch round of 240 workgroups) measured best (5: 1005, 16: 989, 10:
    # 980, 4: 903, 8: 872, 6: 666 TFLOP/s), and the model picks 5 along the
    # stream's key lengths
    assert cs(1375, 99054, 16, 256, 1, 16, 0, 512) == 5
    assert cs(1375, 88054, 16, 256, 1, 16, 0, 512) == 5
    assert cs(1375, 158568, 16, 256, 1, 16, 0, 512) == 5
    # choosing the query groups too (the 16-bit kernel's launches): 4 groups
    # of 11/11/11/10 halves (busiest SIMD 3 halves instead of 4) x 4 key
    # ranges = 256 workgroups, every CU busy
    cl = CoreBookkeeping.choose_launch
    for kv in (88054, 99054, 158568):
        assert cl(1375, kv, 16, 256, 1, 16, 0, 512) == (4, 4)
    assert cl(1375, 99054, 16, 256, 1, 16, 6, 512) == (6, 3)   # forced splits: the fewest groups
    assert cl(1, 1584, 2, 256, 1, 16, 0, 512)[1] == 1           # one row: one group
    ns, g = cl(300, 1584, 2, 256, 1, 16, 0, 512)
    assert 1 <= g <= 2 and ns >= 1


@pytest.mark.parametrize("cid", [0, 2, 4])
def test_plan_before_evict_equals_plan_after(cid):
    """A step's visible table does not depend on whether the eviction that
    commits it has run yet: the graph launch builds the step's tables right
    after the reservation and evicts only once the launch is enqueued.  A
    one-frame reservation rolled back before that eviction (a failed launch)
    leaves the state exactly as before the step."""
    cfg = workloads.get_config(cid)
    core, _ = _pair(cfg)
    for s, nf in enumerate(workloads.step_schedule(cfg)):
        before = core.dump()
        core.append(nf)
        if nf == 1 and s % 3 == 0:
            core.rollback()
            assert core.dump() == before
            core.append(nf)
        planned = core.plan()
        core.evict()
        assert core.plan() == planned
