"""Pins of the CPU oracle against things other than itself.

Each test names what fixes the expected value: a record printed on the pages,
a closed form, a library routine, a brute-force enumeration, a hand
derivation, or an invariant.  The ``planted`` tests plant a plausible mistake
in the oracle (on the CPU) and check that a pin catches it.
"""
import json
import math
import os
import random

import numpy as np
import pytest

import oracle
from oracle import brute, rules
from oracle.allocator import AllocatorError, RefAllocator
from oracle.attention import dense_attention, dense_attention_rows
from oracle.stream import StreamOracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _alloc(cfg, **kw):
    return RefAllocator(cfg.patches_per_frame, cfg.special_per_frame, cfg.special_page_size,
                        cfg.scale_frames, cfg.sliding_window, cfg.max_patch_pages,
                        cfg.max_special_pages(), **kw)


# ---------------------------------------------------------------------------
# visible-set rules
# ---------------------------------------------------------------------------

def test_stats_worked_example_from_pages():
    """The get_cache_stats record printed on the pages, reproduced for several
    append schedules that reach 42 frames."""
    with open(os.path.join(GOLDEN, "stats_example.json")) as fh:
        g = json.load(fh)
    c = g["config"]
    for first in (1, 5, 8, 42):
        a = RefAllocator(c["patches_per_frame"], c["special_per_frame"], 16, c["scale_frames"],
                         c["sliding_window"], c["max_patch_pages"], 64)
        n = 0
        sched = [first] + [1] * (g["frames"] - first)
        for nf in sched:
            a.append(nf)
            a.evict()
            n += nf
        assert n == g["frames"]
        assert a.stats() == g["expected"]


def test_steady_page_count_about_72():
    """About 72 patch pages at steady state for scale 8 / window 64 (the pages'
    step-by-step description), from the closed form and from the allocator."""
    assert rules.steady_patch_pages(8, 64) == 72
    for F in (72, 73, 100, 1000, 10000):
        assert rules.visible_counts(F, 8, 64, 1369, 6)[0] == 72
    cfg = workloads.get_config(1)
    a = _alloc(cfg)
    for nf in workloads.step_schedule(cfg):
        a.append(nf)
        a.evict()
    assert len(a.visible_patch_pages()) == 72


def test_vitl_visible_patch_tokens():
    """The single-block ViT-L workload's ~98.6k visible patch tokens:
    72 pages x 1369 = 98,568, and kv_len = 98,568 + 6F from F = 72 on."""
    for F in (72, 73, 208, 1000, 10000):
        n_patch, n_spec, total = rules.visible_counts(F, 8, 64, 1369, 6)
        assert n_patch * 1369 == 98568
        assert round(n_patch * 1369 / 1000, 1) == 98.6
        assert total == 98568 + 6 * F
    assert rules.visible_counts(8, 8, 64, 1369, 6)[2] == 11000


def test_visible_frames_small_cases():
    """Hand-enumerated cases of the rules (scale 2, window 4)."""
    assert rules.visible_patch_frames(0, 2, 4) == []
    assert rules.visible_patch_frames(1, 2, 4) == [0]
    assert rules.visible_patch_frames(2, 2, 4) == [0, 1]
    assert rules.visible_patch_frames(6, 2, 4) == [0, 1, 2, 3, 4, 5]
    assert rules.visible_patch_frames(7, 2, 4) == [0, 1, 3, 4, 5, 6]
    assert rules.visible_patch_frames(12, 2, 4) == [0, 1, 8, 9, 10, 11]
    assert rules.visible_patch_frames(5, 0, 2) == [3, 4]
    assert rules.visible_patch_frames(5, 8, 64) == [0, 1, 2, 3, 4]
    assert rules.visible_patch_frames(5, 2, 0) == [0, 1]
    assert rules.visible_special_frames(3) == [0, 1, 2]


def _rule_slots(F, P, S, scale, window):
    s = set()
    for f in rules.visible_patch_frames(F, scale, window):
        s |= {(f, t) for t in range(P)}
    for f in rules.visible_special_frames(F):
        s |= {(f, t) for t in range(P, P + S)}
    return s


def _check_rules_against_brute(seed):
    rng = random.Random(seed)
    P = rng.randint(1, 5)
    S = rng.randint(0, 3)
    scale = rng.randint(0, 4)
    window = rng.randint(0, 5)
    sched = [rng.randint(1, 4)] + [rng.choice([1, 1, 1, 2]) for _ in range(rng.randint(0, 15))]
    sim = brute.simulate_visible_slots(sched, P, S, scale, window)
    F = 0
    for nf, slots in zip(sched, sim):
        F += nf
        assert _rule_slots(F, P, S, scale, window) == slots, (seed, F)
        n_patch, n_spec, total = rules.visible_counts(F, scale, window, P, S)
        assert total == len(slots)


@pytest.mark.parametrize("seed", range(60))
def test_rules_vs_brute_force_event_simulation(seed):
    _check_rules_against_brute(seed)


def test_rules_vs_brute_force_tiny_config():
    cfg = workloads.get_config(0)
    sched = workloads.step_schedule(cfg)
    sim = brute.simulate_visible_slots(sched, cfg.patches_per_frame, cfg.special_per_frame,
                                       cfg.scale_frames, cfg.sliding_window)
    F = 0
    for nf, slots in zip(sched, sim):
        F += nf
        assert _rule_slots(F, cfg.patches_per_frame, cfg.special_per_frame, cfg.scale_frames,
                           cfg.sliding_window) == slots


# ---------------------------------------------------------------------------
# reference allocator
# ---------------------------------------------------------------------------

# Hand derivation for the tiny workload (P 16, S 6, special page 16, scale 2,
# window 4, 7 patch pages; step 0 appends frames 0-2, then one frame per step)
# under the allocator's stated conventions: ascending free lists, pop head,
# evicted pages to the tail, lazy special pages.
TINY_TRACE = [
    # F, visible patch ids, patch free list, evicted, special pages, last_page_len, kv_len
    (3, [0, 1, 2], [3, 4, 5, 6], [], 2, 2, 66),
    (4, [0, 1, 2, 3], [4, 5, 6], [], 2, 8, 88),
    (5, [0, 1, 2, 3, 4], [5, 6], [], 2, 14, 110),
    (6, [0, 1, 2, 3, 4, 5], [6], [], 3, 4, 132),
    (7, [0, 1, 3, 4, 5, 6], [2], [2], 3, 10, 138),
    (8, [0, 1, 4, 5, 6, 2], [3], [3], 3, 16, 144),
    (9, [0, 1, 5, 6, 2, 3], [4], [4], 4, 6, 150),
    (10, [0, 1, 6, 2, 3, 4], [5], [5], 4, 12, 156),
    (11, [0, 1, 2, 3, 4, 5], [6], [6], 5, 2, 162),
    (12, [0, 1, 3, 4, 5, 6], [2], [2], 5, 8, 168),
]


def test_allocator_tiny_trace_hand_derived():
    cfg = workloads.get_config(0)
    a = _alloc(cfg)
    F = 0
    for nf, row in zip(workloads.step_schedule(cfg), TINY_TRACE):
        a.append(nf)
        ev = a.evict()
        F += nf
        exp_F, vis, free, evicted, n_sp, lpl, kv = row
        assert F == exp_F
        assert a.visible_patch_pages() == vis
        assert list(a.patch_free) == free
        assert ev == evicted
        assert len(a.all_special) == n_sp and a.all_special == list(range(n_sp))
        assert a.last_page_len() == lpl
        assert a.kv_len() == kv
        a.check_invariants(after_evict=True)


@pytest.mark.parametrize("cid", [0, 1, 2, 3])
def test_allocator_matches_rules_full_schedules(cid):
    """Visible pages hold exactly the rule-derived frames, in order, after every
    step of the whole schedule (10,000 frames for the long stream)."""
    cfg = workloads.get_config(cid)
    a = _alloc(cfg)
    F = 0
    for nf in workloads.step_schedule(cfg):
        a.append(nf)
        a.evict()
        F += nf
        frames = [a.page_frame[p] for p in a.visible_patch_pages()]
        assert frames == rules.visible_patch_frames(F, cfg.scale_frames, cfg.sliding_window)
        assert a.special_tokens == F * cfg.special_per_frame
        assert a.kv_len() == rules.visible_counts(F, cfg.scale_frames, cfg.sliding_window,
                                                  cfg.patches_per_frame, cfg.special_per_frame)[2]
        if F % 97 == 0 or F < 80:
            a.check_invariants(after_evict=True)
    if cid == 3:
        # 60,000 specials in 3,750 full pages: the last page is full here
        assert a.special_tokens == 60000 and len(a.all_special) == 3750
        assert a.last_page_len() == 16


def test_allocator_rollback_restores_exact_state():
    """Deferred flow with Bernoulli rejects: after every rollback the state
    record equals the record taken before that append, byte for byte."""
    cfg = workloads.get_config(4)
    a = _alloc(cfg)
    sched = workloads.step_schedule(cfg)
    acc = workloads.accept_draws(cfg)
    n_rb = 0
    for nf, ok in zip(sched, acc):
        before = a.dump()
        a.append(nf)
        a.check_invariants(after_evict=False)
        # the visible window stays the latest `window` pages while provisional
        assert len(a.visible_patch_pages()) <= cfg.scale_frames + cfg.sliding_window
        if ok:
            a.evict()
            a.check_invariants(after_evict=True)
        else:
            a.rollback()
            assert a.dump() == before
            n_rb += 1
    assert n_rb > 100


def test_allocator_errors():
    a = RefAllocator(4, 2, 4, 1, 2, 4, 8)
    with pytest.raises(AllocatorError) as e:
        a.rollback()
    assert e.value.kind == "bad_state"
    a.append(3)
    with pytest.raises(AllocatorError) as e:
        a.rollback()                       # multi-frame step
    assert e.value.kind == "bad_state"
    a.evict()
    a.append(1)
    a.evict()
    with pytest.raises(AllocatorError):
        a.rollback()                       # after the commit
    before = a.dump()
    with pytest.raises(AllocatorError) as e:
        a.append(3)                        # 1 free page left
    assert e.value.kind == "out_of_pages"
    assert a.dump() == before
    b = RefAllocator(4, 8, 4, 1, 2, 4, 2)
    b.append(1)
    with pytest.raises(AllocatorError) as e:
        b.append(1)                        # special pages exhausted
    assert e.value.kind == "out_of_pages"


def test_allocator_permuted_free_lists():
    """With permuted initial free lists the visible frames are unchanged."""
    cfg = workloads.get_config(0)
    rng = random.Random(3)
    po = list(range(cfg.max_patch_pages)); rng.shuffle(po)
    so = list(range(cfg.max_special_pages())); rng.shuffle(so)
    a = _alloc(cfg, patch_order=po, special_order=so)
    F = 0
    for nf in workloads.step_schedule(cfg):
        a.append(nf)
        a.evict()
        F += nf
        assert [a.page_frame[p] for p in a.visible_patch_pages()] == \
            rules.visible_patch_frames(F, cfg.scale_frames, cfg.sliding_window)
        assert a.all_special == so[:len(a.all_special)]


# ---------------------------------------------------------------------------
# dense attention
# ---------------------------------------------------------------------------

def test_attention_two_keys_hand_values():
    """D = 4, scores 2/sqrt(4) = 1 and 0: weights e/(e+1) and 1/(e+1)."""
    q = np.array([[1.0, 0, 0, 0]])
    k = np.array([[2.0, 0, 0, 0], [0.0, 0, 0, 0]])
    v = np.array([[1.0, 0, 0, 0], [0.0, 1, 0, 0]])
    out = dense_attention_rows(q, k, v)
    np.testing.assert_allclose(out[0], [0.7310585786300049, 0.2689414213699951, 0, 0],
                               rtol=0, atol=1e-15)


def test_attention_closed_forms():
    rng = np.random.default_rng(0)
    D = 64
    # a single visible token: out = v
    q = rng.standard_normal((5, 3, D)); k = rng.standard_normal((1, 3, D))
    v = rng.standard_normal((1, 3, D))
    np.testing.assert_allclose(dense_attention(q, k, v), np.broadcast_to(v, (5, 3, D)), atol=1e-14)
    # q = 0: the mean of the visible values
    k = rng.standard_normal((37, 2, D)); v = rng.standard_normal((37, 2, D))
    out = dense_attention(np.zeros((4, 2, D)), k, v)
    np.testing.assert_allclose(out, np.broadcast_to(v.mean(0), (4, 2, D)), atol=1e-14)
    # all keys equal: the mean of the visible values
    q = rng.standard_normal((4, 2, D))
    kk = np.broadcast_to(rng.standard_normal((1, 2, D)), (37, 2, D))
    np.testing.assert_allclose(dense_attention(q, kk, v), np.broadcast_to(v.mean(0), (4, 2, D)),
                               atol=1e-13)
    # large logits stay finite (max subtraction)
    out = dense_attention(q * 1e3, k, v)
    assert np.isfinite(out).all()


def test_attention_permutation_invariant():
    rng = np.random.default_rng(1)
    q = rng.standard_normal((9, 2, 32)); k = rng.standard_normal((200, 2, 32))
    v = rng.standard_normal((200, 2, 32))
    perm = rng.permutation(200)
    a = dense_attention(q, k, v)
    b = dense_attention(q, k[perm], v[perm])
    assert np.abs(a - b).max() <= 1e-13


def test_attention_vs_torch_sdpa_fp64():
    """Library cross-check: torch's scaled_dot_product_attention on the CPU in
    float64 (default scale 1/sqrt(D))."""
    import torch
    rng = np.random.default_rng(2)
    q = rng.standard_normal((70, 3, 64)); k = rng.standard_normal((513, 3, 64))
    v = rng.standard_normal((513, 3, 64))
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q).permute(1, 0, 2), torch.from_numpy(k).permute(1, 0, 2),
        torch.from_numpy(v).permute(1, 0, 2)).permute(1, 0, 2).numpy()
    out = dense_attention(q, k, v, row_chunk=16)
    assert np.abs(out - ref).max() <= 1e-12


def test_attention_vs_scalar_brute():
    rng = np.random.default_rng(3)
    q = rng.standard_normal((3, 1, 8)); k = rng.standard_normal((11, 1, 8))
    v = rng.standard_normal((11, 1, 8))
    out = dense_attention(q, k, v)
    for i in range(3):
        ref = brute.scalar_attention(q[i, 0], list(k[:, 0]), list(v[:, 0]))
        assert np.abs(out[i, 0] - np.array(ref)).max() <= 1e-13


# ---------------------------------------------------------------------------
# whole stream
# ---------------------------------------------------------------------------

def _tiny_stream_vs_brute(cfg, steps_to_check=None, accept=None):
    """Run the oracle over a tiny stream; compare every output of the checked
    steps with scalar attention over the brute-force visible slots."""
    import torch  # noqa: F401  (generators)
    P, S = cfg.patches_per_frame, cfg.special_per_frame
    T = P + S
    orc = StreamOracle(P, S, cfg.scale_frames, cfg.sliding_window)
    sched = workloads.step_schedule(cfg)
    accept = accept or [True] * len(sched)
    frames_kv = {}          # logical frame -> (k, v) for the brute force
    acc_sched = []
    worst = 0.0
    for s, nf in enumerate(sched):
        q, k, v = [t.double().numpy() for t in workloads.gen_step_qkv(cfg, 0, s, nf)]
        out = orc.step_outputs(0, q, k, v)
        if steps_to_check is None or s in steps_to_check:
            sim = brute.simulate_visible_slots(acc_sched + [nf], P, S, cfg.scale_frames,
                                               cfg.sliding_window)[-1]
            pend = dict(frames_kv)
            for i in range(nf):
                pend[orc.F + i] = (k[i * T:(i + 1) * T], v[i * T:(i + 1) * T])
            slots = sorted(sim)
            for h in range(cfg.num_heads):
                keys = [pend[f][0][t, h] for f, t in slots]
                vals = [pend[f][1][t, h] for f, t in slots]
                for i in range(q.shape[0]):
                    ref = brute.scalar_attention(q[i, h], keys, vals)
                    worst = max(worst, float(np.abs(out[i, h] - np.array(ref)).max()))
        if accept[s]:
            for i in range(nf):
                frames_kv[orc.F + i] = (k[i * T:(i + 1) * T], v[i * T:(i + 1) * T])
            orc.commit({0: (k, v)}, nf)
            acc_sched.append(nf)
    return worst


def test_stream_oracle_tiny_config_vs_brute_every_output():
    cfg = workloads.get_config(0)
    worst = _tiny_stream_vs_brute(cfg)
    assert worst <= 1e-12


def test_stream_oracle_tiny_with_rejects_vs_brute():
    cfg = workloads.get_config(0).replace(total_frames=14, reject_prob=0.4)
    acc = workloads.accept_draws(cfg)
    assert not all(acc)
    worst = _tiny_stream_vs_brute(cfg, accept=acc)
    assert worst <= 1e-12


# Degenerate settings of the method: no special tokens (the special stream
# stays empty), no window (only the scale frames' patches and the specials
# stay visible; each later frame's patches leave at its own step's eviction),
# and a one-frame window without scale frames.
DEGENERATE = {
    "no_special": dict(special_per_frame=0),
    "no_window": dict(sliding_window=0),
    "window1_no_scale": dict(scale_frames=0, sliding_window=1, initial_frames=1),
}


@pytest.mark.parametrize("name", sorted(DEGENERATE))
def test_stream_oracle_degenerate_configs_vs_brute(name):
    cfg = workloads.get_config(0).replace(name=f"tiny_{name}", total_frames=14, reject_prob=0.3,
                                          **DEGENERATE[name])
    acc = workloads.accept_draws(cfg)
    worst = _tiny_stream_vs_brute(cfg, accept=acc)
    assert worst <= 1e-12


def _tiny_oracle_after(cfg, n_steps):
    """Stream oracle of block 0 after the first n_steps steps of cfg."""
    orc = StreamOracle(cfg.patches_per_frame, cfg.special_per_frame, cfg.scale_frames,
                       cfg.sliding_window)
    for s, nf in enumerate(workloads.step_schedule(cfg)[:n_steps]):
        q, k, v = [t.double().numpy() for t in workloads.gen_step_qkv(cfg, 0, s, nf)]
        orc.commit({0: (k, v)}, nf)
    return orc


def test_skip_append_equals_append_before_the_window_fills():
    """While nothing is evicted, attending over the cache plus the frame's own
    rows is attention over the same key multiset as appending the frame (in
    another order), so both oracle paths must agree."""
    cfg = workloads.get_config(0)               # scale 2, window 4: 6 frames before eviction
    for n_steps in (1, 2):                      # F = 3, 4 accepted frames
        orc = _tiny_oracle_after(cfg, n_steps)
        assert orc.F + 1 <= cfg.scale_frames + cfg.sliding_window
        q, k, v = [t.double().numpy() for t in workloads.gen_step_qkv(cfg, 0, 50 + n_steps, 1)]
        skip = orc.skip_append_outputs(0, q, k, v)
        app = orc.step_outputs(0, q, k, v)
        assert np.abs(skip - app).max() <= 1e-12
        assert orc.F == 3 + (n_steps - 1)       # unchanged by either call


def test_skip_append_vs_brute_with_full_window():
    """Window full: the frame sees the brute-force visible slots of F frames
    (the oldest window frame still there, no eviction) plus its own tokens."""
    cfg = workloads.get_config(0)
    P, S, T = cfg.patches_per_frame, cfg.special_per_frame, cfg.tokens_per_frame
    sched = workloads.step_schedule(cfg)[:6]
    orc = _tiny_oracle_after(cfg, len(sched))
    assert orc.F == 8 and orc.F > cfg.scale_frames + cfg.sliding_window
    slots = brute.simulate_visible_slots(sched, P, S, cfg.scale_frames, cfg.sliding_window)[-1]
    q, k, v = [t.double().numpy() for t in workloads.gen_step_qkv(cfg, 0, 77, 1)]
    got = orc.skip_append_outputs(0, q, k, v, rows=np.array([0, T - 1]), heads=[1])
    for out_row, r in zip(got, (0, T - 1)):
        keys, vals = [], []
        for (f, t) in sorted(slots):
            kk, vv = orc.history.get(0, f)
            keys.append(kk[t, 1]); vals.append(vv[t, 1])
        for t in range(T):
            keys.append(k[t, 1]); vals.append(v[t, 1])
        ref = brute.scalar_attention(q[r, 1], keys, vals)
        assert np.abs(out_row[0] - np.array(ref)).max() <= 1e-12


def test_paged_equals_dense_over_mirror_pools():
    """Mirror host pools filled through the reference allocator's write map:
    walking them through its visible table reproduces the rule-derived rows
    exactly, and attention over them equals the stream oracle."""
    cfg = workloads.get_config(0).replace(total_frames=16)
    P, S, H, D = cfg.patches_per_frame, cfg.special_per_frame, cfg.num_heads, cfg.head_dim
    T = P + S
    a = _alloc(cfg)
    ppool = np.zeros((cfg.max_patch_pages, 2, P, H, D))
    spool = np.zeros((cfg.max_special_pages(), 2, cfg.special_page_size, H, D))
    orc = StreamOracle(P, S, cfg.scale_frames, cfg.sliding_window)
    for s, nf in enumerate(workloads.step_schedule(cfg)):
        q, k, v = [t.double().numpy() for t in workloads.gen_step_qkv(cfg, 0, s, nf)]
        wm = a.append(nf)
        a.evict()
        for i in range(nf):
            pg = wm["patch_pages"][i]
            ppool[pg, 0] = k[i * T:i * T + P]
            ppool[pg, 1] = v[i * T:i * T + P]
            for j, (sp, slot) in enumerate(wm["special_slots"][i]):
                spool[sp, 0, slot] = k[i * T + P + j]
                spool[sp, 1, slot] = v[i * T + P + j]
        plan = a.plan()
        kv_len, n_pp, n_sp, n_st, lpl = plan[:5]
        pids = plan[5:5 + n_pp]
        sids = plan[5 + n_pp:5 + n_pp + n_sp]
        Kp = [ppool[p, 0] for p in pids] + [spool[p, 0] for p in sids]
        Vp = [ppool[p, 1] for p in pids] + [spool[p, 1] for p in sids]
        Kp = np.concatenate(Kp)[:kv_len]
        Vp = np.concatenate(Vp)[:kv_len]
        assert kv_len == n_pp * P + (n_sp - 1) * cfg.special_page_size + lpl
        pend = {orc.F + i: (k[i * T:(i + 1) * T], v[i * T:(i + 1) * T]) for i in range(nf)}
        Kd, Vd = orc.visible_kv(0, orc.F + nf, pending=pend)
        assert np.array_equal(Kp, Kd) and np.array_equal(Vp, Vd)
        out_paged = dense_attention(q, Kp, Vp)
        out_orc = orc.step_outputs(0, q, k, v)
        assert np.abs(out_paged - out_orc).max() <= 1e-12
        orc.commit({0: (k, v)}, nf)


# ---------------------------------------------------------------------------
# planted mistakes: each must be caught by one of the pins above
# ---------------------------------------------------------------------------

def test_planted_window_off_by_one_is_caught(monkeypatch):
    good = rules.visible_patch_frames

    def bad(F, scale, window):
        return good(F, scale, window + 1)
    monkeypatch.setattr(rules, "visible_patch_frames", bad)
    caught = 0
    for seed in range(60):
        try:
            _check_rules_against_brute(seed)
        except AssertionError:
            caught += 1
    assert caught > 0


def test_planted_scale_frames_as_latest_is_caught(monkeypatch):
    """Reading 'scale frames' as the most recent frames must fail the pins."""
    def bad(F, scale, window):
        lo = max(0, F - window - scale)
        return list(range(lo, F))
    monkeypatch.setattr(rules, "visible_patch_frames", bad)
    with pytest.raises(AssertionError):
        test_visible_frames_small_cases()


def test_planted_softmax_scale_is_caught(monkeypatch):
    import oracle.attention as att
    good = att.dense_attention_rows

    def bad(q, k, v, scale=None):
        return good(q, k, v, 1.0 / q.shape[-1])
    monkeypatch.setattr(att, "dense_attention_rows", bad)
    with pytest.raises(AssertionError):
        q = np.array([[1.0, 0, 0, 0]])
        k = np.array([[2.0, 0, 0, 0], [0.0, 0, 0, 0]])
        v = np.array([[1.0, 0, 0, 0], [0.0, 1, 0, 0]])
        np.testing.assert_allclose(att.dense_attention_rows(q, k, v)[0],
                                   [0.7310585786300049, 0.2689414213699951, 0, 0], atol=1e-15)


def test_planted_dropped_special_is_caught(monkeypatch):
    """A visible set that forgets the current frame's specials fails the
    brute-force comparison of the whole tiny stream."""
    good = rules.visible_special_frames
    monkeypatch.setattr(rules, "visible_special_frames", lambda F: good(max(F - 1, 0)))
    cfg = workloads.get_config(0)
    assert _tiny_stream_vs_brute(cfg, steps_to_check={0, 5}) > 1e-6


def test_planted_rollback_to_tail_is_caught(monkeypatch):
    """Returning a rolled-back page to the tail of the free list breaks the
    exact-restore pin."""
    def bad_rollback(self):
        u = self._undo
        page = u["patch"][0]
        (self.scale if u["to_scale"][0] else self.live).pop()
        del self.page_frame[page]
        self.patch_free.append(page)
        for sp in reversed(u["special"]):
            self.all_special.pop()
            self.special_free.appendleft(sp)
        self.special_tokens = u["special_tokens"]
        self.frame_count = u["frame_count"]
        self._undo = None
    monkeypatch.setattr(RefAllocator, "rollback", bad_rollback)
    with pytest.raises(AssertionError):
        test_allocator_rollback_restores_exact_state()
