"""Attention parity with the CPU oracle through the C ABI.

Small streams are checked on every step and every output; the ViT-L-shaped
workloads run their whole schedules (bookkeeping checked bit-exact) and are
checked on sampled steps, blocks and query rows -- the rows always include the
first and the last (ragged tail) one.  Tolerances: bf16 max-abs 2e-2 and
rel-L2 1e-2; fp16 max-abs 2.5e-3 and rel-L2 1.25e-3; fp32 max-abs 1e-5 and
rel-L2 1e-5.
"""
import pytest

import workloads
from gpu_helpers import run_stream, say

pytestmark = pytest.mark.gpu

ODD_BF16 = workloads.StreamConfig(
    "odd_bf16", 12, num_blocks=2, num_heads=3, head_dim=64, patches_per_frame=100,
    special_per_frame=6, special_page_size=16, scale_frames=2, sliding_window=3,
    total_frames=16, initial_frames=3, dtype="bf16")
ODD_F32 = ODD_BF16.replace(name="odd_f32", cid=13, dtype="f32")
ODD_F32_D32 = ODD_BF16.replace(name="odd_f32_d32", cid=14, dtype="f32", head_dim=32,
                               patches_per_frame=37, special_per_frame=3, special_page_size=8)
ODD_F16 = ODD_BF16.replace(name="odd_f16", cid=15, dtype="f16")
# include_scale_frames=False of the pages' eviction call: no frame is kept
# beyond the window (scale_frames = 0)
ODD_NO_SCALE = ODD_BF16.replace(name="odd_no_scale", cid=16, scale_frames=0)
# degenerate settings: no special tokens (an empty special stream), no window
# (each frame's patches leave at its own step's eviction)
ODD_NO_SPECIAL = ODD_BF16.replace(name="odd_no_special", cid=17, special_per_frame=0)
ODD_NO_WINDOW = ODD_BF16.replace(name="odd_no_window", cid=18, sliding_window=0)


def test_tiny_config_every_output():
    w = run_stream(workloads.get_config(0), label="tiny")
    say("tiny", w)


@pytest.mark.parametrize("splits", [0, 1, 3])
@pytest.mark.parametrize("cfg", [ODD_BF16, ODD_F16, ODD_F32, ODD_F32_D32, ODD_NO_SCALE,
                                 ODD_NO_SPECIAL, ODD_NO_WINDOW],
                         ids=lambda c: c.name)
def test_small_streams_every_output(cfg, splits):
    w = run_stream(cfg, num_splits=splits, label=f"{cfg.name}/splits={splits}")
    say(cfg.name, splits, w)


def test_small_stream_deferred_rollback():
    cfg = ODD_BF16.replace(name="odd_bf16_rb", reject_prob=0.4, total_frames=20)
    acc = workloads.accept_draws(cfg)
    assert not all(acc)
    w = run_stream(cfg, deferred=True, accept=acc, label="odd_bf16_rb")
    say("rollback", w)


def test_vitl_single_block_stream():
    """208 frames, bf16; outputs checked around the window filling up and at the end."""
    cfg = workloads.get_config(1)
    checks = {0, 1, 63, 64, 65, 120, 200}          # F = 8, 9, 71, 72, 73, 128, 208
    w = run_stream(cfg, check_steps=checks, rows_per_check=96, label="vitl_single_block")
    say("C1", w)


def test_vitl_single_block_f16_stream():
    """The fp16 kernel on the ViT-L shape: window filling and full."""
    cfg = workloads.get_config(1).replace(dtype="f16", total_frames=90)
    w = run_stream(cfg, check_steps={0, 63, 64, 81}, rows_per_check=96, label="vitl_f16")
    say("C1 f16", w)


def test_vitl_single_block_no_scale_frames():
    """include_scale_frames=False (scale_frames = 0) at the ViT-L shape."""
    cfg = workloads.get_config(1).replace(scale_frames=0, total_frames=80)
    w = run_stream(cfg, check_steps={0, 56, 71}, rows_per_check=64, label="vitl_no_scale")
    say("C1 no scale", w)


def test_vitl_single_block_peaky_queries():
    """q scaled x4: outputs of order 0.1-1, where a missing page shows."""
    cfg = workloads.get_config(1).replace(total_frames=80)
    w = run_stream(cfg, check_steps={71}, rows_per_check=64, q_scale=4.0, label="peaky")
    say("peaky", w)


def test_vitl_24_block_frame_step_stream():
    """1000 frames x 24 blocks: every step appended, evicted and planned;
    attention of all 24 blocks checked at F = 8, 9, 72, 73, 500, 1000."""
    cfg = workloads.get_config(2)
    checks = {0, 1, 64, 65, 492, 992}
    w = run_stream(cfg, check_steps=checks, rows_per_check=24, heads=range(0, 16, 3),
                   dump_every=50, label="vitl_24_block")
    say("C2", w)


def test_vitl_long_stream():
    """10,000 frames x 4 blocks: 60,000 specials in 3,750 pages, ~9,900
    evictions; attention checked at F = 8, 73, 2500, 10000."""
    cfg = workloads.get_config(3)
    checks = {0, 65, 2492, 9992}
    w = run_stream(cfg, check_steps=checks, rows_per_check=16, heads=(0, 7, 15),
                   dump_every=500, label="vitl_long")
    say("C3", w)


def test_vitl_rollback_f32_stream():
    """500 offered frames, fp32, each single frame rejected with p = 0.3 and
    rolled back under deferred eviction; state equals the pre-append snapshot
    after every rollback."""
    cfg = workloads.get_config(4)
    acc = workloads.accept_draws(cfg)
    rejected = [s for s, a in enumerate(acc) if not a]
    checks = set(range(0, 500, 50)) | set(rejected[:3]) | {1, 2, 499}
    w = run_stream(cfg, check_steps=checks, rows_per_check=16, heads=(0, 9),
                   deferred=True, accept=acc, label="vitl_rollback_f32")
    say("C4", w)
