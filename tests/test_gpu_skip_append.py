"""Skip-append frames through the C ABI: a frame processed without storing
its K/V attends over the visible set and its own rows; the bookkeeping does
not move, and the frames after it see the cache as if it never came.  Checked
against the oracle on every skip frame and on the normal steps around them;
tolerances as in the parity tests."""
import pytest
import torch

import paged_kv_cache_312_amd as lbm
import workloads
from gpu_helpers import DEV, make_cache, run_stream, say
from test_gpu_parity import ODD_BF16, ODD_F16, ODD_F32, ODD_F32_D32

pytestmark = pytest.mark.gpu

# single-frame steps 2.. of the small streams (window 3, scale 2): skips before
# and after the window fills, two in a row, and the last step
SMALL_SKIPS = {2, 4, 5, 8, 12, 13}


@pytest.mark.parametrize("splits", [0, 3])
@pytest.mark.parametrize("cfg", [ODD_BF16, ODD_F16, ODD_F32, ODD_F32_D32], ids=lambda c: c.name)
def test_small_streams_with_skip_append(cfg, splits):
    w = run_stream(cfg, num_splits=splits, skip_steps=SMALL_SKIPS,
                   label=f"{cfg.name}/skip/splits={splits}")
    say(cfg.name, splits, w)


def test_vitl_single_block_skip_append():
    """ViT-L shape: skip frames while the window fills and once it is full."""
    cfg = workloads.get_config(1).replace(total_frames=84)
    skips = {30, 63, 64, 70}                     # F = 37, 69, 69, 74 at the skip (full at 72)
    checks = skips | {65, 71, 76}
    w = run_stream(cfg, check_steps=checks, rows_per_check=64, skip_steps=skips,
                   label="vitl_skip")
    say("C1 skip", w)


def test_skip_append_protocol():
    cfg = ODD_BF16.replace(name="odd_proto", total_frames=6)
    cache, _ = make_cache(cfg)
    T = cfg.tokens_per_frame
    q, k, v = workloads.gen_step_qkv(cfg, 0, 0, 1, DEV)
    with pytest.raises(lbm.LbmError) as e:          # nothing cached yet
        cache.plan_transient(T, T)
    assert e.value.name == "LBM_ERR_BAD_STATE"
    q3, k3, v3 = workloads.gen_step_qkv(cfg, 0, 0, 3, DEV)
    for b in range(cfg.num_blocks):
        cache.append_frame(b, k3, v3)
    cache.evict_frames()
    cache.plan(3 * T)
    with pytest.raises(lbm.LbmError) as e:          # normal plan
        cache.run_transient(0, q, k, v)
    assert e.value.name == "LBM_ERR_BAD_STATE"
    cache.plan_transient(T, T)
    with pytest.raises(lbm.LbmError) as e:          # skip-append plan
        cache.run(0, q)
    assert e.value.name == "LBM_ERR_BAD_STATE"
    with pytest.raises(ValueError):                 # own rows must match the plan
        cache.run_transient(0, q, k[:T - 1], v[:T - 1])
    for bad in (0, cfg.initial_frames * T + 1):
        with pytest.raises(lbm.LbmError) as e:
            cache.plan_transient(T, bad)
        assert e.value.name == "LBM_ERR_INVALID_ARG"
    # a step open with some blocks not appended
    cache.append_frame(0, k, v)
    with pytest.raises(lbm.LbmError) as e:
        cache.plan_transient(T, T)
    assert e.value.name == "LBM_ERR_BAD_STATE"
    torch.cuda.synchronize()
    cache.close()
