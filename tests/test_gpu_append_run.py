"""lbm_append_run: one block's append and attention of a frame step in one
call.  The attention is checked against the oracle (dense softmax over the
rule-derived visible set, the step's own rows included) on every output of
small streams and on sampled rows of the ViT-L-shaped single-block stream; the
bookkeeping against the reference allocator after every step; the pools by
reading every visible row back through the table, byte for byte against the
inputs (the rows each call's append wrote, which its attention then read
back through the plan's own positions); and the protocol errors, which leave
the cache as it was."""
import numpy as np
import pytest
import torch

import paged_kv_cache_312_amd as lbm
import workloads
from gpu_helpers import DEV, make_cache, run_stream, say
from test_gpu_api import SMALL_BF16, _gather_visible
from test_gpu_parity import ODD_BF16, ODD_F16, ODD_F32, ODD_F32_D32, ODD_NO_SCALE, ODD_NO_SPECIAL

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("splits", [0, 3])
@pytest.mark.parametrize("cfg", [ODD_BF16, ODD_F16, ODD_F32, ODD_F32_D32, ODD_NO_SCALE,
                                 ODD_NO_SPECIAL], ids=lambda c: c.name)
def test_small_streams_fused_every_output(cfg, splits):
    """Every step fused, every block and output checked (the first step's
    frames have no earlier key: all of its keys are the step's own rows)."""
    n = len(workloads.step_schedule(cfg))
    w = run_stream(cfg, num_splits=splits, fused_steps=range(n), label=f"fused {cfg.name}")
    say(f"{cfg.name} splits={splits}: worst max_abs {w['max_abs']:.3e}, splits {sorted(w['splits'])}")


def test_small_stream_fused_and_separate_steps_mixed():
    """Fused steps between steps made of lbm_append_frame + lbm_plan + lbm_run."""
    cfg = ODD_BF16
    n = len(workloads.step_schedule(cfg))
    run_stream(cfg, fused_steps=[s for s in range(n) if s % 3 != 1], label="mixed")


def test_vitl_single_block_fused():
    """The ViT-L shapes (1375 own rows, ~99k visible keys at the end), sampled."""
    cfg = workloads.get_config("vitl_single_block").replace(total_frames=90)
    n = len(workloads.step_schedule(cfg))
    run_stream(cfg, check_steps=[0, 1, 71, 72, n - 1], rows_per_check=96, heads=[0, 7, 15],
               fused_steps=range(n), label="vitl fused")


@pytest.mark.parametrize("cfg", [workloads.get_config(0), SMALL_BF16,
                                 SMALL_BF16.replace(name="small_f16", dtype="f16"),
                                 SMALL_BF16.replace(name="small_bf16_wide", patches_per_frame=300,
                                                    num_heads=4)],
                         ids=["tiny_f32", "small_bf16", "small_f16", "small_bf16_wide"])
def test_fused_append_gather_back_is_byte_exact(cfg):
    """After each fused step, the rows the table points at are the input rows,
    byte for byte, in visible order (scale, window, specials) (the wide
    case: own rows over several tiles and key ranges)."""
    from oracle import rules
    cache, _ = make_cache(cfg)
    T, P = cfg.tokens_per_frame, cfg.patches_per_frame
    frames = {}
    F = 0
    for s, nf in enumerate(workloads.step_schedule(cfg)):
        for b in range(cfg.num_blocks):
            q, k, v = workloads.gen_step_qkv(cfg, b, s, nf, DEV)
            cache.append_run(b, q, k, v)
            for i in range(nf):
                frames[(b, F + i)] = (k[i * T:(i + 1) * T], v[i * T:(i + 1) * T])
        F += nf
        torch.cuda.synchronize()
        for b in range(cfg.num_blocks):
            Kg, Vg = _gather_visible(cache, b)
            pf = rules.visible_patch_frames(F, cfg.scale_frames, cfg.sliding_window)
            Ke = torch.cat([frames[(b, f)][0][:P] for f in pf] +
                           [frames[(b, f)][0][P:] for f in range(F)])
            Ve = torch.cat([frames[(b, f)][1][:P] for f in pf] +
                           [frames[(b, f)][1][P:] for f in range(F)])
            iv = torch.int16 if Kg.dtype == torch.bfloat16 else torch.int32
            assert torch.equal(Kg.view(iv), Ke.view(iv)), f"step {s} block {b}: K"
            assert torch.equal(Vg.view(iv), Ve.view(iv)), f"step {s} block {b}: V"
    cache.close()


@pytest.mark.parametrize("nq", [1, 33, 300])
def test_fused_step_with_fewer_queries(nq):
    """lbm_append_run with fewer query rows than the step has own rows
    (wavefronts without rows take the load-only path).  Each output against
    the oracle's dense softmax over the visible set built from the input rows
    (own rows included), and the stored rows byte for byte."""
    from oracle import attention, rules
    cfg = SMALL_BF16.replace(name="small_bf16_wide", patches_per_frame=300, num_heads=4)
    cache, _ = make_cache(cfg)
    T, P = cfg.tokens_per_frame, cfg.patches_per_frame
    frames = {}
    F = 0
    worst = 0.0
    for s, nf in enumerate(workloads.step_schedule(cfg)):
        outs = []
        for b in range(cfg.num_blocks):
            q, k, v = workloads.gen_step_qkv(cfg, b, s, nf, DEV)
            qs = q[:nq].contiguous()
            outs.append((qs, cache.append_run(b, qs, k, v)))
            for i in range(nf):
                frames[(b, F + i)] = (k[i * T:(i + 1) * T], v[i * T:(i + 1) * T])
        F += nf
        torch.cuda.synchronize()
        pf = rules.visible_patch_frames(F, cfg.scale_frames, cfg.sliding_window)
        for b in range(cfg.num_blocks):
            Ke = torch.cat([frames[(b, f)][0][:P] for f in pf] +
                           [frames[(b, f)][0][P:] for f in range(F)])
            Ve = torch.cat([frames[(b, f)][1][:P] for f in pf] +
                           [frames[(b, f)][1][P:] for f in range(F)])
            qs, o = outs[b]
            ref = attention.dense_attention(qs.float().cpu().numpy(), Ke.float().cpu().numpy(),
                                            Ve.float().cpu().numpy())
            err = float(np.abs(o.float().cpu().numpy() - ref).max())
            worst = max(worst, err)
            assert err < 2e-2, f"step {s} block {b}: max abs {err:.3e}"
            Kg, Vg = _gather_visible(cache, b)
            assert torch.equal(Kg.view(torch.int16), Ke.view(torch.int16)), f"step {s} block {b}: K"
            assert torch.equal(Vg.view(torch.int16), Ve.view(torch.int16)), f"step {s} block {b}: V"
    say(f"fused, {nq} queries: worst max_abs {worst:.3e}")
    cache.close()


def test_fused_protocol_errors():
    cfg = SMALL_BF16
    cache, _ = make_cache(cfg)
    T = cfg.tokens_per_frame

    def code(fn, *a):
        with pytest.raises(lbm.LbmError) as e:
            fn(*a)
        return e.value.name

    q3, k3, v3 = workloads.gen_step_qkv(cfg, 0, 0, 3, DEV)
    # block 1 before block 0
    assert code(cache.append_run, 1, q3, k3, v3) == "LBM_ERR_BAD_STATE"
    # more frames than the window holds
    q4, k4, v4 = workloads.gen_step_qkv(cfg, 0, 0, 4, DEV)
    assert code(cache.append_run, 0, q4, k4, v4) == "LBM_ERR_INVALID_ARG"
    assert cache.stats()["frame_count"] == 0
    # a step opened by lbm_append_frame is not continued by lbm_append_run
    cache.append_frame(0, k3, v3)
    assert code(cache.append_run, 1, q3, k3, v3) == "LBM_ERR_BAD_STATE"
    cache.append_frame(1, k3, v3)
    cache.evict_frames()
    # a fused step: every block once; lbm_run refuses its plan
    q1, k1, v1 = workloads.gen_step_qkv(cfg, 0, 1, 1, DEV)
    cache.append_run(0, q1, k1, v1)
    assert code(cache.append_run, 0, q1, k1, v1) == "LBM_ERR_BAD_STATE"  # block 1 missing
    assert code(cache.run, 0, q1) == "LBM_ERR_BAD_STATE"
    assert code(cache.append_run, 1, q1[:T - 1], k1, v1) == "LBM_ERR_BAD_STATE"  # other q count
    cache.append_run(1, q1, k1, v1)
    assert code(cache.append_run, 1, q1, k1, v1) == "LBM_ERR_BAD_STATE"  # twice
    assert cache.stats()["frame_count"] == 4
    cache.close()


def test_fused_call_refused_without_a_window():
    """No window: a one-frame step cannot keep its frame visible, so the
    fused call is refused before anything changes."""
    cfg = ODD_BF16.replace(name="odd_no_window_f", cid=19, sliding_window=0)
    cache, _ = make_cache(cfg)
    q, k, v = workloads.gen_step_qkv(cfg, 0, 0, 1, DEV)
    before = cache.dump_state()
    with pytest.raises(lbm.LbmError) as e:
        cache.append_run(0, q, k, v)
    assert e.value.name == "LBM_ERR_INVALID_ARG"
    assert cache.dump_state() == before
    cache.close()
