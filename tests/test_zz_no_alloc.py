"""The allocation-free stateless attention (lbm_paged_attention_static) against
the workspace entry point (lbm_paged_attention) through the C ABI: two calls
in a row on one GPU, the second with a smaller input, each checked to the
stated bf16 tolerance against the workspace call and, with the split count
forced equal, bit for bit; the oracle checks the first call's output too."""
import numpy as np
import pytest
import torch

import paged_kv_cache_312_amd as lbm
from gpu_helpers import BF16_MAX_ABS, BF16_REL_L2, DEV, say
from oracle.attention import dense_attention

pytestmark = pytest.mark.gpu

H, D, P, SPS = 16, 64, 1369, 16


def _cfg(num_splits=0):
    return lbm.make_config(num_blocks=1, num_heads=H, head_dim=D, patches_per_frame=P,
                           special_per_frame=6, special_page_size=SPS, scale_frames=8,
                           sliding_window=64, max_patch_pages=73, max_special_pages=64,
                           max_frames_per_step=8, max_q_tokens=2048, dtype=lbm.LBM_BF16,
                           num_splits=num_splits)


def _inputs(seed, n_pp, n_st, nq):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    pp = torch.randn((73, 2, P, H, D), generator=g, device=DEV).to(torch.bfloat16)
    sp = torch.randn((64, 2, SPS, H, D), generator=g, device=DEV).to(torch.bfloat16)
    q = torch.randn((nq, H, D), generator=g, device=DEV).to(torch.bfloat16)
    pids = torch.randperm(73, generator=g, device=DEV)[:n_pp].to(torch.int32)
    n_sp = (n_st + SPS - 1) // SPS
    sids = torch.randperm(64, generator=g, device=DEV)[:max(n_sp, 1)].to(torch.int32)
    return pp, sp, q, pids, sids


def _call(fn, cfg, pp, sp, q, pids, n_pp, sids, n_st, ws=None):
    out = torch.full_like(q, float("nan"))
    st = torch.cuda.current_stream().cuda_stream
    args = [cfg, q.data_ptr(), out.data_ptr(), q.shape[0], pp.data_ptr(), sp.data_ptr(),
            pids.data_ptr(), n_pp, sids.data_ptr(), n_st]
    if ws is not None:
        args.append(ws.data_ptr())
    fn(*args, st)
    torch.cuda.synchronize()
    return out


def _close(a, b):
    a, b = a.double(), b.double()
    err = (a - b).abs().max().item()
    rel = ((a - b).norm() / b.norm()).item()
    return err, rel


@pytest.mark.parametrize("forced", [0, 3], ids=["planner", "three_splits"])
def test_static_matches_workspace_call(forced):
    cfg = _cfg(forced)
    _, _, ws_bytes = lbm.lbm_query_sizes(cfg)
    ws = torch.empty(ws_bytes // 4, dtype=torch.int32, device=DEV)
    # two calls in a row, the second smaller (fewer pages, fewer queries, a
    # partial special page), so stale scratch from the first would show
    for i, (n_pp, n_st, nq) in enumerate(((72, 620, 1375), (5, 37, 300))):
        say("static scratch call", i, "forced splits", forced, "pages", n_pp, "specials", n_st,
            "queries", nq)
        pp, sp, q, pids, sids = _inputs(100 + i, n_pp, n_st, nq)
        ref = _call(lbm.lbm_paged_attention, cfg, pp, sp, q, pids, n_pp, sids, n_st, ws)
        got = _call(lbm.lbm_paged_attention_static, cfg, pp, sp, q, pids, n_pp, sids, n_st)
        assert not torch.isnan(got.float()).any()
        err, rel = _close(got, ref)
        say("  max-abs", err, "rel-L2", rel)
        assert err <= BF16_MAX_ABS and rel <= BF16_REL_L2
        if forced:
            assert torch.equal(got.view(torch.int16), ref.view(torch.int16))
        if i == 0 and forced == 0:
            # oracle on a sample of heads: dense fp64 attention over the listed rows
            kv_k = torch.cat([pp[pids.long(), 0].reshape(-1, H, D),
                              sp[sids.long(), 0].reshape(-1, H, D)[:n_st]])
            kv_v = torch.cat([pp[pids.long(), 1].reshape(-1, H, D),
                              sp[sids.long(), 1].reshape(-1, H, D)[:n_st]])
            heads = [0, 9]
            exp = dense_attention(q[:, heads].double().cpu().numpy(),
                                  kv_k[:, heads].double().cpu().numpy(),
                                  kv_v[:, heads].double().cpu().numpy())
            err, rel = _close(got[:, heads].cpu(), torch.from_numpy(exp))
            say("  vs oracle max-abs", err, "rel-L2", rel)
            assert err <= BF16_MAX_ABS and rel <= BF16_REL_L2


def test_static_rejects_a_visible_set_beyond_the_config():
    """More visible keys than the config allows (its scale and window pages,
    special pages and own rows) is refused before any launch, as the
    workspace call refuses it."""
    cfg = _cfg()
    q = torch.zeros((1, H, D), dtype=torch.bfloat16, device=DEV)
    ids = torch.zeros(80, dtype=torch.int32, device=DEV)
    for fn, extra in ((lbm.lbm_paged_attention_static, []),
                      (lbm.lbm_paged_attention, [q.data_ptr()])):
        with pytest.raises(lbm.LbmError) as ei:
            # 80 patch pages of 1369 keys: past 72 pages + 64 x 16 specials + 2048 rows
            fn(cfg, q.data_ptr(), q.data_ptr(), 1, q.data_ptr(), q.data_ptr(), ids.data_ptr(), 80,
               ids.data_ptr(), 0, *extra, torch.cuda.current_stream().cuda_stream)
        assert ei.value.name == "LBM_ERR_INVALID_ARG"
        assert "visible length" in str(ei.value)
