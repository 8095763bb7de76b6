"""Edge cases of the attention kernels through the stateless entry point
(lbm_paged_attention), where the caller's tables set the visible length
freely: lengths at and around the 64-key tile edges (one key, a partial
tile, exact tiles, a patch page plus a ragged special tail), query counts at
the edges of the kernels' row blocks (32-row halves, 64-row wavefronts,
128- and 256-row workgroups, the configured maximum), split counts from the
planner's to more splits than tiles, and every dtype.

Expected values: dense softmax attention (the oracle, fp64) over the visible
rows gathered in table order -- the listed patch pages, P tokens each, then
the first n_special_tokens tokens of the listed special pages ("How FlashInfer's
Paged KV Cache Attention Outperforms SDPA Fallback in Streaming Inference",
FAQ on variable sequence lengths; "How the Paged KV Cache Attention Mechanism
Enables Long Sequence Inference in LingBot-Map", "Building the Visible Page
Table").  Inputs are seeded unit-normal draws shared by both sides."""
import numpy as np
import pytest
import torch

import paged_kv_cache_312_amd as lbm
import workloads
from gpu_helpers import DEV, compare, say
from oracle import dense_attention

pytestmark = pytest.mark.gpu

P, SPS, H = 100, 16, 2          # patch page tokens, special page tokens, heads
N_PP, N_SP = 12, 12             # pages in each pool
MAX_Q = 300
DTYPE_CODE = {"bf16": 0, "f32": 1, "f16": 2}

# (patch pages, special tokens) -> visible length
KV_CASES = [(0, 1), (0, 63), (0, 64), (0, 65), (1, 0), (1, 27), (1, 28), (1, 29), (2, 27),
            (10, 0), (10, 191)]
TQ_CASES = [1, 31, 32, 33, 63, 64, 65, 127, 128, 129, 255, 256, 257, MAX_Q]
SPLITS = [0, 1, 3, 16]


def _config(dtype: str, head_dim: int, splits: int):
    return lbm.make_config(num_blocks=1, num_heads=H, head_dim=head_dim, patches_per_frame=P,
                           special_per_frame=6, special_page_size=SPS, scale_frames=2,
                           sliding_window=8, max_patch_pages=N_PP, max_special_pages=N_SP,
                           max_frames_per_step=1, max_q_tokens=MAX_Q, dtype=DTYPE_CODE[dtype],
                           num_splits=splits)


@pytest.mark.parametrize("dtype,head_dim", [("bf16", 64), ("f16", 64), ("f32", 64), ("f32", 32)])
def test_tile_and_row_edges(dtype, head_dim):
    D = head_dim
    seed0 = 9100 + 10 * DTYPE_CODE[dtype] + D
    pp = workloads.gen_normal((N_PP, 2, P, H, D), seed0 + 1, dtype, DEV)
    sp = workloads.gen_normal((N_SP, 2, SPS, H, D), seed0 + 2, dtype, DEV)
    q_all = workloads.gen_normal((MAX_Q, H, D), seed0 + 3, dtype, DEV)
    rng = np.random.default_rng(seed0)
    pid = rng.permutation(N_PP).astype(np.int32)
    sid = rng.permutation(N_SP).astype(np.int32)
    pid_d = torch.from_numpy(pid).to(DEV)
    sid_d = torch.from_numpy(sid).to(DEV)
    pp_h, sp_h = pp.double().cpu().numpy(), sp.double().cpu().numpy()
    q_h = q_all.double().cpu().numpy()
    stream = torch.cuda.current_stream().cuda_stream
    worst = 0.0
    n = 0
    for n_pp, n_st in KV_CASES:
        # visible rows in table order: whole patch pages, then special tokens
        k_rows = [pp_h[p, 0] for p in pid[:n_pp]] + [sp_h[s, 0] for s in sid]
        v_rows = [pp_h[p, 1] for p in pid[:n_pp]] + [sp_h[s, 1] for s in sid]
        kv = n_pp * P + n_st
        K = np.concatenate(k_rows)[:kv]
        V = np.concatenate(v_rows)[:kv]
        for tq in TQ_CASES:
            ref = dense_attention(q_h[:tq], K, V)
            q = q_all[:tq].contiguous()
            for splits in SPLITS:
                cfg = _config(dtype, D, splits)
                ws = torch.empty(lbm.lbm_query_sizes(cfg)[2], dtype=torch.uint8, device=DEV)
                out = torch.full_like(q, float("nan"))
                lbm.lbm_paged_attention(cfg, q.data_ptr(), out.data_ptr(), tq, pp.data_ptr(),
                                        sp.data_ptr(), pid_d.data_ptr(), n_pp, sid_d.data_ptr(),
                                        n_st, ws.data_ptr(), stream)
                torch.cuda.synchronize()
                st = compare(out.double().cpu().numpy(), ref, dtype,
                             f"{dtype} D={D} kv={kv} tq={tq} splits={splits}")
                worst = max(worst, st["max_abs"])
                n += 1
        say(f"{dtype} D={D}: kv={kv} done ({n} cases), worst max-abs {worst:.3e}")


# query counts around the 16-bit kernel's 512-row groups (the step's 32-row
# halves dealt over ceil(Tq / 512) groups: 15/14/14 at 1375)
TQ_GROUP_CASES = [511, 512, 513, 1024, 1025, 1375]


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_query_group_edges(dtype):
    """Query counts that fill, just exceed or split unevenly over the 16-bit
    kernel's 512-row workgroups, on short and tile-ragged key sets, with the
    planner's and a forced split count; every output against the oracle."""
    D, max_q = 64, max(TQ_GROUP_CASES)
    seed0 = 9300 + DTYPE_CODE[dtype]
    pp = workloads.gen_normal((N_PP, 2, P, H, D), seed0 + 1, dtype, DEV)
    sp = workloads.gen_normal((N_SP, 2, SPS, H, D), seed0 + 2, dtype, DEV)
    q_all = workloads.gen_normal((max_q, H, D), seed0 + 3, dtype, DEV)
    rng = np.random.default_rng(seed0)
    pid = rng.permutation(N_PP).astype(np.int32)
    sid = rng.permutation(N_SP).astype(np.int32)
    pid_d = torch.from_numpy(pid).to(DEV)
    sid_d = torch.from_numpy(sid).to(DEV)
    pp_h, sp_h = pp.double().cpu().numpy(), sp.double().cpu().numpy()
    q_h = q_all.double().cpu().numpy()
    stream = torch.cuda.current_stream().cuda_stream
    worst = 0.0
    for n_pp, n_st in [(0, 65), (2, 27), (10, 191)]:
        k_rows = [pp_h[p, 0] for p in pid[:n_pp]] + [sp_h[s, 0] for s in sid]
        v_rows = [pp_h[p, 1] for p in pid[:n_pp]] + [sp_h[s, 1] for s in sid]
        kv = n_pp * P + n_st
        K = np.concatenate(k_rows)[:kv]
        V = np.concatenate(v_rows)[:kv]
        for tq in TQ_GROUP_CASES:
            ref = dense_attention(q_h[:tq], K, V)
            q = q_all[:tq].contiguous()
            for splits in [0, 3]:
                cfg = lbm.make_config(num_blocks=1, num_heads=H, head_dim=D, patches_per_frame=P,
                                      special_per_frame=6, special_page_size=SPS, scale_frames=2,
                                      sliding_window=8, max_patch_pages=N_PP, max_special_pages=N_SP,
                                      max_frames_per_step=1, max_q_tokens=max_q,
                                      dtype=DTYPE_CODE[dtype], num_splits=splits)
                ws = torch.empty(lbm.lbm_query_sizes(cfg)[2], dtype=torch.uint8, device=DEV)
                out = torch.full_like(q, float("nan"))
                lbm.lbm_paged_attention(cfg, q.data_ptr(), out.data_ptr(), tq, pp.data_ptr(),
                                        sp.data_ptr(), pid_d.data_ptr(), n_pp, sid_d.data_ptr(),
                                        n_st, ws.data_ptr(), stream)
                torch.cuda.synchronize()
                st = compare(out.double().cpu().numpy(), ref, dtype,
                             f"{dtype} kv={kv} tq={tq} splits={splits}")
                worst = max(worst, st["max_abs"])
    say(f"{dtype} query-group edges: worst max-abs {worst:.3e}")


def test_empty_visible_set_is_rejected():
    cfg = _config("bf16", 64, 0)
    ws = torch.empty(lbm.lbm_query_sizes(cfg)[2], dtype=torch.uint8, device=DEV)
    q = torch.zeros(4, H, 64, dtype=torch.bfloat16, device=DEV)
    out = torch.empty_like(q)
    ids = torch.zeros(1, dtype=torch.int32, device=DEV)
    pool = torch.zeros(1, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(lbm.LbmError) as e:
        lbm.lbm_paged_attention(cfg, q.data_ptr(), out.data_ptr(), 4, pool.data_ptr(),
                                pool.data_ptr(), ids.data_ptr(), 0, ids.data_ptr(), 0,
                                ws.data_ptr(), torch.cuda.current_stream().cuda_stream)
    assert e.value.name == "LBM_ERR_INVALID_ARG"


def test_misaligned_buffers_are_rejected():
    """A workspace off 256-byte alignment, or a pool off 16, is refused before
    any launch."""
    cfg = _config("bf16", 64, 0)
    ws = torch.empty(lbm.lbm_query_sizes(cfg)[2] + 256, dtype=torch.uint8, device=DEV)
    q = torch.zeros(4, H, 64, dtype=torch.bfloat16, device=DEV)
    out = torch.empty_like(q)
    ids = torch.zeros(1, dtype=torch.int32, device=DEV)
    pool = torch.zeros(64, dtype=torch.bfloat16, device=DEV)
    st = torch.cuda.current_stream().cuda_stream
    for ws_ptr, pool_ptr in ((ws.data_ptr() + 64, pool.data_ptr()),
                             (ws.data_ptr(), pool.data_ptr() + 8)):
        with pytest.raises(lbm.LbmError) as e:
            lbm.lbm_paged_attention(cfg, q.data_ptr(), out.data_ptr(), 4, pool_ptr, pool_ptr,
                                    ids.data_ptr(), 1, ids.data_ptr(), 0, ws_ptr, st)
        assert e.value.name == "LBM_ERR_INVALID_ARG"
        assert "aligned" in str(e.value)


# (tile, key within the tile) of the planted score jumps: block 0 and block 1
# of inner tiles, a second, larger jump later in the same row, and the last
# (masked) tile
JUMPS = [(3, 5), (5, 40), (7, 50), (9, 0), (11, 33), (12, 2)]


@pytest.mark.parametrize("dtype,head_dim", [("bf16", 64), ("f16", 64), ("f32", 64)])
@pytest.mark.parametrize("splits", [1, 3])
def test_running_max_jumps(dtype, head_dim, splits):
    """Rows whose scores jump far above the running max inside key block 0
    or block 1 of a tile (the kernels' rescale paths), once or twice per row,
    on inner tiles and on the last, partly masked tile; compared with dense
    attention (the oracle) over the same rows.  A planted key dominates its
    row, whose output is then that key's V row, so V is drawn at 1/4 scale:
    the outputs stay in the range of the workload's averaged ones, for which
    the fp16 and bf16 bounds are set."""
    D = head_dim
    n_pp, n_st = 7, 91                    # 791 keys: 12 full tiles and a 23-key tail
    kv = n_pp * P + n_st
    seed0 = 9400 + 10 * DTYPE_CODE[dtype] + splits
    pp = workloads.gen_normal((N_PP, 2, P, H, D), seed0 + 1, dtype, DEV)
    sp = workloads.gen_normal((N_SP, 2, SPS, H, D), seed0 + 2, dtype, DEV)
    tq = 96
    q = workloads.gen_normal((tq, H, D), seed0 + 3, dtype, DEV)
    pp[:, 1] *= 0.25
    sp[:, 1] *= 0.25
    rng = np.random.default_rng(seed0)
    pid = rng.permutation(N_PP).astype(np.int32)
    sid = rng.permutation(N_SP).astype(np.int32)

    def slot(pos):
        """(pool, page, token) of visible key position pos under the tables."""
        if pos < n_pp * P:
            return pp, int(pid[pos // P]), pos % P
        j = pos - n_pp * P
        return sp, int(sid[j // SPS]), j % SPS

    # planted row j (query row 3j) jumps at JUMPS[j % 6] shifted by 2(j // 6),
    # and, for even j, again at JUMPS[(j + 2) % 6] shifted by 2(j // 6) + 1
    # with a larger score (no two plants share a key): K at that key is a
    # multiple of the row's query for head j % H, placing its score s1
    # (first) or s2 (second) above the unplanted ones.  The 16-bit kernel
    # lets weights grow to 2^64 (bf16) or 2^12 (fp16) past a running max of
    # 0 before it raises the max, so the bf16 plants sit ~72 and ~144 log2
    # units up (each past the limit), the others ~20 and ~43.
    s1, s2 = (50.0, 100.0) if dtype == "bf16" else (14.0, 30.0)
    for j, r in enumerate(range(0, tq, 3)):
        h = j % H
        qr = q[r, h].float()
        plants = [(JUMPS[j % 6], 2 * (j // 6), s1)]
        if j % 2 == 0:
            plants.append((JUMPS[(j + 2) % 6], 2 * (j // 6) + 1, s2))
        for (t, k), off, score in plants:
            pos = t * 64 + k + off
            assert pos < kv
            pool, page, tok = slot(pos)
            gain = score / float((qr * qr).sum()) * (D ** 0.5)
            pool[page, 0, tok, h] = (qr * gain).to(pool.dtype)
    pp_h, sp_h, q_h = pp.double().cpu().numpy(), sp.double().cpu().numpy(), q.double().cpu().numpy()
    K = np.concatenate([pp_h[p, 0] for p in pid[:n_pp]] + [sp_h[s, 0] for s in sid])[:kv]
    V = np.concatenate([pp_h[p, 1] for p in pid[:n_pp]] + [sp_h[s, 1] for s in sid])[:kv]
    ref = dense_attention(q_h, K, V)
    cfg = _config(dtype, D, splits)
    ws = torch.empty(lbm.lbm_query_sizes(cfg)[2], dtype=torch.uint8, device=DEV)
    out = torch.full_like(q, float("nan"))
    pid_d = torch.from_numpy(pid).to(DEV)   # kept alive until the launch has run
    sid_d = torch.from_numpy(sid).to(DEV)
    lbm.lbm_paged_attention(cfg, q.data_ptr(), out.data_ptr(), tq, pp.data_ptr(), sp.data_ptr(),
                            pid_d.data_ptr(), n_pp, sid_d.data_ptr(), n_st, ws.data_ptr(),
                            torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    # the planted keys dominate their rows (a weight of 2^8 or more against
    # the rest), which the test checks so that it exercises what it claims
    s = np.einsum("qhd,khd->qhk", q_h, K) / np.sqrt(D) * np.log2(np.e)
    lead = [s[r, j % H].max() - np.partition(s[r, j % H], -2)[-2]
            for j, r in enumerate(range(0, tq, 3))]
    assert min(lead) > 8.0, f"planted jumps too small: {min(lead):.1f}"
    st = compare(out.double().cpu().numpy(), ref, dtype, f"{dtype} jumps splits={splits}")
    say(f"{dtype} splits={splits}: max-abs {st['max_abs']:.3e}, smallest lead {min(lead):.1f}")


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("splits", [1, 3])
def test_rows_far_from_zero(dtype, splits):
    """Rows whose every score lies far above or far below 0 (log2 units),
    beside ordinary rows in the same wavefronts: the 16-bit kernel keeps a
    row's running max at 0 while its first scores stay in a window around 0,
    and otherwise starts it at their max and subtracts it from every later
    score (the biased path).  Head 1's keys get a constant added to feature
    0, and some query rows a large +-value there, which shifts each of those
    rows' scores by about +-90 log2 units; compared with dense attention (the
    oracle) over the same rows.  (The fp32 kernel has no such path; its
    tolerance, set for scores of ordinary size, does not cover scores this
    large, whose fp32 rounding grows with their magnitude.)"""
    D = 64
    n_pp, n_st = 7, 91                    # 791 keys: 12 full tiles and a 23-key tail
    kv = n_pp * P + n_st
    seed0 = 9600 + 10 * DTYPE_CODE[dtype] + splits
    pp = workloads.gen_normal((N_PP, 2, P, H, D), seed0 + 1, dtype, DEV)
    sp = workloads.gen_normal((N_SP, 2, SPS, H, D), seed0 + 2, dtype, DEV)
    tq = 200
    q = workloads.gen_normal((tq, H, D), seed0 + 3, dtype, DEV)
    pp[:, 0, :, 1, 0] += 8.0
    sp[:, 0, :, 1, 0] += 8.0
    # rows 4i get +64 in feature 0 of head 1, rows 4i+1 get -64: 8 * 64 / 8 =
    # 64 natural units (~92 log2 units) of shift, plus a spread of ~12 log2
    # units per key from the keys' own feature 0
    q[0::4, 1, 0] = 64.0
    q[1::4, 1, 0] = -64.0
    rng = np.random.default_rng(seed0)
    pid = rng.permutation(N_PP).astype(np.int32)
    sid = rng.permutation(N_SP).astype(np.int32)
    pp_h, sp_h, q_h = pp.double().cpu().numpy(), sp.double().cpu().numpy(), q.double().cpu().numpy()
    K = np.concatenate([pp_h[p, 0] for p in pid[:n_pp]] + [sp_h[s, 0] for s in sid])[:kv]
    V = np.concatenate([pp_h[p, 1] for p in pid[:n_pp]] + [sp_h[s, 1] for s in sid])[:kv]
    ref = dense_attention(q_h, K, V)
    # the shifted rows' scores really lie outside the window (all above 32 or
    # all below -32 log2 units)
    s = np.einsum("qd,kd->qk", q_h[:, 1], K[:, 1]) / np.sqrt(D) * np.log2(np.e)
    assert s[0::4].min() > 32.0 and s[1::4].max() < -32.0, (s[0::4].min(), s[1::4].max())
    cfg = _config(dtype, D, splits)
    ws = torch.empty(lbm.lbm_query_sizes(cfg)[2], dtype=torch.uint8, device=DEV)
    out = torch.full_like(q, float("nan"))
    pid_d = torch.from_numpy(pid).to(DEV)   # kept alive until the launch has run
    sid_d = torch.from_numpy(sid).to(DEV)
    lbm.lbm_paged_attention(cfg, q.data_ptr(), out.data_ptr(), tq, pp.data_ptr(), sp.data_ptr(),
                            pid_d.data_ptr(), n_pp, sid_d.data_ptr(), n_st, ws.data_ptr(),
                            torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    st = compare(out.double().cpu().numpy(), ref, dtype, f"{dtype} far rows splits={splits}")
    say(f"{dtype} splits={splits}: max-abs {st['max_abs']:.3e}")
