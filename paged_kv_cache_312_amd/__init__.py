"""Python binding of the two-stream paged-KV streaming-attention library.

Thin marshalling over the C ABI of ``include/lbm.h``: the functions below carry
the C names and pass plain integers (device pointers, hipStream_t handles).
``PagedKVCache`` adds ownership of the device memory through torch tensors
(pools, workspace) -- torch is used for device memory and streams only; every
step of the path runs in the library's HIP kernels and host code.
"""
from __future__ import annotations

import ctypes
import weakref
from ctypes import byref, c_int32, c_int64, c_size_t, c_void_p
from typing import List, Optional, Sequence, Tuple

from ._lib import (LBM_BF16, LBM_F16, LBM_F32, LbmConfig, LbmError, LbmStats, check, core_lib, lib)

__all__ = [
    "LBM_BF16", "LBM_F16", "LBM_F32", "LbmConfig", "LbmError", "LbmStats", "make_config",
    "lbm_query_sizes", "lbm_cache_create", "lbm_cache_destroy", "lbm_cache_reset",
    "lbm_cache_seed_free_lists", "lbm_append_frame", "lbm_evict_frames",
    "lbm_rollback_last_frame", "lbm_plan", "lbm_run", "lbm_plan_transient", "lbm_run_transient",
    "lbm_append_run", "lbm_run_batch", "MAX_BATCH", "lbm_graph_create", "lbm_graph_launch", "lbm_graph_destroy",
    "lbm_graph_num_splits", "StepGraph",
    "lbm_paged_attention", "lbm_paged_attention_static", "lbm_get_stats",
    "lbm_dump_state", "lbm_get_plan", "lbm_plan_num_splits", "lbm_last_error",
    "PagedKVCache", "CoreBookkeeping",
]


def make_config(num_blocks: int, num_heads: int, head_dim: int, patches_per_frame: int,
                special_per_frame: int, special_page_size: int, scale_frames: int,
                sliding_window: int, max_patch_pages: int, max_special_pages: int,
                max_frames_per_step: int, max_q_tokens: int, dtype: int,
                num_splits: int = 0) -> LbmConfig:
    return LbmConfig(num_blocks, num_heads, head_dim, patches_per_frame, special_per_frame,
                     special_page_size, scale_frames, sliding_window, max_patch_pages,
                     max_special_pages, max_frames_per_step, max_q_tokens, dtype, num_splits)


def _err():
    return lib().lbm_last_error()


def _ck(st, name):
    check(st, name, _err)


def _i32_array(seq):
    arr = (c_int32 * max(1, len(seq)))(*seq)
    return arr


# ---------------------------------------------------------------------------
# C-named entry points (pointers and streams are plain ints)
# ---------------------------------------------------------------------------

def lbm_last_error() -> str:
    m = lib().lbm_last_error()
    return m.decode() if m else ""


def lbm_query_sizes(cfg: LbmConfig) -> Tuple[int, int, int]:
    pp, sp, ws = c_size_t(), c_size_t(), c_size_t()
    _ck(lib().lbm_query_sizes(byref(cfg), byref(pp), byref(sp), byref(ws)), "lbm_query_sizes")
    return pp.value, sp.value, ws.value


def lbm_cache_create(cfg: LbmConfig, patch_pools: Sequence[int], special_pools: Sequence[int],
                     workspace: int) -> int:
    n = cfg.num_blocks
    pp = (c_void_p * n)(*patch_pools)
    sp = (c_void_p * n)(*special_pools)
    h = c_void_p()
    _ck(lib().lbm_cache_create(byref(cfg), pp, sp, c_void_p(workspace), byref(h)),
        "lbm_cache_create")
    return h.value


def lbm_cache_destroy(handle: int) -> None:
    lib().lbm_cache_destroy(c_void_p(handle))


def lbm_cache_reset(handle: int) -> None:
    _ck(lib().lbm_cache_reset(c_void_p(handle)), "lbm_cache_reset")


def lbm_cache_seed_free_lists(handle: int, patch_order: Sequence[int],
                              special_order: Sequence[int]) -> None:
    _ck(lib().lbm_cache_seed_free_lists(c_void_p(handle), _i32_array(patch_order),
                                        len(patch_order), _i32_array(special_order),
                                        len(special_order)), "lbm_cache_seed_free_lists")


def lbm_append_frame(handle: int, block_idx: int, k: int, v: int, num_frames: int,
                     stream: int) -> None:
    _ck(lib().lbm_append_frame(c_void_p(handle), block_idx, c_void_p(k), c_void_p(v),
                               num_frames, c_void_p(stream)), "lbm_append_frame")


def lbm_evict_frames(handle: int, cap: int = 4096) -> List[int]:
    buf = (c_int32 * max(1, cap))()
    n = c_int32()
    _ck(lib().lbm_evict_frames(c_void_p(handle), buf, cap, byref(n)), "lbm_evict_frames")
    return list(buf[:min(n.value, cap)])


def lbm_rollback_last_frame(handle: int) -> None:
    _ck(lib().lbm_rollback_last_frame(c_void_p(handle)), "lbm_rollback_last_frame")


def lbm_plan(handle: int, num_q_tokens: int, stream: int) -> None:
    _ck(lib().lbm_plan(c_void_p(handle), num_q_tokens, c_void_p(stream)), "lbm_plan")


def lbm_plan_num_splits(handle: int) -> int:
    return lib().lbm_plan_num_splits(c_void_p(handle))


def lbm_run(handle: int, block_idx: int, q: int, out: int, num_q_tokens: int,
            stream: int) -> None:
    _ck(lib().lbm_run(c_void_p(handle), block_idx, c_void_p(q), c_void_p(out), num_q_tokens,
                      c_void_p(stream)), "lbm_run")


def lbm_plan_transient(handle: int, num_q_tokens: int, num_own_tokens: int, stream: int) -> None:
    _ck(lib().lbm_plan_transient(c_void_p(handle), num_q_tokens, num_own_tokens,
                                 c_void_p(stream)), "lbm_plan_transient")


def lbm_run_transient(handle: int, block_idx: int, q: int, k: int, v: int, out: int,
                      num_q_tokens: int, stream: int) -> None:
    _ck(lib().lbm_run_transient(c_void_p(handle), block_idx, c_void_p(q), c_void_p(k),
                                c_void_p(v), c_void_p(out), num_q_tokens, c_void_p(stream)),
        "lbm_run_transient")


def lbm_append_run(handle: int, block_idx: int, q: int, k: int, v: int, out: int,
                   num_frames: int, num_q_tokens: int, stream: int) -> None:
    _ck(lib().lbm_append_run(c_void_p(handle), block_idx, c_void_p(q), c_void_p(k), c_void_p(v),
                             c_void_p(out), num_frames, num_q_tokens, c_void_p(stream)),
        "lbm_append_run")


MAX_BATCH = 8


def lbm_run_batch(handles: List[int], block_idx: int, qs: List[int], outs: List[int],
                  stream: int) -> None:
    n = len(handles)
    arr = lambda xs: (c_void_p * max(n, 1))(*[c_void_p(x) for x in xs])
    _ck(lib().lbm_run_batch(arr(handles), n, block_idx, arr(qs), arr(outs), c_void_p(stream)),
        "lbm_run_batch")


def lbm_graph_create(handle: int, num_frames: int, ks: List[int], vs: List[int], qs: List[int],
                     outs: List[int]) -> int:
    arr = lambda xs: (c_void_p * len(xs))(*[c_void_p(x) for x in xs])
    g = c_void_p()
    _ck(lib().lbm_graph_create(c_void_p(handle), num_frames, arr(ks), arr(vs), arr(qs), arr(outs),
                               ctypes.byref(g)), "lbm_graph_create")
    return g.value


def lbm_graph_launch(graph: int, stream: int) -> None:
    _ck(lib().lbm_graph_launch(c_void_p(graph), c_void_p(stream)), "lbm_graph_launch")


def lbm_graph_num_splits(graph: int) -> int:
    return lib().lbm_graph_num_splits(c_void_p(graph))


def lbm_graph_destroy(graph: int) -> None:
    lib().lbm_graph_destroy(c_void_p(graph))


def lbm_paged_attention(cfg: LbmConfig, q: int, out: int, num_q_tokens: int, patch_pool: int,
                        special_pool: int, patch_ids: int, n_patch_pages: int,
                        special_ids: int, n_special_tokens: int, workspace: int,
                        stream: int) -> None:
    _ck(lib().lbm_paged_attention(byref(cfg), c_void_p(q), c_void_p(out), num_q_tokens,
                                  c_void_p(patch_pool), c_void_p(special_pool),
                                  c_void_p(patch_ids), n_patch_pages, c_void_p(special_ids),
                                  n_special_tokens, c_void_p(workspace), c_void_p(stream)),
        "lbm_paged_attention")


def lbm_paged_attention_static(cfg: LbmConfig, q: int, out: int, num_q_tokens: int,
                               patch_pool: int, special_pool: int, patch_ids: int,
                               n_patch_pages: int, special_ids: int, n_special_tokens: int,
                               stream: int) -> None:
    _ck(lib().lbm_paged_attention_static(byref(cfg), c_void_p(q), c_void_p(out), num_q_tokens,
                                         c_void_p(patch_pool), c_void_p(special_pool),
                                         c_void_p(patch_ids), n_patch_pages,
                                         c_void_p(special_ids), n_special_tokens,
                                         c_void_p(stream)),
        "lbm_paged_attention_static")


def lbm_get_stats(handle: int) -> dict:
    s = LbmStats()
    _ck(lib().lbm_get_stats(c_void_p(handle), byref(s)), "lbm_get_stats")
    return s.as_dict()


def _record(fn, name, handle) -> List[int]:
    n = c_int64()
    _ck(fn(c_void_p(handle), None, 0, byref(n)), name)
    buf = (c_int32 * max(1, n.value))()
    _ck(fn(c_void_p(handle), buf, n.value, byref(n)), name)
    return list(buf[:n.value])


def lbm_dump_state(handle: int) -> List[int]:
    return _record(lib().lbm_dump_state, "lbm_dump_state", handle)


def lbm_get_plan(handle: int) -> List[int]:
    return _record(lib().lbm_get_plan, "lbm_get_plan", handle)


# ---------------------------------------------------------------------------
# torch-owned memory around one cache
# ---------------------------------------------------------------------------

class PagedKVCache:
    """A cache whose pools and workspace are torch tensors on one device.

    Tensors: ``patch_pools`` [num_blocks, max_patch_pages, 2, P, H, D] and
    ``special_pools`` [num_blocks, max_special_pages, 2, SPS, H, D] in the
    config dtype; ``workspace`` a byte tensor of the queried size.
    """

    def __init__(self, cfg: LbmConfig, device="cuda"):
        import torch
        self.torch = torch
        self.cfg = cfg
        self.device = torch.device(device)
        if self.device.type == "cuda" and self.device.index is None:
            self.device = torch.device("cuda", torch.cuda.current_device())
        self.dtype = {LBM_BF16: torch.bfloat16, LBM_F16: torch.float16,
                      LBM_F32: torch.float32}[cfg.dtype]
        pp_bytes, sp_bytes, ws_bytes = lbm_query_sizes(cfg)
        P, H, D = cfg.patches_per_frame, cfg.num_heads, cfg.head_dim
        self.patch_pools = torch.empty((cfg.num_blocks, cfg.max_patch_pages, 2, P, H, D),
                                       dtype=self.dtype, device=self.device)
        self.special_pools = torch.empty((cfg.num_blocks, max(1, cfg.max_special_pages), 2,
                                          cfg.special_page_size, H, D), dtype=self.dtype,
                                         device=self.device)
        # 256-byte alignment: torch's caching allocator returns 512-byte aligned blocks
        self.workspace = torch.zeros(max(256, ws_bytes), dtype=torch.uint8, device=self.device)
        assert self.workspace.data_ptr() % 256 == 0
        pps = [self.patch_pools[b].data_ptr() for b in range(cfg.num_blocks)]
        sps = [self.special_pools[b].data_ptr() for b in range(cfg.num_blocks)]
        self.handle = lbm_cache_create(cfg, pps, sps, self.workspace.data_ptr())

    def close(self):
        # graphs captured over this cache go first (they hold its handle)
        for g in list(getattr(self, "_graphs", ())):
            g.close()
        if getattr(self, "handle", None):
            lbm_cache_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def _stream(self, stream=None) -> int:
        if stream is None:
            stream = self.torch.cuda.current_stream(self.device)
        return stream.cuda_stream

    def _check_tensor(self, t, rows: Optional[int] = None):
        c = self.cfg
        if t.device != self.device or t.dtype != self.dtype or not t.is_contiguous():
            raise ValueError("tensor must be contiguous, on the cache device, in the cache dtype")
        if t.dim() != 3 or t.shape[1] != c.num_heads or t.shape[2] != c.head_dim:
            raise ValueError(f"tensor must be [tokens, {c.num_heads}, {c.head_dim}]")
        if rows is not None and t.shape[0] != rows:
            raise ValueError(f"expected {rows} rows, got {t.shape[0]}")

    def append_frame(self, block_idx: int, k, v, stream=None) -> None:
        T = self.cfg.patches_per_frame + self.cfg.special_per_frame
        nf = k.shape[0] // T
        self._check_tensor(k, nf * T)
        self._check_tensor(v, nf * T)
        lbm_append_frame(self.handle, block_idx, k.data_ptr(), v.data_ptr(), nf,
                         self._stream(stream))

    def evict_frames(self) -> List[int]:
        return lbm_evict_frames(self.handle, max(16, self.cfg.max_patch_pages))

    def rollback_last_frame(self) -> None:
        lbm_rollback_last_frame(self.handle)

    def plan(self, num_q_tokens: int, stream=None) -> None:
        self._own_rows = None
        lbm_plan(self.handle, num_q_tokens, self._stream(stream))

    def run(self, block_idx: int, q, out=None, stream=None):
        self._check_tensor(q)
        if out is None:
            out = self.torch.empty_like(q)
        else:
            self._check_tensor(out, q.shape[0])
        lbm_run(self.handle, block_idx, q.data_ptr(), out.data_ptr(), q.shape[0],
                self._stream(stream))
        return out

    def plan_transient(self, num_q_tokens: int, num_own_tokens: int, stream=None) -> None:
        """Plan a skip-append step (the frame's own rows follow the visible set)."""
        self._own_rows = None
        lbm_plan_transient(self.handle, num_q_tokens, num_own_tokens, self._stream(stream))
        self._own_rows = num_own_tokens

    def run_transient(self, block_idx: int, q, k, v, out=None, stream=None):
        """Attention of a skip-append step: q over the visible set and the
        frame's own k, v rows, which are never stored."""
        self._check_tensor(q)
        # the library reads exactly the planned number of own rows from k and v
        # (without a skip-append plan it refuses the call before any launch)
        self._check_tensor(k, getattr(self, "_own_rows", None))
        self._check_tensor(v, k.shape[0])
        if out is None:
            out = self.torch.empty_like(q)
        else:
            self._check_tensor(out, q.shape[0])
        lbm_run_transient(self.handle, block_idx, q.data_ptr(), k.data_ptr(), v.data_ptr(),
                          out.data_ptr(), q.shape[0], self._stream(stream))
        return out

    def append_run(self, block_idx: int, q, k, v, out=None, stream=None):
        """One block's append and attention of a frame step in one call
        (block 0 also reserves, plans for q's rows and evicts); returns out."""
        T = self.cfg.patches_per_frame + self.cfg.special_per_frame
        nf = k.shape[0] // T
        self._check_tensor(k, nf * T)
        self._check_tensor(v, nf * T)
        self._check_tensor(q)
        if out is None:
            out = self.torch.empty_like(q)
        else:
            self._check_tensor(out, q.shape[0])
        self._own_rows = None
        lbm_append_run(self.handle, block_idx, q.data_ptr(), k.data_ptr(), v.data_ptr(),
                       out.data_ptr(), nf, q.shape[0], self._stream(stream))
        return out

    def capture_step(self, num_frames: int, ks, vs, qs, outs) -> "StepGraph":
        """Capture a whole frame step over fixed per-block buffers (k, v, q,
        out lists, one tensor per block) as a HIP graph."""
        return StepGraph(self, num_frames, ks, vs, qs, outs)

    @staticmethod
    def run_batch(caches: List["PagedKVCache"], block_idx: int, qs, outs=None, stream=None):
        """Block ``block_idx`` of several caches (independent streams, each
        planned) in one batched launch; returns the outputs."""
        if outs is None:
            outs = [c.torch.empty_like(q) for c, q in zip(caches, qs)]
        for c, q, o in zip(caches, qs, outs):
            c._check_tensor(q)
            c._check_tensor(o, q.shape[0])
        lbm_run_batch([c.handle for c in caches], block_idx, [q.data_ptr() for q in qs],
                      [o.data_ptr() for o in outs], caches[0]._stream(stream))
        return outs

    def reset(self) -> None:
        lbm_cache_reset(self.handle)

    def seed_free_lists(self, patch_order, special_order) -> None:
        lbm_cache_seed_free_lists(self.handle, list(patch_order), list(special_order))

    def stats(self) -> dict:
        return lbm_get_stats(self.handle)

    def dump_state(self) -> List[int]:
        return lbm_dump_state(self.handle)

    def get_plan(self) -> List[int]:
        return lbm_get_plan(self.handle)

    def num_splits(self) -> int:
        return lbm_plan_num_splits(self.handle)


# ---------------------------------------------------------------------------
# host-only bookkeeping (liblbm_core.so), for tests without a GPU
# ---------------------------------------------------------------------------

class CoreBookkeeping:
    """The library's page bookkeeping driven directly, no device involved."""

    def __init__(self, cfg: LbmConfig):
        self._L = core_lib()
        h = c_void_p()
        self._ck(self._L.lbmcore_create(byref(cfg), byref(h)), "lbmcore_create")
        self.h = h

    def _ck(self, st, name):
        check(st, name, self._L.lbmcore_last_error)

    def __del__(self):
        try:
            if self.h:
                self._L.lbmcore_destroy(self.h)
                self.h = None
        except Exception:
            pass

    def _rec(self, fn, name):
        n = c_int64()
        self._ck(fn(self.h, None, 0, byref(n)), name)
        buf = (c_int32 * max(1, n.value))()
        self._ck(fn(self.h, buf, n.value, byref(n)), name)
        return list(buf[:n.value])

    def seed_free_lists(self, patch_order, special_order):
        self._ck(self._L.lbmcore_seed_free_lists(self.h, _i32_array(patch_order), len(patch_order),
                                                 _i32_array(special_order), len(special_order)),
                 "lbmcore_seed_free_lists")

    def reset(self):
        self._ck(self._L.lbmcore_reset(self.h), "lbmcore_reset")

    def append(self, nf: int):
        self._ck(self._L.lbmcore_append(self.h, nf), "lbmcore_append")

    def write_map(self):
        return self._rec(self._L.lbmcore_write_map, "lbmcore_write_map")

    def evict(self, cap: int = 4096):
        buf = (c_int32 * max(1, cap))()
        n = c_int32()
        self._ck(self._L.lbmcore_evict(self.h, buf, cap, byref(n)), "lbmcore_evict")
        return list(buf[:min(cap, n.value)])

    def rollback(self):
        self._ck(self._L.lbmcore_rollback(self.h), "lbmcore_rollback")

    def plan(self):
        return self._rec(self._L.lbmcore_plan, "lbmcore_plan")

    def dump(self):
        return self._rec(self._L.lbmcore_dump, "lbmcore_dump")

    def stats(self):
        s = LbmStats()
        self._ck(self._L.lbmcore_stats(self.h, byref(s)), "lbmcore_stats")
        return s.as_dict()

    @staticmethod
    def choose_splits(num_q_tokens, kv_len, num_heads, num_cu, wg_per_cu, split_cap, forced=0,
                      rows_per_wg=0):
        return core_lib().lbmcore_choose_splits(num_q_tokens, kv_len, num_heads, num_cu,
                                                wg_per_cu, split_cap, forced, rows_per_wg)

    @staticmethod
    def choose_launch(num_q_tokens, kv_len, num_heads, num_cu, wg_per_cu, split_cap, forced=0,
                      rows_per_wg=0):
        """(splits, query groups) as the 16-bit kernel's launches choose them."""
        g = c_int32(0)
        ns = core_lib().lbmcore_choose_launch(num_q_tokens, kv_len, num_heads, num_cu, wg_per_cu,
                                              split_cap, forced, rows_per_wg, byref(g))
        return ns, g.value


class StepGraph:
    """A frame step replayed as one HIP graph over fixed buffers: fill the
    buffers, then ``launch()`` does append, evict, plan and every block's
    attention (outputs in the ``outs`` tensors)."""

    def __init__(self, cache: PagedKVCache, num_frames: int, ks, vs, qs, outs):
        T = cache.cfg.patches_per_frame + cache.cfg.special_per_frame
        B = cache.cfg.num_blocks
        if not (len(ks) == len(vs) == len(qs) == len(outs) == B):
            raise ValueError(f"one k, v, q and out tensor per block ({B})")
        for t in list(ks) + list(vs) + list(qs) + list(outs):
            cache._check_tensor(t, num_frames * T)
        self.cache = cache
        self.buffers = (list(ks), list(vs), list(qs), list(outs))   # kept alive
        self.handle = lbm_graph_create(cache.handle, num_frames, [t.data_ptr() for t in ks],
                                       [t.data_ptr() for t in vs], [t.data_ptr() for t in qs],
                                       [t.data_ptr() for t in outs])
        if not hasattr(cache, "_graphs"):
            cache._graphs = weakref.WeakSet()
        cache._graphs.add(self)

    def num_splits(self) -> int:
        return lbm_graph_num_splits(self.handle)

    def launch(self, stream=None) -> None:
        if not self.handle:
            raise ValueError("the graph is closed")
        lbm_graph_launch(self.handle, self.cache._stream(stream))

    def close(self) -> None:
        if self.handle:
            lbm_graph_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
