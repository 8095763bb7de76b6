"""The logical frame history and the per-step outputs of the streaming path.

State: the accepted frames, numbered in acceptance order, and for each one a
way to obtain its exact per-block K/V rows (a ``History`` object).  A step
brings nf new frames (several for the first pass, one per streaming step:
[P1] "Step-by-Step Streaming Inference", items 1-2) with their q/k/v rows
[nf * T, H, D], patches first and then specials ([P3] "Key methods",
append_frame).  The step's queries attend, with no mask inside the step, over
the visible set after the step's frames are appended and eviction has run
([P1] "Step-by-Step Streaming Inference", items 2-4; one visible table per
frame step, [P1] "FlashInfer Paged-Kernel Integration").  A provisional frame
that is rejected is dropped from the history ([P3] "Flow-Based Keyframe
Selection").

The visible set comes from ``rules`` (the closed form), never from a page table.
"""
from __future__ import annotations

from typing import Callable, Dict, Iterable, List, Optional, Tuple

import numpy as np

from . import rules
from .attention import dense_attention


class DictHistory:
    """In-memory history: (block, frame) -> (k [T,H,D], v [T,H,D]) as float64."""

    def __init__(self):
        self._kv: Dict[Tuple[int, int], Tuple[np.ndarray, np.ndarray]] = {}

    def put(self, block: int, frame: int, k: np.ndarray, v: np.ndarray) -> None:
        self._kv[(block, frame)] = (np.asarray(k, np.float64), np.asarray(v, np.float64))

    def drop(self, block: int, frame: int) -> None:
        self._kv.pop((block, frame), None)

    def get(self, block: int, frame: int) -> Tuple[np.ndarray, np.ndarray]:
        return self._kv[(block, frame)]

    def rows(self, block: int, frame: int, lo: int, hi: int, heads: Optional[List[int]] = None):
        """Token rows [lo, hi) of one frame, optionally some heads only."""
        k, v = self._kv[(block, frame)]
        k, v = k[lo:hi], v[lo:hi]
        if heads is not None:
            k, v = k[:, heads], v[:, heads]
        return k, v


class StreamOracle:
    """Plain fp64 streaming attention over the rule-derived visible set."""

    def __init__(self, patches_per_frame: int, special_per_frame: int, scale_frames: int,
                 sliding_window: int, history=None):
        self.P = patches_per_frame
        self.S = special_per_frame
        self.scale_frames = scale_frames
        self.window = sliding_window
        self.F = 0
        self.history = DictHistory() if history is None else history

    @property
    def T(self) -> int:
        return self.P + self.S

    def visible_kv(self, block: int, F: int, heads: Optional[Iterable[int]] = None,
                   pending: Optional[Dict[int, Tuple[np.ndarray, np.ndarray]]] = None):
        """Gather the visible K/V rows of ``block`` when F frames are accepted,
        in visible order: scale frames' patches, window frames' patches, then
        every frame's specials.  ``pending`` supplies frames not yet in the
        history (the current step's)."""
        hs = None if heads is None else list(heads)

        def rows_of(f, lo, hi):
            if pending is not None and f in pending:
                k, v = pending[f]
                k, v = np.asarray(k[lo:hi], np.float64), np.asarray(v[lo:hi], np.float64)
                if hs is not None:
                    k, v = k[:, hs], v[:, hs]
                return k, v
            return self.history.rows(block, f, lo, hi, hs)

        ks, vs = [], []
        for f in rules.visible_patch_frames(F, self.scale_frames, self.window):
            k, v = rows_of(f, 0, self.P)
            ks.append(k)
            vs.append(v)
        for f in rules.visible_special_frames(F):
            k, v = rows_of(f, self.P, self.P + self.S)
            ks.append(k)
            vs.append(v)
        return np.concatenate(ks, axis=0), np.concatenate(vs, axis=0)

    def step_outputs(self, block: int, q: np.ndarray, k_new: np.ndarray, v_new: np.ndarray,
                     rows: Optional[np.ndarray] = None, heads: Optional[List[int]] = None):
        """Outputs of the current step for ``block``: q, k_new, v_new are
        [nf*T, H, D].  Optionally only the given query rows / heads.  Does not
        change the history."""
        nf = q.shape[0] // self.T
        assert q.shape[0] == nf * self.T and k_new.shape[0] == nf * self.T
        pending = {}
        for i in range(nf):
            sl = slice(i * self.T, (i + 1) * self.T)
            pending[self.F + i] = (np.asarray(k_new[sl], np.float64),
                                   np.asarray(v_new[sl], np.float64))
        hs = list(range(q.shape[1])) if heads is None else list(heads)
        K, V = self.visible_kv(block, self.F + nf, None if heads is None else hs, pending)
        qq = np.asarray(q, np.float64)[:, hs, :]
        if rows is not None:
            qq = qq[np.asarray(rows)]
        return dense_attention(qq, K, V)

    def skip_append_outputs(self, block: int, q: np.ndarray, k_own: np.ndarray,
                            v_own: np.ndarray, rows: Optional[np.ndarray] = None,
                            heads: Optional[List[int]] = None):
        """Outputs of a frame processed without storing its K/V (skip-append,
        [P1] "Implementation Examples"; [P3] "Manual Cache Control for Advanced
        Use Cases"): q, k_own, v_own are the frame's [T', H, D] rows.  Its
        queries attend over the visible set of the F accepted frames followed
        by its own rows; the history and F are unchanged.  The pages say only
        that such a frame's K/V is not written to the cache; that it still
        attends to its own tokens is the plain reading of a block that
        computes attention over the cache and the current tokens."""
        hs = list(range(q.shape[1])) if heads is None else list(heads)
        K, V = self.visible_kv(block, self.F, None if heads is None else hs)
        K = np.concatenate([K, np.asarray(k_own, np.float64)[:, hs, :]], axis=0)
        V = np.concatenate([V, np.asarray(v_own, np.float64)[:, hs, :]], axis=0)
        qq = np.asarray(q, np.float64)[:, hs, :]
        if rows is not None:
            qq = qq[np.asarray(rows)]
        return dense_attention(qq, K, V)

    def commit(self, block_kv: Dict[int, Tuple[np.ndarray, np.ndarray]], nf: int) -> None:
        """Accept the step: store each block's new frames in the history."""
        for b, (k_new, v_new) in block_kv.items():
            for i in range(nf):
                sl = slice(i * self.T, (i + 1) * self.T)
                if isinstance(self.history, DictHistory):
                    self.history.put(b, self.F + i, k_new[sl], v_new[sl])
        self.F += nf

    def commit_count(self, nf: int) -> None:
        """Accept the step when the history regenerates frames by itself."""
        self.F += nf
