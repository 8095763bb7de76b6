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
        def kv_of(f):
            if pending is not None and f in pending:
                return pending[f]
            return self.history.get(block, f)

        ks, vs = [], []
        for f in rules.visible_patch_frames(F, self.scale_frames, self.window):
            k, v = kv_of(f)
            ks.append(k[:self.P])
            vs.append(v[:self.P])
        for f in rules.visible_special_frames(F):
            k, v = kv_of(f)
            ks.append(k[self.P:self.P + self.S])
            vs.append(v[self.P:self.P + self.S])
        K = np.concatenate(ks, axis=0)
        V = np.concatenate(vs, axis=0)
        if heads is not None:
            heads = list(heads)
            K = K[:, heads, :]
            V = V[:, heads, :]
        return K, V

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
        K, V = self.visible_kv(block, self.F + nf, hs, pending)
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
