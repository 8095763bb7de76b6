"""Brute-force re-derivations used to pin the vectorised oracle on tiny inputs.

These are deliberately written another way than ``rules`` and ``attention``:

* ``simulate_visible_slots`` replays the stream event by event -- append a
  frame's token slots, then evict the oldest non-scale frame's patch slots
  while more than ``sliding_window`` non-scale frames hold patch slots -- and
  keeps an explicit set of (frame, token) slots ([P1] "Sliding-Window Eviction
  Strategy"; [P3] "Sliding-Window Eviction Strategy"; specials are never
  evicted, [P2] "Special Stream (Append-Only)").
* ``scalar_attention`` evaluates the softmax with Python floats and
  ``math.exp``, one query row and one head at a time.
"""
from __future__ import annotations

import math
from typing import List, Set, Tuple


def simulate_visible_slots(step_frames: List[int], P: int, S: int, scale_frames: int,
                           sliding_window: int) -> List[Set[Tuple[int, int]]]:
    """For each step (frames per step listed in ``step_frames``), the set of
    visible (frame, token) slots after that step's append and eviction.
    Token t < P is a patch token of the frame, t >= P a special token."""
    slots: Set[Tuple[int, int]] = set()
    window_frames: List[int] = []          # non-scale frames holding patch slots, oldest first
    out = []
    frame = 0
    for nf in step_frames:
        for _ in range(nf):
            for t in range(P + S):
                slots.add((frame, t))
            if frame >= scale_frames:
                window_frames.append(frame)
            frame += 1
        while len(window_frames) > sliding_window:
            old = window_frames.pop(0)
            for t in range(P):
                slots.discard((old, t))
        out.append(set(slots))
    return out


def scalar_attention(q_row, keys, values) -> List[float]:
    """One query row, one head: q_row [D], keys/values lists of [D] rows."""
    D = len(q_row)
    scale = 1.0 / math.sqrt(D)
    scores = []
    for kr in keys:
        acc = 0.0
        for a, b in zip(q_row, kr):
            acc += float(a) * float(b)
        scores.append(acc * scale)
    m = max(scores)
    w = [math.exp(s - m) for s in scores]
    den = sum(w)
    Dv = len(values[0])
    out = [0.0] * Dv
    for wj, vr in zip(w, values):
        for d in range(Dv):
            out[d] += wj * float(vr[d])
    return [o / den for o in out]
