"""Visible-set rules, written as closed forms over the logical frame history.

After a step the stream holds F accepted frames, numbered 0..F-1 in
acceptance order; the frames of the current step are included (the current
frame is appended, then eviction runs, then attention reads the table:
[P1] "Step-by-Step Streaming Inference", items 2-4).

* Scale frames: the first ``scale_frames`` frames ever accepted keep their
  patch pages for the whole stream ([P3] "Sliding-Window Eviction Strategy",
  scale protection; [P3] FAQ "What distinguishes scale frames from window
  frames in the KV cache?").
* Window frames: of the frames after the scale frames, only the latest
  ``sliding_window`` keep their patch pages; older ones are evicted oldest
  first ([P1] "Sliding-Window Eviction Strategy"; [P3] window management).
* Special tokens: every frame's special tokens stay visible for the whole
  stream, they are never evicted ([P2] "Special Stream (Append-Only)";
  [P1] "Two-Stream KV Cache Design").

Token order inside the visible set is scale pages, then live pages, then the
special stream ([P4] FAQ "How does the paged cache handle variable sequence
lengths across frames?").  The attention result does not depend on it.
"""
from __future__ import annotations

from typing import List, Tuple


def visible_patch_frames(F: int, scale_frames: int, sliding_window: int) -> List[int]:
    """Frames whose patch tokens are visible once F frames have been accepted,
    in visible-table order (scale frames, then the window, oldest first)."""
    if F < 0 or scale_frames < 0 or sliding_window < 0:
        raise ValueError("negative count")
    scale = list(range(min(scale_frames, F)))
    lo = max(scale_frames, F - sliding_window)
    live = list(range(lo, F))
    return scale + live


def visible_special_frames(F: int) -> List[int]:
    """Frames whose special tokens are visible: all of them, oldest first."""
    return list(range(F))


def visible_counts(F: int, scale_frames: int, sliding_window: int,
                   patches_per_frame: int, special_per_frame: int) -> Tuple[int, int, int]:
    """(visible patch frames, visible special tokens, total visible tokens)."""
    n_patch = min(F, scale_frames) + min(max(F - scale_frames, 0), sliding_window)
    n_special = F * special_per_frame
    return n_patch, n_special, n_patch * patches_per_frame + n_special


def steady_patch_pages(scale_frames: int, sliding_window: int) -> int:
    """Patch pages visible once the window is full: scale pages plus window
    pages ([P1] "Step-by-Step Streaming Inference", item 3, about 72 for the
    defaults 8 and 64)."""
    return scale_frames + sliding_window
