"""Reference page allocator for the two-stream cache (plain Python lists).

What the pages fix:

* two separate page pools: a recyclable patch stream with one page per frame,
  page size = patches per frame, no padding; and an append-only special stream
  whose tokens are packed continuously across pages ([P4] "Two-Stream Design";
  [P2] "Patch Stream (Recyclable)", "Special Stream (Append-Only)");
* append splits a frame into its patch part and its special part; patches go
  to a fresh or recycled page, specials to the continuous special pages
  ([P2] "Appending New Frames"; patches first, then specials: [P3] "Key methods");
* eviction pops the oldest live-window page while the window is larger than
  ``sliding_window`` and returns it to the free list; scale pages and special
  pages are never evicted, nothing is copied ([P3] "Sliding-Window Eviction
  Strategy"; [P2] "Evicting Stale Frames"; [P4] "Cache Reuse and Page Recycling");
* the visible table lists scale pages, then the latest window of live pages,
  then the special pages, and ``last_page_len`` is the number of valid tokens
  on the final (special) page ([P2] "Building the Visible Page Table";
  [P4] FAQ "How does the paged cache handle variable sequence lengths across
  frames?");
* deferred eviction and rollback of a provisional frame restore the cache
  state ([P3] "Flow-Based Keyframe Selection" and "Key methods");
* the stats record {frame_count, scale_pages, live_pages, free_pages,
  special_tokens} ([P3] "Inspecting Cache Statistics").

What the pages leave open, and the reading taken here (a convention; bit-exact
comparison is relative to it):

* free lists start in ascending id order; allocation pops the head; eviction
  pushes to the tail; rollback pushes back to the head;
* a special page is taken from its free list when a special token must be
  written and the count of special tokens so far is a multiple of the page size;
* eviction runs once after a step's whole append; evict is a commit: any later
  rollback is refused;
* rollback undoes only the last append, and only when it was one frame;
* the visible live pages are the latest ``sliding_window`` ones even while a
  provisional frame makes the live FIFO one longer than the window.
"""
from __future__ import annotations

import collections
from typing import Dict, List, Optional, Sequence

OUT_OF_PAGES = "out_of_pages"
BAD_STATE = "bad_state"
INVALID_ARG = "invalid_arg"


class AllocatorError(Exception):
    def __init__(self, kind: str, msg: str):
        super().__init__(f"{kind}: {msg}")
        self.kind = kind


class RefAllocator:
    def __init__(self, patches_per_frame: int, special_per_frame: int, special_page_size: int,
                 scale_frames: int, sliding_window: int, max_patch_pages: int,
                 max_special_pages: int, max_frames_per_step: int = 1 << 30,
                 patch_order: Optional[Sequence[int]] = None,
                 special_order: Optional[Sequence[int]] = None):
        if (patches_per_frame < 1 or special_per_frame < 0 or special_page_size < 1 or
                scale_frames < 0 or sliding_window < 0 or max_patch_pages < 1 or
                max_special_pages < 0):
            raise AllocatorError(INVALID_ARG, "bad configuration")
        self.P = patches_per_frame
        self.S = special_per_frame
        self.sps = special_page_size
        self.scale_frames = scale_frames
        self.window = sliding_window
        self.max_patch_pages = max_patch_pages
        self.max_special_pages = max_special_pages
        self.max_frames_per_step = max_frames_per_step
        self._patch_order = list(range(max_patch_pages)) if patch_order is None else list(patch_order)
        self._special_order = (list(range(max_special_pages)) if special_order is None
                               else list(special_order))
        if sorted(self._patch_order) != list(range(max_patch_pages)):
            raise AllocatorError(INVALID_ARG, "patch order is not a permutation")
        if sorted(self._special_order) != list(range(max_special_pages)):
            raise AllocatorError(INVALID_ARG, "special order is not a permutation")
        self.reset()

    # -- state -----------------------------------------------------------------
    def reset(self) -> None:
        """Empty cache, as for a new video ([P3] "Manual Cache Control for
        Advanced Use Cases": clean_kv_cache)."""
        self.patch_free = collections.deque(self._patch_order)
        self.special_free = collections.deque(self._special_order)
        self.scale: List[int] = []
        self.live = collections.deque()
        self.all_special: List[int] = []
        self.special_tokens = 0
        self.frame_count = 0
        self.page_frame: Dict[int, int] = {}     # patch page -> logical frame it holds
        self._undo = None

    # -- operations ------------------------------------------------------------
    def append(self, nf: int) -> dict:
        """Reserve pages for ``nf`` new frames.  Returns the write map:
        ``patch_pages`` (one per frame) and, per frame, the (page, slot) of each
        special token."""
        if nf < 1 or nf > self.max_frames_per_step:
            raise AllocatorError(INVALID_ARG, f"frames per step {nf}")
        # check capacity first so a refused append changes nothing
        if len(self.patch_free) < nf:
            raise AllocatorError(OUT_OF_PAGES, "patch free list exhausted")
        need_sp = 0
        t = self.special_tokens
        for _ in range(nf * self.S):
            if t % self.sps == 0:
                need_sp += 1
            t += 1
        if len(self.special_free) < need_sp:
            raise AllocatorError(OUT_OF_PAGES, "special free list exhausted")

        undo = {"nf": nf, "frame_count": self.frame_count, "special_tokens": self.special_tokens,
                "patch": [], "to_scale": [], "special": []}
        wmap = {"patch_pages": [], "special_slots": []}
        for _ in range(nf):
            page = self.patch_free.popleft()
            f = self.frame_count
            if f < self.scale_frames:
                self.scale.append(page)
                undo["to_scale"].append(True)
            else:
                self.live.append(page)
                undo["to_scale"].append(False)
            undo["patch"].append(page)
            self.page_frame[page] = f
            self.frame_count += 1
            wmap["patch_pages"].append(page)
            slots = []
            for _s in range(self.S):
                if self.special_tokens % self.sps == 0:
                    sp = self.special_free.popleft()
                    self.all_special.append(sp)
                    undo["special"].append(sp)
                slots.append((self.all_special[self.special_tokens // self.sps],
                              self.special_tokens % self.sps))
                self.special_tokens += 1
            wmap["special_slots"].append(slots)
        self._undo = undo
        return wmap

    def evict(self) -> List[int]:
        """Pop oldest live pages while the window is over-full; commit the step."""
        out = []
        while len(self.live) > self.window:
            page = self.live.popleft()
            self.patch_free.append(page)
            del self.page_frame[page]
            out.append(page)
        self._undo = None
        return out

    def rollback(self) -> None:
        """Undo the last single-frame append (before its evict)."""
        u = self._undo
        if u is None or u["nf"] != 1:
            raise AllocatorError(BAD_STATE, "nothing to roll back")
        page = u["patch"][0]
        if u["to_scale"][0]:
            assert self.scale[-1] == page
            self.scale.pop()
        else:
            assert self.live[-1] == page
            self.live.pop()
        del self.page_frame[page]
        self.patch_free.appendleft(page)
        for sp in reversed(u["special"]):
            assert self.all_special[-1] == sp
            self.all_special.pop()
            self.special_free.appendleft(sp)
        self.special_tokens = u["special_tokens"]
        self.frame_count = u["frame_count"]
        self._undo = None

    # -- views -----------------------------------------------------------------
    def visible_patch_pages(self) -> List[int]:
        live = list(self.live)
        if self.window == 0:
            live = []
        elif len(live) > self.window:
            live = live[len(live) - self.window:]
        return list(self.scale) + live

    def last_page_len(self) -> int:
        if self.special_tokens == 0:
            return 0
        return (self.special_tokens - 1) % self.sps + 1

    def kv_len(self) -> int:
        return len(self.visible_patch_pages()) * self.P + self.special_tokens

    def plan(self) -> List[int]:
        """Canonical plan record: [kv_len, n_patch_pages, n_special_pages,
        special_tokens, last_page_len, patch ids..., special ids...]."""
        pp = self.visible_patch_pages()
        return ([self.kv_len(), len(pp), len(self.all_special), self.special_tokens,
                 self.last_page_len()] + pp + list(self.all_special))

    def stats(self) -> dict:
        return {"frame_count": self.frame_count, "scale_pages": len(self.scale),
                "live_pages": len(self.live), "free_pages": len(self.patch_free),
                "special_tokens": self.special_tokens}

    def dump(self) -> List[int]:
        """Canonical state record: [frame_count, special_tokens, |scale|, scale...,
        |live|, live..., |patch free|, patch free..., |special|, special...,
        |special free|, special free...]."""
        out = [self.frame_count, self.special_tokens]
        for seq in (self.scale, self.live, self.patch_free, self.all_special, self.special_free):
            out.append(len(seq))
            out.extend(seq)
        return out

    def check_invariants(self, after_evict: bool) -> None:
        """Conservation and disjointness of both page sets; after an evict,
        resident patch pages are at most scale_frames + sliding_window; inside
        a provisional single-frame window, at most one more."""
        pages = list(self.scale) + list(self.live) + list(self.patch_free)
        assert sorted(pages) == list(range(self.max_patch_pages)), "patch pages not conserved"
        sp = list(self.all_special) + list(self.special_free)
        assert sorted(sp) == list(range(self.max_special_pages)), "special pages not conserved"
        resident = len(self.scale) + len(self.live)
        bound = self.scale_frames + self.window
        if after_evict:
            assert resident <= bound, "residency bound after evict"
        elif self._undo is not None and self._undo["nf"] == 1:
            assert resident <= bound + 1, "residency bound inside a provisional step"
        assert len(self.scale) <= self.scale_frames
        assert len(self.all_special) == -(-self.special_tokens // self.sps)
        assert set(self.page_frame) == set(self.scale) | set(self.live)
