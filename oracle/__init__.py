"""CPU oracle for two-stream paged-KV streaming attention.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this package; only the test-suite, the smoke check and the bench's
CPU-baseline leg use it.  It shares no code with the HIP path.

What it computes, in fp64, from the pages' rules and not from any paging:

* ``rules``      -- which frames' patch tokens and special tokens a step sees
                    (closed form of the scale / sliding-window / special rules);
* ``attention``  -- plain softmax(q k^T / sqrt(D)) v over a given token set;
* ``allocator``  -- a reference page allocator (free lists, scale list, live
                    FIFO, append-only special pages, undo of the last frame)
                    whose tables are compared bit-exact with the library's;
* ``stream``     -- the logical frame history and per-step outputs;
* ``brute``      -- scalar, loop-by-loop re-derivations used to pin the above.

Sources, cited by page title and section throughout:

* [P1] "How Paged KV Cache Attention Enables ~20 FPS Streaming Inference in LingBot-Map"
* [P2] "How the Paged KV Cache Attention Mechanism Enables Long Sequence Inference in LingBot-Map"
* [P3] "How LingBot-Map Uses KV Caching for Efficient Streaming Inference"
* [P4] "How FlashInfer's Paged KV Cache Attention Outperforms SDPA Fallback in Streaming Inference"

Every function here is pinned by a ``-m "not gpu"`` test against something
other than itself (a worked example printed on the pages, a closed form, a
library routine, a brute-force enumeration or an invariant).
"""
from .rules import (visible_patch_frames, visible_special_frames, visible_counts,
                    steady_patch_pages)
from .attention import dense_attention, dense_attention_rows
from .allocator import RefAllocator, AllocatorError
from .stream import StreamOracle, DictHistory

__all__ = [
    "visible_patch_frames", "visible_special_frames", "visible_counts", "steady_patch_pages",
    "dense_attention", "dense_attention_rows", "RefAllocator", "AllocatorError",
    "StreamOracle", "DictHistory",
]
