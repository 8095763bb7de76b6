"""The C-ABI libraries load and export every entry point the headers declare
(no device calls: this runs without a GPU)."""
import ctypes
import os
import re

import pytest

from paged_kv_cache_312_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared(header, prefix):
    with open(os.path.join(ROOT, "include", header)) as fh:
        text = fh.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(%s\w+)\s*\(" % prefix, text)))


def test_headers_declare_the_boundary():
    names = _declared("lbm.h", "lbm_")
    for n in ("lbm_cache_create", "lbm_append_frame", "lbm_evict_frames",
              "lbm_rollback_last_frame", "lbm_plan", "lbm_run"):
        assert n in names


def test_liblbm_exports_every_declared_symbol():
    names = _declared("lbm.h", "lbm_")
    lib = ctypes.CDLL(_lib.LIB_PATH)
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing, missing
    assert set(names) == set(_lib.LBM_FUNCS), set(names) ^ set(_lib.LBM_FUNCS)


def test_liblbm_core_exports_every_declared_symbol():
    names = _declared("lbm_core.h", "lbmcore_")
    lib = ctypes.CDLL(_lib.CORE_PATH)
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing, missing
    assert set(names) == set(_lib.CORE_FUNCS)


def test_struct_layouts_match_header():
    assert ctypes.sizeof(_lib.LbmConfig) == 14 * 4
    assert ctypes.sizeof(_lib.LbmStats) == 5 * 4


def test_query_sizes_without_device():
    """lbm_query_sizes is pure host arithmetic."""
    import paged_kv_cache_312_amd as p
    import workloads
    cfg = p.make_config(**workloads.lbm_config_fields(workloads.get_config(2)))
    pp, sp, ws = p.lbm_query_sizes(cfg)
    assert pp == 73 * 2 * 1369 * 16 * 64 * 2
    assert sp == cfg.max_special_pages * 2 * 16 * 16 * 64 * 2
    assert ws > 0 and ws % 256 == 0
    bad = p.make_config(**dict(workloads.lbm_config_fields(workloads.get_config(2)), num_heads=0))
    with pytest.raises(p.LbmError):
        p.lbm_query_sizes(bad)
