"""The C ABI: every function declared in include/moe_cache.h is exported by
libmoecache.so, and argument checks fail with MOE_EINVAL before any GPU work."""
import ctypes
import os
import re

import numpy as np
import pytest

import expert_cache_host_amd as m
from expert_cache_host_amd.binding import MoeError, Opts, load_library

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "moe_cache.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^[A-Za-z_][\w\s\*]*?\b(moe_\w+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_boundary():
    names = declared_functions()
    for must in ("moe_cache_create", "moe_layer_forward", "moe_cache_stats", "moe_cache_destroy"):
        assert must in names
    assert len(names) >= 20


@pytest.mark.parametrize("name", declared_functions())
def test_symbol_exported(name):
    lib = ctypes.CDLL(m.lib_path())
    assert hasattr(lib, name)


def test_default_opts():
    o = Opts()
    load_library().moe_cache_default_opts(ctypes.byref(o))
    assert (o.top_k, o.miss_mode, o.n_shared, o.norm_topk, o.max_fills_per_call) == (8, 0, 0, 1, -1)


@pytest.mark.parametrize("args,msg", [
    (dict(layers=0), "layers"),
    (dict(n_experts=0), "n_experts"),
    (dict(n_experts=513), "n_experts"),
    (dict(slots=0), "slots"),
    (dict(slots=9), "slots"),
    (dict(d_model=96), "d_model"),
    (dict(d_ff=48), "d_ff"),
    (dict(top_k=0), "top_k"),
    (dict(top_k=9), "top_k"),
    (dict(n_shared=2), "n_shared"),
    (dict(max_fills_per_call=-2), "max_fills"),
])
def test_create_rejects_bad_arguments(args, msg):
    base = dict(layers=1, n_experts=8, slots=4, d_model=64, d_ff=32, top_k=2, n_shared=0,
                max_fills_per_call=-1)
    base.update(args)
    w = np.zeros(8 * 3 * 64 * 32 // 32 * 18 * 4, np.uint8)
    with pytest.raises((MoeError, ValueError)) as ei:
        m.MoECache(base["layers"], base["n_experts"], base["slots"], base["d_model"], base["d_ff"], w,
                   top_k=base["top_k"], n_shared=base["n_shared"],
                   max_fills_per_call=base["max_fills_per_call"])
    if isinstance(ei.value, MoeError):
        assert ei.value.status == -1
        assert msg in str(ei.value)


def test_forward_rejects_null_cache():
    lib = load_library()
    assert lib.moe_layer_forward(None, 0, None, 1, None, None, None, None) == -1
    assert lib.moe_cache_stats(None, -1, None) == -1
    lib.moe_cache_destroy(None)  # no-op


def test_slot_bytes():
    assert m.slot_bytes(2816, 704) % 4096 == 0
    assert m.slot_bytes(2816, 704) >= 3_345_408
    assert m.slot_bytes(100, 32) == 0


def test_planner_rejects_bad_ids():
    p = m.Planner(8, 4)
    with pytest.raises(MoeError):
        p.plan([8])
    with pytest.raises(MoeError):
        p.plan([-1])
