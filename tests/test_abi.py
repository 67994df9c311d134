"""The C ABI without a GPU: the library loads, exports every function the header
declares, the binding's structs match the C layout, and invalid arguments are
rejected before any device work."""
import ctypes
import os
import re
import subprocess
import sys

import pytest

import moe_expert_execution_amd as M
import synth
from oracle import formats as OF

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ftmoe.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(M.LIB_PATH):
        from moe_expert_execution_amd.build import build
        build(verbose=False)
    return M.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[\w\s\*]+?\b(ft_\w+)\s*\(", text, flags=re.M)))


def test_exports_every_declared_function(lib):
    names = declared_functions()
    assert len(names) >= 15, names
    for n in names:
        assert hasattr(lib, n), f"{n} not exported"
    assert set(names) <= set(M._SIGS), "binding lacks a signature"


def test_struct_layout_matches_header(tmp_path):
    structs = {"ft_shape": M.FtShape, "ft_profile": M.FtProfile, "ft_classify_out": M.FtClassifyOut,
               "ft_stats": M.FtStats, "ft_timing": M.FtTiming}
    src = ['#include <stdio.h>', '#include <stddef.h>', '#include "ftmoe.h"', 'int main(void) {']
    for cname, py in structs.items():
        src.append(f'printf("{cname} size %zu\\n", sizeof({cname}));')
        for f, _ in py._fields_:
            src.append(f'printf("{cname} {f} %zu\\n", offsetof({cname}, {f}));')
    src.append("return 0; }")
    c = tmp_path / "layout.c"
    c.write_text("\n".join(src))
    exe = tmp_path / "layout"
    subprocess.check_call(["gcc", "-std=c99", "-I", os.path.dirname(HEADER), str(c), "-o", str(exe)])
    out = subprocess.check_output([str(exe)], text=True).split("\n")
    got = {tuple(l.split()[:2]): int(l.split()[2]) for l in out if l.strip()}
    for cname, py in structs.items():
        assert got[(cname, "size")] == ctypes.sizeof(py), cname
        for f, _ in py._fields_:
            assert got[(cname, f)] == getattr(py, f).offset, (cname, f)


@pytest.mark.parametrize("name", ["tiny", "decode", "fp8", "mxfp4"])
def test_record_bytes_agree(lib, name):
    cfg = synth.CONFIGS[name]
    shp = M.shape(cfg.layers, cfg.E, cfg.k, cfg.d, cfg.f, cfg.fmt)
    assert M.ft_record_bytes(shp) == cfg.S == OF.record_size(cfg.fmt, cfg.d, cfg.f)


def test_argument_errors_without_device_work(lib):
    bad = M.shape(1, 300, 2, 256, 128, "bf16")                 # routing supports E <= 256
    st = lib.ft_moe_route(ctypes.byref(bad), 1, 1, 4, 1, 1, None)
    assert st == M.FT_ERR_ARG and "256" in M.ft_last_error()
    assert M.ft_record_bytes(M.shape(1, 8, 2, 100, 128, "bf16")) == 0   # d not a multiple of 128
    h = ctypes.c_void_p()
    prof = M.profile(20000, 60000)
    for shp, msg in [(M.shape(0, 8, 2, 256, 128), "layers"), (M.shape(1, 8, 9, 256, 128), "top_k"),
                     (M.shape(1, 8, 2, 256, 100), "multiples of 128"), (M.shape(1, 8, 2, 256, 128, 7), "fmt")]:
        st = lib.ft_cache_create(ctypes.byref(shp), ctypes.byref(prof), ctypes.c_void_p(1), 4, 16, ctypes.byref(h))
        assert st == M.FT_ERR_ARG and msg in M.ft_last_error(), (msg, M.ft_last_error())
    ok = M.shape(1, 8, 2, 256, 128)
    st = lib.ft_cache_create(ctypes.byref(ok), ctypes.byref(M.profile(0, 1)), ctypes.c_void_p(1), 4, 16,
                             ctypes.byref(h))
    assert st == M.FT_ERR_ARG
    st = lib.ft_cache_create(ctypes.byref(ok), ctypes.byref(prof), ctypes.c_void_p(1), 40000, 16, ctypes.byref(h))
    assert st == M.FT_ERR_ARG and "num_slots" in M.ft_last_error()
    assert lib.ft_cache_classify(None, 0, 1, 1, None, None) == M.FT_ERR_ARG
    assert lib.ft_moe_forward(None, 0, 0, 1, 1, 1, 1, 1, None) == M.FT_ERR_ARG
    assert lib.ft_cache_resize(None, 4) == M.FT_ERR_ARG
    assert lib.ft_cache_profile(None, 4, ctypes.byref(M.profile(1, 1))) == M.FT_ERR_ARG
    assert lib.ft_cache_set_profile(None, ctypes.byref(M.profile(1, 1))) == M.FT_ERR_ARG
    assert lib.ft_cache_destroy(None) == M.FT_OK


def test_multi_gpu_bench_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_bandwidth_profile_store_is_keyed_by_format_and_gpu(tmp_path):
    from moe_expert_execution_amd import bwprofile as B
    d = str(tmp_path)
    assert B.load("bf16", "gpu-a", d) is None
    B.save("bf16", "gpu-a", 52000, 104000, d)
    B.save("fp8", "gpu-a", 51000, 99000, d)
    assert B.load("bf16", "gpu-a", d) == (52000, 104000)
    assert B.load("fp8", "gpu-a", d) == (51000, 99000)
    assert B.load("mxfp4", "gpu-a", d) is None      # another format: not measured
    assert B.load("bf16", "gpu-b", d) is None       # another GPU: not this profile
    B.save("bf16", "gpu-a", 53000, 100000, d)
    assert B.load("bf16", "gpu-a", d) == (53000, 100000)
