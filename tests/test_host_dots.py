"""The host branch's dot kernels (moe_expert_execution_amd/csrc/host_dots.h)
on the CPU: for every record format, both paths (one streaming pass for few
vectors; decode once + register-blocked tiles for many) give the dots of the
oracle-decoded matrix rows with the vectors, within fp32 rounding (the
streaming pass is called directly for 1..8 vectors, the dispatcher above
that); the streaming pass gives each vector the bits of a one-vector pass,
and the one-vector whole-panel pass the bits of the two half-panel passes.  A small g++ harness includes the header as the library does.  CPU
only."""
import os
import subprocess

import numpy as np
import pytest

import synth
from oracle import formats as OF

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "moe_expert_execution_amd", "csrc")
FMT = {"bf16": 0, "fp8": 1, "mxfp4": 2}

HARNESS = r"""
#include <stdio.h>
#include <stdlib.h>
#include <vector>
#include "host_dots.h"
using namespace ftmoe::hostk;
int main(int argc, char** argv) {
    const int fmt = atoi(argv[1]), K = atoi(argv[2]), nt = atoi(argv[3]), p = atoi(argv[4]), h = atoi(argv[5]);
    const long long off = atoll(argv[6]), soff = atoll(argv[7]);
    const int blocked = atoi(argv[11]);
    FILE* f = fopen(argv[8], "rb"); fseek(f, 0, SEEK_END); long n = ftell(f); fseek(f, 0, SEEK_SET);
    std::vector<unsigned char> rec(n); if (fread(rec.data(), 1, n, f) != (size_t)n) return 2; fclose(f);
    std::vector<float> v((size_t)nt * K);
    f = fopen(argv[9], "rb"); if (fread(v.data(), 4, v.size(), f) != v.size()) return 3; fclose(f);
    std::vector<const float*> vec(nt);
    for (int i = 0; i < nt; ++i) vec[i] = v.data() + (size_t)i * K;
    std::vector<float> wdec(16 * (size_t)K), out(blocked == 2 ? 32 : 16 * nt);
    if (blocked >= 3) {     // bf16: 3 = the decoded rows, 4 = their dots with bf16 vectors (v.bin holds bf16)
        const long long ld = decoded_ld(K);
        std::vector<uint16_t> w16(16 * (size_t)ld);
        half_panel_decode_bf16(fmt, rec.data(), off, soff, p, h, K, w16.data(), ld);
        f = fopen(argv[10], "wb");
        if (blocked == 3) {
            for (int r = 0; r < 16; ++r) fwrite(w16.data() + r * ld, 2, K, f);
        } else {
            const uint16_t* v16 = reinterpret_cast<const uint16_t*>(v.data());
            std::vector<const uint16_t*> vec16(nt);
            for (int i = 0; i < nt; ++i) vec16[i] = v16 + (size_t)i * K;
            dots_16xT_bf16(w16.data(), ld, K, vec16.data(), nt, out.data());
            fwrite(out.data(), 4, out.size(), f);
        }
        fclose(f);
        return 0;
    }
    if (blocked == 2) panel_dots_1(fmt, rec.data(), off, soff, p, K, vec[0], out.data());
    else if (blocked) { half_panel_decode(fmt, rec.data(), off, soff, p, h, K, wdec.data());
                   dots_16xT(wdec.data(), K, vec.data(), nt, out.data()); }
    else if (nt == 1) half_panel_dots_stream<1>(fmt, rec.data(), off, soff, p, h, K, vec.data(), out.data());
    else if (nt == 2) half_panel_dots_stream<2>(fmt, rec.data(), off, soff, p, h, K, vec.data(), out.data());
    else if (nt == 3) half_panel_dots_stream<3>(fmt, rec.data(), off, soff, p, h, K, vec.data(), out.data());
    else if (nt == 4) half_panel_dots_stream<4>(fmt, rec.data(), off, soff, p, h, K, vec.data(), out.data());
    else if (nt == 5) half_panel_dots_stream<5>(fmt, rec.data(), off, soff, p, h, K, vec.data(), out.data());
    else if (nt == 6) half_panel_dots_stream<6>(fmt, rec.data(), off, soff, p, h, K, vec.data(), out.data());
    else if (nt == 7) half_panel_dots_stream<7>(fmt, rec.data(), off, soff, p, h, K, vec.data(), out.data());
    else if (nt == 8) half_panel_dots_stream<8>(fmt, rec.data(), off, soff, p, h, K, vec.data(), out.data());
    else half_panel_dots(fmt, rec.data(), off, soff, p, h, K, vec.data(), nt, wdec.data(), out.data());
    f = fopen(argv[10], "wb"); fwrite(out.data(), 4, out.size(), f); fclose(f);
    return 0;
}
"""


@pytest.fixture(scope="module")
def harness(tmp_path_factory):
    d = tmp_path_factory.mktemp("hostdots")
    src = d / "h.cpp"
    src.write_text(HARNESS)
    exe = d / "h"
    subprocess.check_call(["g++", "-O2", "-std=c++17", "-mavx512f", "-mavx512bw", "-mavx512vl", "-mavx512dq", "-mavx512bf16",
                           "-I", CSRC, str(src), "-o", str(exe)])
    return exe, d


def offsets(fmt, d, f):
    """(gate, down, gate scales, down scales) byte offsets of the record layout."""
    fd = d * f
    if fmt == "bf16":
        return 0, 4 * fd, 0, 0
    if fmt == "fp8":
        nb = (d // 128) * (f // 128)
        return 0, 2 * fd, 3 * fd, 3 * fd + 8 * nb
    cb, sb = fd // 2, fd // 32
    return 0, 2 * cb, 3 * cb, 3 * cb + 2 * sb


@pytest.mark.parametrize("fmt", ["bf16", "fp8", "mxfp4"])
@pytest.mark.parametrize("blocked", [0, 1])
@pytest.mark.parametrize("nt", [1, 2, 3, 4, 5, 6, 7, 8, 13])
def test_half_panel_dots_match_decoded_rows(harness, fmt, blocked, nt):
    exe, tmp = harness
    d, f = 256, 128
    cfg = synth.CONFIGS["tiny"].with_(fmt=fmt, d=d, f=f, E=2, cfg_id=93)
    rec = synth.bank(cfg, 0, 1)[0]
    Wg, Wu, Wd = OF.decode_record(rec, fmt, d, f)
    og, od, osg, osd = offsets(fmt, d, f)
    rng = np.random.default_rng(nt + 10 * blocked)
    (tmp / "rec.bin").write_bytes(rec.tobytes())
    for mat, K, rows, off, soff in (("gate", d, Wg.T, og, osg), ("down", f, Wd.T, od, osd)):
        v = rng.standard_normal((nt, K)).astype(np.float32)
        (tmp / "v.bin").write_bytes(v.tobytes())
        for p in range(rows.shape[0] // 32):
            for h in (0, 1):
                subprocess.check_call([str(exe), str(FMT[fmt]), str(K), str(nt), str(p), str(h), str(off), str(soff),
                                       str(tmp / "rec.bin"), str(tmp / "v.bin"), str(tmp / "o.bin"), str(blocked)])
                got = np.fromfile(tmp / "o.bin", dtype=np.float32).reshape(nt, 16)
                ref = v.astype(np.float64) @ rows[32 * p + 16 * h: 32 * p + 16 * h + 16].T
                bound = 1e-5 * (np.abs(v).astype(np.float64) @ np.abs(rows[32 * p + 16 * h: 32 * p + 16 * h + 16]).T)
                assert np.all(np.abs(got - ref) <= bound + 1e-30), (mat, p, h, np.abs(got - ref).max())


@pytest.mark.parametrize("fmt", ["bf16", "fp8", "mxfp4"])
def test_panel_dots_1_same_bits_as_halves(harness, fmt):
    """One vector over a whole panel (rows 32p .. 32p + 31): the same float32
    bits as the streaming pass over its two halves (bf16, block-FP8), and
    within the bound of the oracle-decoded rows (every format); gate (K = d)
    and down (K = f) panels."""
    exe, tmp = harness
    d, f = 384, 256
    cfg = synth.CONFIGS["tiny"].with_(fmt=fmt, d=d, f=f, E=2, cfg_id=92)
    rec = synth.bank(cfg, 0, 1)[0]
    Wg, Wu, Wd = OF.decode_record(rec, fmt, d, f)
    og, od, osg, osd = offsets(fmt, d, f)
    rng = np.random.default_rng(5)
    (tmp / "rec.bin").write_bytes(rec.tobytes())

    def run(K, p, h, off, soff, mode, n):
        subprocess.check_call([str(exe), str(FMT[fmt]), str(K), "1", str(p), str(h), str(off), str(soff),
                               str(tmp / "rec.bin"), str(tmp / "v.bin"), str(tmp / "o.bin"), str(mode)])
        return np.fromfile(tmp / "o.bin", dtype=np.float32)[:n]

    for K, rows, off, soff in ((d, Wg.T, og, osg), (f, Wd.T, od, osd)):
        v = rng.standard_normal((1, K)).astype(np.float32)
        (tmp / "v.bin").write_bytes(v.tobytes())
        for p in range(rows.shape[0] // 32):
            whole = run(K, p, 0, off, soff, 2, 32)
            halves = np.concatenate([run(K, p, 0, off, soff, 0, 16), run(K, p, 1, off, soff, 0, 16)])
            if fmt != "mxfp4":      # MXFP4 scales each chunk's sum instead: fp32 rounding of the same products
                assert np.array_equal(whole.view(np.uint32), halves.view(np.uint32)), (K, p)
            ref = v.astype(np.float64) @ rows[32 * p: 32 * p + 32].T
            bound = 1e-5 * (np.abs(v).astype(np.float64) @ np.abs(rows[32 * p: 32 * p + 32]).T)
            assert np.all(np.abs(whole - ref[0]) <= bound[0] + 1e-30), (K, p)


def _bf16_rne(a):
    """float64 -> bf16 bits: to float32, then round to nearest even on the upper 16 bits."""
    u = np.asarray(a, np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


@pytest.mark.parametrize("fmt", ["bf16", "fp8", "mxfp4"])
@pytest.mark.parametrize("nt", [4, 7, 13])
def test_bf16_blocked_dots(harness, fmt, nt):
    """Many vectors in bf16: the decoded half-panel rows are the oracle's
    values exactly for bf16 and MXFP4 and e4m3 x block scale rounded to bf16
    for FP8 (within 2^-8 relative); their dots with bf16 vectors are the fp64
    dots of those same bf16 operands within fp32 rounding."""
    _check_bf16_blocked(harness, fmt, nt, 256, 128, down=True)


@pytest.mark.parametrize("fmt", ["bf16", "fp8", "mxfp4"])
def test_bf16_blocked_dots_sliced(harness, fmt):
    """As above with K = 2,304: the dots run over column slices of 1,024 (two
    whole slices and a ragged one), accumulators carried across slices."""
    _check_bf16_blocked(harness, fmt, 13, 2304, 128, down=False)


def _check_bf16_blocked(harness, fmt, nt, d, f, down):
    exe, tmp = harness
    cfg = synth.CONFIGS["tiny"].with_(fmt=fmt, d=d, f=f, E=2, cfg_id=91)
    rec = synth.bank(cfg, 0, 1)[0]
    Wg, Wu, Wd = OF.decode_record(rec, fmt, d, f)
    og, od, osg, osd = offsets(fmt, d, f)
    rng = np.random.default_rng(nt)
    (tmp / "rec.bin").write_bytes(rec.tobytes())
    mats = ((d, Wg.T, og, osg), (f, Wd.T, od, osd)) if down else ((d, Wg.T, og, osg),)
    for K, rows, off, soff in mats:
        v16 = _bf16_rne(rng.standard_normal((nt, K)))                            # bf16 vectors
        v64 = OF.bf16_to_f64(v16)
        (tmp / "v.bin").write_bytes(v16.tobytes() + bytes(2 * nt * K))
        for p in range(rows.shape[0] // 32):
            for h in (0, 1):
                args = [str(exe), str(FMT[fmt]), str(K), str(nt), str(p), str(h), str(off), str(soff),
                        str(tmp / "rec.bin"), str(tmp / "v.bin"), str(tmp / "o.bin")]
                subprocess.check_call(args + ["3"])
                w16 = OF.bf16_to_f64(np.fromfile(tmp / "o.bin", dtype=np.uint16)).reshape(16, K)
                ref_w = rows[32 * p + 16 * h: 32 * p + 16 * h + 16]
                if fmt == "fp8":
                    assert np.all(np.abs(w16 - ref_w) <= 2.0 ** -8 * np.abs(ref_w)), (K, p, h)
                else:
                    assert np.array_equal(w16, ref_w), (K, p, h)
                subprocess.check_call(args + ["4"])
                got = np.fromfile(tmp / "o.bin", dtype=np.float32).reshape(nt, 16)
                ref = v64 @ w16.T
                bound = 1e-5 * (np.abs(v64) @ np.abs(w16).T)
                assert np.all(np.abs(got - ref) <= bound + 1e-30), (K, p, h, np.abs(got - ref).max())


def test_fp8_every_code(harness):
    """A block-FP8 gate matrix whose codes run through all 254 non-NaN e4m3
    codes (both signs, zero, subnormals, the largest normal): the fp32
    decode gives each element as the oracle's decode times the block scale,
    rounded once to fp32 (read back by dots with one-hot vectors), and the
    streaming passes and the one-vector panel pass stay within the fp32
    bound of the oracle's dots."""
    exe, tmp = harness
    d, f = 256, 128
    cfg = synth.CONFIGS["tiny"].with_(fmt="fp8", d=d, f=f, E=2, cfg_id=94)
    rec = synth.bank(cfg, 0, 1)[0].copy()
    codes = np.array([c for c in range(256) if c & 0x7F != 0x7F], dtype=np.uint8)
    rec[: d * f] = np.resize(codes, d * f)
    Wg = OF.decode_record(rec, "fp8", d, f)[0]
    rows = Wg.T                                   # f rows of length d
    assert np.isin(codes, rec[: d * f]).all()
    og, _, osg, _ = offsets("fp8", d, f)
    (tmp / "rec.bin").write_bytes(rec.tobytes())
    (tmp / "v.bin").write_bytes(np.eye(d, dtype=np.float32).tobytes())
    for p in range(f // 32):
        for h in (0, 1):
            subprocess.check_call([str(exe), "1", str(d), str(d), str(p), str(h), str(og), str(osg),
                                   str(tmp / "rec.bin"), str(tmp / "v.bin"), str(tmp / "o.bin"), "1"])
            got = np.fromfile(tmp / "o.bin", dtype=np.float32).reshape(d, 16)
            want = rows[32 * p + 16 * h: 32 * p + 16 * h + 16].T.astype(np.float32)
            assert np.array_equal(got, want), (p, h)
    rng = np.random.default_rng(94)
    for nt in (1, 2, 3):
        v = rng.standard_normal((nt, d)).astype(np.float32)
        (tmp / "v.bin").write_bytes(v.tobytes())
        for p in range(f // 32):
            halves = []
            for h in (0, 1):
                subprocess.check_call([str(exe), "1", str(d), str(nt), str(p), str(h), str(og), str(osg),
                                       str(tmp / "rec.bin"), str(tmp / "v.bin"), str(tmp / "o.bin"), "0"])
                halves.append(np.fromfile(tmp / "o.bin", dtype=np.float32).reshape(nt, 16))
            got = np.concatenate(halves, axis=1)
            blk = rows[32 * p: 32 * p + 32]
            ref = v.astype(np.float64) @ blk.T
            bound = 1e-5 * (np.abs(v).astype(np.float64) @ np.abs(blk).T)
            assert np.all(np.abs(got - ref) <= bound + 1e-30), (nt, p, np.abs(got - ref).max())
            if nt == 1:
                subprocess.check_call([str(exe), "1", str(d), "1", str(p), "0", str(og), str(osg),
                                       str(tmp / "rec.bin"), str(tmp / "v.bin"), str(tmp / "o.bin"), "2"])
                assert np.array_equal(np.fromfile(tmp / "o.bin", dtype=np.float32), got[0]), p


@pytest.mark.parametrize("fmt", ["bf16", "fp8", "mxfp4"])
def test_stream_rows_per_pass_same_bits(harness, fmt):
    """The streaming pass for NT vectors takes the 16 rows in passes of fewer
    rows as NT grows (so its accumulators stay in registers); each row's
    multiply-adds keep their order, so every vector's dots are the bits the
    one-vector pass gives it."""
    exe, tmp = harness
    d, f = 512, 256
    cfg = synth.CONFIGS["tiny"].with_(fmt=fmt, d=d, f=f, E=2, cfg_id=95)
    rec = synth.bank(cfg, 0, 1)[0]
    og, od, osg, osd = offsets(fmt, d, f)
    (tmp / "rec.bin").write_bytes(rec.tobytes())
    rng = np.random.default_rng(95)
    v = rng.standard_normal((8, d)).astype(np.float32)

    def run(vs, p, h):
        (tmp / "v.bin").write_bytes(vs.tobytes())
        subprocess.check_call([str(exe), str(FMT[fmt]), str(d), str(len(vs)), str(p), str(h), str(og), str(osg),
                               str(tmp / "rec.bin"), str(tmp / "v.bin"), str(tmp / "o.bin"), "0"])
        return np.fromfile(tmp / "o.bin", dtype=np.float32).reshape(len(vs), 16)

    for p, h in ((0, 0), (f // 32 - 1, 1)):
        one = np.concatenate([run(v[i: i + 1], p, h) for i in range(8)])
        for nt in (2, 3, 4, 6, 7, 8):
            assert np.array_equal(run(v[:nt], p, h), one[:nt]), (nt, p, h)
