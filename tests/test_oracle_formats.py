"""Pins for the oracle's record decoders (CPU only)."""
import os

import numpy as np
import pytest
import torch

from oracle import formats as F

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_e4m3_matches_torch_float8_e4m3fn():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = F.e4m3fn_to_f64(codes)
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], got[ok])
    assert np.nanmax(got) == 448.0 and got[1] == 2.0 ** -9


def test_e8m0_matches_torch_float8_e8m0fnu():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    got = F.e8m0_to_f64(codes)
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], got[ok])


def test_e2m1_matches_ocp_table():
    rows = [l.split() for l in open(os.path.join(GOLD, "e2m1_values.txt")) if l.strip() and not l.startswith("#")]
    codes = np.array([int(r[0]) for r in rows], dtype=np.uint8)
    vals = np.array([float(r[1]) for r in rows])
    got = F.e2m1_to_f64(codes)
    assert np.array_equal(got, vals)
    assert np.array_equal(np.signbit(got), np.signbit(vals))


def test_bf16_matches_torch_bfloat16():
    rng = np.random.default_rng(1)
    u = rng.integers(0, 65536, size=4096, dtype=np.uint16)
    u = u[((u >> 7) & 0xFF) != 0xFF]           # finite patterns only
    ref = torch.from_numpy(u.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(F.bf16_to_f64(u), ref)


def _bf16_bits(a):
    return torch.from_numpy(np.asarray(a, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_bf16_record_layout_and_orientation():
    d, f = 128, 128
    rng = np.random.default_rng(2)
    gT = rng.integers(-50, 50, (f, d)).astype(np.float32)   # small ints: exact in bf16
    uT = rng.integers(-50, 50, (f, d)).astype(np.float32)
    dT = rng.integers(-50, 50, (d, f)).astype(np.float32)
    rec = np.concatenate([_bf16_bits(m).reshape(-1) for m in (gT, uT, dT)]).view(np.uint8)
    assert rec.size == F.record_size("bf16", d, f)
    Wg, Wu, Wd = F.decode_record(rec, "bf16", d, f)
    assert Wg.shape == (d, f) and Wd.shape == (f, d)
    assert np.array_equal(Wg, gT.T) and np.array_equal(Wu, uT.T) and np.array_equal(Wd, dT.T)


def test_fp8_record_block_scales():
    d, f = 256, 128
    one = np.uint8(0x38)          # e4m3 1.0
    codes = np.full(3 * d * f, one, dtype=np.uint8)
    codes[0] = 0x40               # gate row 0, col 0 = 2.0
    nb = (f // 128) * (d // 128)
    sg = np.array([[3.0, 5.0]], np.float32)        # [f/128 x d/128] = [1 x 2]
    su = np.array([[7.0, 11.0]], np.float32)
    sd = np.array([[13.0], [17.0]], np.float32)    # [d/128 x f/128] = [2 x 1]
    rec = np.concatenate([codes, sg.reshape(-1).view(np.uint8), su.reshape(-1).view(np.uint8),
                          sd.reshape(-1).view(np.uint8)])
    assert rec.size == F.record_size("fp8", d, f) and nb == 2
    Wg, Wu, Wd = F.decode_record(rec, "fp8", d, f)
    # Wg[k, n] = WgT[n, k]; column block of k selects the scale
    assert Wg[0, 0] == 6.0 and Wg[1, 0] == 3.0 and Wg[128, 0] == 5.0 and Wg[255, 127] == 5.0
    assert Wu[5, 7] == 7.0 and Wu[200, 7] == 11.0
    # Wd[n, c] = WdT[c, n]; row block of c (output dim) selects the scale
    assert Wd[3, 0] == 13.0 and Wd[3, 130] == 17.0


def test_mxfp4_record_nibbles_and_scales():
    d, f = 64, 32
    cb, sb = d * f // 2, d * f // 32
    codes = np.zeros(3 * cb, dtype=np.uint8)
    codes[0] = 0x72               # gate row 0: col 0 = code 2 (1.0), col 1 = code 7 (6.0)
    codes[cb + 1] = 0xF0 | 0x5    # up row 0: col 2 = 3.0, col 3 = code 15 (-6.0)
    scales = np.full(3 * sb, 127, dtype=np.uint8)    # 2^0
    scales[0] = 129                                  # gate row 0, k-block 0 -> 4
    scales[1] = 126                                  # gate row 0, k-block 1 -> 0.5
    rec = np.concatenate([codes, scales])
    assert rec.size == F.record_size("mxfp4", d, f)
    Wg, Wu, Wd = F.decode_record(rec, "mxfp4", d, f)
    assert Wg[0, 0] == 4.0 and Wg[1, 0] == 24.0 and Wg[2, 0] == 0.0
    assert Wu[2, 0] == 3.0 and Wu[3, 0] == -6.0
    codes2 = codes.copy()
    codes2[16] = 0x04             # gate row 0: col 32 = 2.0, in k-block 1
    Wg2, _, _ = F.decode_record(np.concatenate([codes2, scales]), "mxfp4", d, f)
    assert Wg2[32, 0] == 1.0
    assert np.all(Wd == 0)
