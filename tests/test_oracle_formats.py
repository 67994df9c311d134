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


def _panelize(logical: np.ndarray, unit: int) -> np.ndarray:
    """Logical [rows x row_bytes] -> panel-interleaved bytes, one unit at a time."""
    rows, rb = logical.shape
    U = rb // unit
    out = np.zeros(rows * rb, dtype=np.uint8)
    for r in range(rows):
        for c in range(U):
            dst = (r // 32) * 32 * rb + ((c // 2) * 64 + (c % 2) * 32 + r % 32) * unit
            out[dst:dst + unit] = logical[r, c * unit:(c + 1) * unit]
    return out


def test_unpanel_moves_each_unit_to_its_row_and_column():
    # 64 rows x 6 units of 2 bytes; each unit holds (row, column) so any misplacement shows
    rows, U, unit = 64, 6, 2
    logical = np.zeros((rows, U * unit), np.uint8)
    for r in range(rows):
        for c in range(U):
            logical[r, c * unit:(c + 1) * unit] = (r, c)
    phys = _panelize(logical, unit)
    assert np.array_equal(F.unpanel(phys, rows, U * unit, unit), logical)
    # unit (row 33, column 3) lies in panel 1 at unit (3 // 2) * 64 + 32 + 1 = 97
    o = 32 * U * unit + 97 * unit
    assert tuple(phys[o:o + 2]) == (33, 3)


def test_bf16_record_layout_and_orientation():
    d, f = 128, 64
    rng = np.random.default_rng(2)
    gT = rng.integers(-50, 50, (f, d)).astype(np.float32)   # small ints: exact in bf16
    uT = rng.integers(-50, 50, (f, d)).astype(np.float32)
    dT = rng.integers(-50, 50, (d, f)).astype(np.float32)
    rec = np.concatenate([_panelize(_bf16_bits(m).view(np.uint8), 16) for m in (gT, uT, dT)])
    assert rec.size == F.record_size("bf16", d, f)
    Wg, Wu, Wd = F.decode_record(rec, "bf16", d, f)
    assert Wg.shape == (d, f) and Wd.shape == (f, d)
    assert np.array_equal(Wg, gT.T) and np.array_equal(Wu, uT.T) and np.array_equal(Wd, dT.T)


def test_fp8_record_block_scales():
    d, f = 256, 128
    one = np.uint8(0x38)          # e4m3 1.0
    codes = np.full(3 * d * f, one, dtype=np.uint8)
    codes[0] = 0x40               # gate row 0, col 0 = 2.0 (unit 0 of panel 0)
    codes[16 * 33] = 0x30         # gate row 1, cols 16..31 (unit 33): col 16 = 0.5
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
    assert Wg[16, 1] == 1.5 and Wg[17, 1] == 3.0
    assert Wu[5, 7] == 7.0 and Wu[200, 7] == 11.0
    # Wd[n, c] = WdT[c, n]; row block of c (output dim) selects the scale
    assert Wd[3, 0] == 13.0 and Wd[3, 130] == 17.0


def test_mxfp4_record_nibbles_and_scales():
    d, f = 64, 64
    cb, sb = d * f // 2, d * f // 32
    codes = np.zeros(3 * cb, dtype=np.uint8)
    codes[0] = 0x72               # gate row 0: col 0 = code 2 (1.0), col 1 = code 7 (6.0)
    codes[cb + 1] = 0xF0 | 0x5    # up row 0: col 2 = 3.0, col 3 = code 15 (-6.0)
    scales = np.full(3 * sb, 127, dtype=np.uint8)    # 2^0
    scales[0] = 129                                  # gate row 0, k-block 0 -> 4
    scales[32] = 126                                 # gate row 0, k-block 1 (scale unit 32) -> 0.5
    rec = np.concatenate([codes, scales])
    assert rec.size == F.record_size("mxfp4", d, f)
    Wg, Wu, Wd = F.decode_record(rec, "mxfp4", d, f)
    assert Wg[0, 0] == 4.0 and Wg[1, 0] == 24.0 and Wg[2, 0] == 0.0
    assert Wu[2, 0] == 3.0 and Wu[3, 0] == -6.0
    codes2 = codes.copy()
    codes2[16 * 32] = 0x04        # gate row 0, chunk 1 (unit 32): col 32 = 2.0, in k-block 1
    Wg2, _, _ = F.decode_record(np.concatenate([codes2, scales]), "mxfp4", d, f)
    assert Wg2[32, 0] == 1.0
    assert np.all(Wd == 0)


@pytest.mark.parametrize("fmt", ["bf16", "fp8", "mxfp4"])
def test_records_decode_to_the_generator_draws(fmt):
    """A record from the seeded generator decodes to that generator's row-major
    draws: exactly for bf16 and MXFP4 codes, and within block-FP8 rounding
    (half an e4m3 step of the block scale, saturating at 448) for fp8."""
    import synth
    c = synth.CONFIGS["tiny"].with_(fmt=fmt, d=256, f=128, cfg_id=77)
    rec = synth.record(c, 0, 5)
    Wg, Wu, Wd = F.decode_record(rec, fmt, c.d, c.f)
    draws = synth.logical_streams(c, 0, 5)
    for got, raw in zip((Wg.T, Wu.T, Wd.T), draws):
        if fmt == "bf16":
            assert np.array_equal(got, F.bf16_to_f64(raw))
        elif fmt == "fp8":
            rows, K = raw.shape
            amax = np.abs(raw.astype(np.float64)).reshape(rows // 128, 128, K // 128, 128).max(axis=(1, 3))
            s = np.repeat(np.repeat(amax / 448.0, 128, 0), 128, 1)
            # e4m3: 3 mantissa bits -> relative half-step 2^-4; subnormal step 2^-9
            bound = np.maximum(np.abs(raw) * 2.0 ** -4, 2.0 ** -10 * s) + 1e-12
            assert np.all(np.abs(got - raw) <= bound)
        else:
            packed, sc = raw
            codes = np.empty((packed.shape[0], packed.shape[1] * 2), np.uint8)
            codes[:, 0::2] = packed & 0xF
            codes[:, 1::2] = packed >> 4
            ref = F.e2m1_to_f64(codes) * np.repeat(F.e8m0_to_f64(sc), 32, axis=1)
            assert np.array_equal(got, ref)
