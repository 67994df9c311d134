"""Decoding of one layer-expert record into fp64 matrices.

A slot holds a complete layer-expert record: every bank (gate/up, down, and for
quantised formats their codes and block scales) belongs to one layer and one
expert ("The Expert Cache That Follows the Router", section "One logical
expert, two physical levels of memory").  The byte layout is the library's
documented record layout; this module decodes it independently:

  bf16 : WgT [f x d] | WuT [f x d] | WdT [d x f]                   (bf16)
  fp8  : codes WgT | WuT | WdT (e4m3fn)  then fp32 scales
         sg [f/128 x d/128] | su [f/128 x d/128] | sd [d/128 x f/128]
  mxfp4: codes WgT [f x d/2] | WuT | WdT [d x f/2] (two e2m1 per byte,
         low nibble = even column) then e8m0 scales
         sg [f x d/32] | su [f x d/32] | sd [d x f/32]

Code matrices and e8m0 scale matrices [rows x K] are stored in 32-row
panels (panel p = rows 32p..32p+31, one contiguous block); inside a panel,
unit c of row r (16 bytes of codes, or one scale byte, counted along K) sits
at unit (c // 2) * 64 + (c % 2) * 32 + r % 32.  fp8 block scales are plain
row-major.  ``unpanel`` undoes the interleave with one reshape/transpose.

The decoded matrices are returned in the orientation of the FFN definition:
Wg, Wu [d x f] and Wd [f x d], so that FFN(x) = (silu(x Wg) * (x Wu)) Wd.
"""
import numpy as np


def bf16_to_f64(u16) -> np.ndarray:
    """bf16 bit patterns -> float64 (a bf16 is the top half of an fp32)."""
    u = np.asarray(u16, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def e4m3fn_to_f64(codes) -> np.ndarray:
    """OCP FP8 E4M3 ("fn": no infinities; S.1111.111 is NaN; bias 7).
    Normal: (-1)^s * (1 + m/8) * 2^(e-7); subnormal (e = 0): (-1)^s * m * 2^-9."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = np.where(c >> 7, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    val = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    val = np.where((e == 15) & (m == 7), np.nan, val)
    return s * val


def e2m1_to_f64(nibbles) -> np.ndarray:
    """OCP MX FP4 E2M1 (bias 1, no inf/NaN).  Normal: (-1)^s (1 + m/2) 2^(e-1);
    subnormal (e = 0): (-1)^s * m * 0.5."""
    n = np.asarray(nibbles, dtype=np.uint8).astype(np.int64) & 0xF
    s = np.where(n >> 3, -1.0, 1.0)
    e = (n >> 1) & 0x3
    m = n & 0x1
    val = np.where(e == 0, m * 0.5, (1.0 + m / 2.0) * np.exp2(e - 1.0))
    return s * val


def e8m0_to_f64(codes) -> np.ndarray:
    """OCP MX E8M0 shared scale: 2^(e - 127); 0xFF is NaN."""
    e = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    return np.where(e == 255, np.nan, np.exp2(e - 127.0))


def record_size(fmt: str, d: int, f: int) -> int:
    if fmt == "bf16":
        return 6 * d * f
    if fmt == "fp8":
        return 3 * d * f + 12 * (d // 128) * (f // 128)
    if fmt == "mxfp4":
        return 3 * d * f // 2 + 3 * d * f // 32
    raise ValueError(fmt)


def unpanel(phys, rows: int, row_bytes: int, unit: int) -> np.ndarray:
    """Physical panel-interleaved bytes -> logical row-major [rows x row_bytes]."""
    U = row_bytes // unit                      # units per row (even)
    a = np.asarray(phys, dtype=np.uint8).reshape(rows // 32, U // 2, 2, 32, unit)
    # physical (panel, c // 2, c % 2, r, byte) -> logical (panel, r, c // 2, c % 2, byte)
    return a.transpose(0, 3, 1, 2, 4).reshape(rows, row_bytes)


def _codes(buf, off, rows, row_bytes):
    phys = np.frombuffer(buf, dtype=np.uint8, count=rows * row_bytes, offset=off)
    return unpanel(phys, rows, row_bytes, 16)


def _bf16_mat(buf, off, rows, cols):
    u = np.ascontiguousarray(_codes(buf, off, rows, 2 * cols)).view(np.uint16)
    return bf16_to_f64(u), off + 2 * rows * cols


# The decoders above applied once to every code point; indexing these tables is
# the same function, evaluated faster on large records.
_E4M3_TABLE = e4m3fn_to_f64(np.arange(256, dtype=np.uint8))
_E2M1_TABLE = e2m1_to_f64(np.arange(16, dtype=np.uint8))


def _fp8_mat(codes_buf, off, rows, cols, scales):
    c = _codes(codes_buf, off, rows, cols)
    w = _E4M3_TABLE[c]
    # each element scales by the fp32 scale of its 128x128 block
    w = w.reshape(rows // 128, 128, cols // 128, 128) * scales[:, None, :, None]
    return w.reshape(rows, cols)


def _mx_mat(buf, off, rows, cols, soff):
    packed = _codes(buf, off, rows, cols // 2)
    codes = np.empty((rows, cols), dtype=np.uint8)
    codes[:, 0::2] = packed & 0xF
    codes[:, 1::2] = packed >> 4
    sc = unpanel(np.frombuffer(buf, dtype=np.uint8, count=rows * cols // 32, offset=soff), rows, cols // 32, 1)
    w = _E2M1_TABLE[codes].reshape(rows, cols // 32, 32) * e8m0_to_f64(sc)[:, :, None]
    return w.reshape(rows, cols)


def decode_record(rec, fmt: str, d: int, f: int):
    """Return (Wg [d x f], Wu [d x f], Wd [f x d]) in float64."""
    buf = memoryview(np.ascontiguousarray(rec, dtype=np.uint8)).cast("B")
    if len(buf) < record_size(fmt, d, f):
        raise ValueError("record too short")
    if fmt == "bf16":
        gT, o = _bf16_mat(buf, 0, f, d)
        uT, o = _bf16_mat(buf, o, f, d)
        dT, o = _bf16_mat(buf, o, d, f)
    elif fmt == "fp8":
        base = 3 * d * f
        nb_gu = (f // 128) * (d // 128)

        def scales(i, r, c):
            off = base + 4 * nb_gu * i
            return np.frombuffer(buf, dtype=np.float32, count=r * c, offset=off).reshape(r, c).astype(np.float64)

        gT = _fp8_mat(buf, 0, f, d, scales(0, f // 128, d // 128))
        uT = _fp8_mat(buf, d * f, f, d, scales(1, f // 128, d // 128))
        dT = _fp8_mat(buf, 2 * d * f, d, f, scales(2, d // 128, f // 128))
    elif fmt == "mxfp4":
        cb = d * f // 2
        sb = d * f // 32
        base = 3 * cb
        gT = _mx_mat(buf, 0, f, d, base)
        uT = _mx_mat(buf, cb, f, d, base + sb)
        dT = _mx_mat(buf, 2 * cb, d, f, base + 2 * sb)
    else:
        raise ValueError(fmt)
    return gT.T.copy(), uT.T.copy(), dT.T.copy()
