"""Seeded input generators (see the package docstring)."""
import ctypes
import os
import subprocess
import threading

import numpy as np
from scipy.special import erfinv, ndtri

from .configs import MoEConfig, record_bytes

FMT_CODES = {"bf16": 0, "fp8": 1, "mxfp4": 2}
_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gen.c")
_LIB = os.path.join(_HERE, "libsynth.so")
_lock = threading.Lock()
_lib = None

# tensor ids in the seed key
T_GATE, T_UP, T_DOWN, T_ROUTER, T_X, T_EPS, T_ZIPF = 1, 2, 3, 20, 30, 31, 40


def build_lib(force: bool = False) -> str:
    """Compile gen.c into libsynth.so (plain C, gcc)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + f".tmp{os.getpid()}"
        subprocess.check_call(["gcc", "-O3", "-fPIC", "-shared", "-pthread", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _L():
    global _lib
    with _lock:
        if _lib is None:
            lib = ctypes.CDLL(build_lib())
            i64, u64, vp = ctypes.c_int64, ctypes.c_uint64, ctypes.c_void_p
            lib.sx_key.restype = u64
            lib.sx_key.argtypes = [u64, vp, ctypes.c_int]
            lib.sx_fill_u16.argtypes = [vp, i64, u64, vp]
            lib.sx_fill_f32.argtypes = [vp, i64, u64, vp]
            lib.sx_fill_bytes.argtypes = [vp, i64, u64]
            lib.sx_fill_u8.argtypes = [vp, i64, u64, vp]
            lib.sx_gen_bank.restype = ctypes.c_int
            lib.sx_gen_bank.argtypes = [ctypes.c_int, i64, i64, u64, i64, i64, i64, i64, i64, i64,
                                        vp, i64, vp, vp, vp, ctypes.c_int]
            _lib = lib
    return _lib


def _ptr(a):
    return ctypes.c_void_p(a.ctypes.data)


def key(seed: int, *parts: int) -> int:
    p = np.asarray(parts, dtype=np.int64)
    return int(_L().sx_key(ctypes.c_uint64(seed), _ptr(p), len(parts)))


def f32_to_bf16(a) -> np.ndarray:
    """Round fp32 to bf16 bit patterns, to nearest even (finite inputs)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def bf16_to_f32(u16) -> np.ndarray:
    return (np.asarray(u16, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


_tables = {}


def normal_table_f32(sigma: float) -> np.ndarray:
    """65536 quantiles sigma * Phi^-1((i + 0.5) / 65536) in fp32."""
    k = ("f32", sigma)
    if k not in _tables:
        _tables[k] = (ndtri((np.arange(65536) + 0.5) / 65536.0) * sigma).astype(np.float32)
    return _tables[k]


def normal_table_bf16(sigma: float) -> np.ndarray:
    k = ("bf16", sigma)
    if k not in _tables:
        _tables[k] = f32_to_bf16(normal_table_f32(sigma))
    return _tables[k]


def e8m0_table(sigma: float = 0.02, block: int = 32) -> np.ndarray:
    """E8M0 scale bytes for MX blocks: the block max of `block` |N(0, sigma)|
    draws, sampled by inverse CDF (amax = sigma*sqrt(2)*erfinv(U**(1/block))),
    then the shared exponent floor(log2(amax)) - 2 (2 = largest e2m1 exponent),
    biased by 127."""
    k = ("e8m0", sigma, block)
    if k not in _tables:
        u = (np.arange(65536) + 0.5) / 65536.0
        amax = sigma * np.sqrt(2.0) * erfinv(u ** (1.0 / block))
        e = np.floor(np.log2(amax)).astype(np.int64) - 2 + 127
        _tables[k] = np.clip(e, 0, 254).astype(np.uint8)
    return _tables[k]


def fill_u16(n: int, k: int, table: np.ndarray) -> np.ndarray:
    out = np.empty(n, dtype=np.uint16)
    _L().sx_fill_u16(_ptr(out), n, ctypes.c_uint64(k), _ptr(table))
    return out


def fill_f32(n: int, k: int, table: np.ndarray) -> np.ndarray:
    out = np.empty(n, dtype=np.float32)
    _L().sx_fill_f32(_ptr(out), n, ctypes.c_uint64(k), _ptr(table))
    return out


def fill_u8(n: int, k: int, table: np.ndarray) -> np.ndarray:
    out = np.empty(n, dtype=np.uint8)
    _L().sx_fill_u8(_ptr(out), n, ctypes.c_uint64(k), _ptr(table))
    return out


def fill_bytes(n: int, k: int) -> np.ndarray:
    out = np.empty(n, dtype=np.uint8)
    _L().sx_fill_bytes(_ptr(out), n, ctypes.c_uint64(k))
    return out


def logical_streams(cfg: MoEConfig, layer: int, expert: int):
    """The generator's draws for one record, row-major, before any packing:
    [(gate, up, down)] where each entry is, per format,
      bf16 : bf16 bits [rows x K]
      fp8  : fp32 values [rows x K] (the record holds their block-FP8 encoding)
      mxfp4: (packed e2m1 bytes [rows x K/2], e8m0 scale bytes [rows x K/32])
    with (rows, K) = (f, d) for gate/up and (d, f) for down."""
    out = []
    for t in range(3):
        rows, K = (cfg.f, cfg.d) if t < 2 else (cfg.d, cfg.f)
        k = key(cfg.seed, cfg.cfg_id, t + 1, layer, expert)
        if cfg.fmt == "bf16":
            out.append(fill_u16(rows * K, k, normal_table_bf16(0.02)).reshape(rows, K))
        elif cfg.fmt == "fp8":
            out.append(fill_f32(rows * K, k, normal_table_f32(0.02)).reshape(rows, K))
        else:
            sk = key(cfg.seed, cfg.cfg_id, t + 11, layer, expert)
            out.append((fill_bytes(rows * K // 2, k).reshape(rows, K // 2),
                        fill_u8(rows * K // 32, sk, e8m0_table()).reshape(rows, K // 32)))
    return out


def router(cfg: MoEConfig, layer: int) -> np.ndarray:
    """Router matrix W_r [d x E] (bf16 bits), entries ~ N(0, 0.02)."""
    k = key(cfg.seed, cfg.cfg_id, T_ROUTER, layer)
    return fill_u16(cfg.d * cfg.E, k, normal_table_bf16(0.02)).reshape(cfg.d, cfg.E)


def tokens(cfg: MoEConfig, T: int, *tag: int) -> np.ndarray:
    """Hidden states x [T x d] (bf16 bits) ~ N(0, 1); `tag` selects the draw."""
    k = key(cfg.seed, cfg.cfg_id, T_X, *tag)
    return fill_u16(T * cfg.d, k, normal_table_bf16(1.0)).reshape(T, cfg.d)


def ar1_tokens(cfg: MoEConfig, layer: int, steps: int, rho: float = 0.9, s: float = 0.436) -> np.ndarray:
    """Per-layer AR(1) hidden-state stream: x_0 ~ N(0,1), x_t = rho*x_{t-1} + s*eps_t,
    kept in fp32 and returned as bf16 bits [steps x d] (one token per step)."""
    d = cfg.d
    eps = fill_f32(steps * d, key(cfg.seed, cfg.cfg_id, T_EPS, layer), normal_table_f32(1.0)).reshape(steps, d)
    x = np.empty((steps, d), dtype=np.float32)
    x[0] = eps[0]
    r, sc = np.float32(rho), np.float32(s)
    for t in range(1, steps):
        x[t] = r * x[t - 1] + sc * eps[t]
    return f32_to_bf16(x)


def zipf_routes(cfg: MoEConfig, T: int, step: int, alpha: float = 1.1):
    """Routes drawn from a Zipf(alpha) expert popularity: per token, k distinct
    experts sampled without replacement with p_r proportional to r^-alpha over a
    seeded permutation of the experts; weights ~ Dirichlet(1,...,1) (fp32)."""
    E, k = cfg.E, cfg.k
    perm_rng = np.random.Generator(np.random.PCG64(key(cfg.seed, cfg.cfg_id, T_ZIPF, 0)))
    perm = perm_rng.permutation(E)
    p = np.arange(1, E + 1, dtype=np.float64) ** (-alpha)
    p /= p.sum()
    rng = np.random.Generator(np.random.PCG64(key(cfg.seed, cfg.cfg_id, T_ZIPF, 1 + step, T)))
    ids = np.empty((T, k), dtype=np.int32)
    for t in range(T):
        ids[t] = perm[rng.choice(E, size=k, replace=False, p=p)]
    e = rng.standard_exponential((T, k))
    w = (e / e.sum(axis=1, keepdims=True)).astype(np.float32)
    return ids, w


def bank(cfg: MoEConfig, rec0: int = 0, rec1: int = None, out: np.ndarray = None,
         nthreads: int = None, layer_offset: int = 0) -> np.ndarray:
    """Records [rec0, rec1) of the host bank (flat id = layer*E + expert) as a
    [n x S] uint8 array; `out` may be a caller buffer (e.g. pinned memory)."""
    if rec1 is None:
        rec1 = cfg.layers * cfg.E
    S = cfg.S
    n = rec1 - rec0
    if out is None:
        out = np.empty((n, S), dtype=np.uint8)
    assert out.dtype == np.uint8 and out.size >= n * S and out.flags.c_contiguous
    if nthreads is None:
        nthreads = max(1, min(16, len(os.sched_getaffinity(0))))
    rc = _L().sx_gen_bank(FMT_CODES[cfg.fmt], cfg.d, cfg.f, ctypes.c_uint64(cfg.seed), cfg.cfg_id, cfg.E,
                          rec0, rec1, layer_offset, cfg.layer_alias, _ptr(out), S,
                          _ptr(normal_table_bf16(0.02)), _ptr(normal_table_f32(0.02)), _ptr(e8m0_table()),
                          int(nthreads))
    if rc != 0:
        raise ValueError("sx_gen_bank rejected the shape")
    return out.reshape(-1)[: n * S].reshape(n, S)


def record(cfg: MoEConfig, layer: int, expert: int) -> np.ndarray:
    """One layer-expert record as S bytes."""
    r = layer * cfg.E + expert
    return bank(cfg, r, r + 1, nthreads=1)[0]
