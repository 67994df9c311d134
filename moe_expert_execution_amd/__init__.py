"""Python binding of the ftmoe C ABI (include/ftmoe.h): argument marshalling only.

Every step of the MoE layer runs in libftmoe.so (HIP kernels for gfx950 and the
library's host workers).  The functions here carry the C names and take device
pointers as integers (e.g. ``tensor.data_ptr()``) and a HIP stream as an
integer (``torch.cuda.current_stream().cuda_stream``); PyTorch is only used by
callers for device memory and streams.  If the shared library has not been
built, loading fails loudly: there is no fallback implementation.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libftmoe.so")

FT_OK, FT_ERR_ARG, FT_ERR_NOMEM, FT_ERR_HIP, FT_ERR_STATE, FT_ERR_UNSUPPORTED = range(6)
FT_FMT_BF16, FT_FMT_FP8_B128, FT_FMT_MXFP4_B32 = 0, 1, 2
FMT = {"bf16": FT_FMT_BF16, "fp8": FT_FMT_FP8_B128, "mxfp4": FT_FMT_MXFP4_B32}
FT_HIT, FT_FILL, FT_CPU = 0, 1, 2
FT_MODE_CACHED, FT_MODE_STREAMED, FT_PREFETCH_NEXT, FT_SINGLE_BUFFER, FT_WARM_DECODE = 0, 1, 0x100, 0x200, 0x400
ROUTE_INVALID = -(2 ** 31)

i32, i64, u32, u64, vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32, ctypes.c_uint64, ctypes.c_void_p


class FtShape(ctypes.Structure):
    _fields_ = [("layers", i32), ("experts", i32), ("top_k", i32), ("d_model", i32), ("d_ff", i32), ("fmt", i32)]


class FtProfile(ctypes.Structure):
    _fields_ = [("bp_mbps", u32), ("bh_mbps", u32), ("max_fetch", i32)]


class FtClassifyOut(ctypes.Structure):
    _fields_ = [("counts", vp), ("uniq", vp), ("cls", vp), ("slot", vp), ("ev_slot", vp), ("ev_old", vp),
                ("ev_new", vp), ("cpu_ids", vp), ("capacity", i32)]


class FtStats(ctypes.Structure):
    _fields_ = [("calls", u64), ("routes", u64), ("unique", u64), ("hits", u64), ("misses", u64), ("fills", u64),
                ("cpu_experts", u64), ("evictions", u64), ("bytes_filled", u64), ("layers_streamed", u64),
                ("clock", u64), ("error_flags", i32), ("num_slots", i32), ("host_experts", u64),
                ("host_bytes", u64), ("host_seconds", ctypes.c_double)]

    def as_dict(self):
        return {k: getattr(self, k) for k, _ in self._fields_}


FT_K_GEMV_GU, FT_K_GEMV_DOWN, FT_K_GEMM_GU, FT_K_GEMM_DOWN, FT_K_FILL = range(5)


class FtTiming(ctypes.Structure):
    _fields_ = [("launches", u64 * 5), ("ms", ctypes.c_double * 5), ("gemv_experts", u64), ("gemv_rows", u64),
                ("gemm_experts", u64), ("gemm_rows", u64)]


class FtError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"ftmoe status {status}: {msg}")
        self.status = status


_lib = None

# name -> (restype, argtypes)
_SIGS = {
    "ft_cache_create": (i32, [ctypes.POINTER(FtShape), ctypes.POINTER(FtProfile), vp, i64, i32, ctypes.POINTER(vp)]),
    "ft_cache_create_layers": (i32, [ctypes.POINTER(FtShape), ctypes.POINTER(FtProfile), ctypes.POINTER(vp), i64, i32,
                                     ctypes.POINTER(vp)]),
    "ft_cache_destroy": (i32, [vp]),
    "ft_record_bytes": (i64, [ctypes.POINTER(FtShape)]),
    "ft_moe_route": (i32, [ctypes.POINTER(FtShape), vp, vp, i32, vp, vp, vp]),
    "ft_cache_classify": (i32, [vp, i32, vp, i32, ctypes.POINTER(FtClassifyOut), vp]),
    "ft_moe_forward": (i32, [vp, i32, i32, vp, vp, vp, i32, vp, vp]),
    "ft_moe_forward_noalloc": (i32, [vp, i32, vp, vp, vp, i32, vp, vp]),
    "ft_cache_resize": (i32, [vp, i64]),
    "ft_cache_profile": (i32, [vp, i32, ctypes.POINTER(FtProfile)]),
    "ft_cache_set_profile": (i32, [vp, ctypes.POINTER(FtProfile)]),
    "ft_cache_stats": (i32, [vp, ctypes.POINTER(FtStats)]),
    "ft_cache_snapshot": (i32, [vp, vp, vp, vp, vp]),
    "ft_cache_set_timing": (i32, [vp, i32]),
    "ft_cache_timing": (i32, [vp, ctypes.POINTER(FtTiming)]),
    "ft_cache_read_slot": (i32, [vp, i64, vp]),
    "ft_host_alloc": (i32, [ctypes.c_size_t, ctypes.POINTER(vp)]),
    "ft_host_free": (i32, [vp]),
    "ft_last_error": (ctypes.c_char_p, []),
}


def lib():
    """Load libftmoe.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m moe_expert_execution_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def ft_last_error() -> str:
    return lib().ft_last_error().decode()


def _check(status):
    if status != FT_OK:
        raise FtError(status, ft_last_error())


def shape(layers, experts, top_k, d_model, d_ff, fmt="bf16") -> FtShape:
    return FtShape(layers, experts, top_k, d_model, d_ff, FMT[fmt] if isinstance(fmt, str) else fmt)


def profile(bp_mbps, bh_mbps, max_fetch=-1) -> FtProfile:
    return FtProfile(bp_mbps, bh_mbps, max_fetch)


def ft_record_bytes(shp: FtShape) -> int:
    return lib().ft_record_bytes(ctypes.byref(shp))


def ft_host_alloc(nbytes: int) -> int:
    p = vp()
    _check(lib().ft_host_alloc(nbytes, ctypes.byref(p)))
    return p.value


def ft_host_free(ptr: int) -> None:
    _check(lib().ft_host_free(ptr))


def host_array(ptr: int, nbytes: int) -> np.ndarray:
    """A uint8 NumPy view of `nbytes` of (pinned) host memory at `ptr`."""
    return np.ctypeslib.as_array(ctypes.cast(ptr, ctypes.POINTER(ctypes.c_uint8)), shape=(nbytes,))


def ft_cache_create(shp: FtShape, prof: FtProfile, host_bank: int, num_slots: int, max_tokens: int) -> int:
    h = vp()
    _check(lib().ft_cache_create(ctypes.byref(shp), ctypes.byref(prof), host_bank, num_slots, max_tokens,
                                 ctypes.byref(h)))
    return h.value


def ft_cache_create_layers(shp: FtShape, prof: FtProfile, layer_banks, num_slots: int, max_tokens: int) -> int:
    """`layer_banks`: one pinned host address per layer (entries may repeat)."""
    table = (vp * len(layer_banks))(*layer_banks)
    h = vp()
    _check(lib().ft_cache_create_layers(ctypes.byref(shp), ctypes.byref(prof), table, num_slots, max_tokens,
                                        ctypes.byref(h)))
    return h.value


def ft_cache_destroy(h: int) -> None:
    _check(lib().ft_cache_destroy(h))


def ft_moe_route(shp: FtShape, x: int, wr: int, T: int, ids: int, w: int, stream: int = 0) -> None:
    _check(lib().ft_moe_route(ctypes.byref(shp), x, wr, T, ids, w, stream))


def ft_cache_classify(h: int, layer: int, ids: int, T: int, out=None, stream: int = 0) -> None:
    _check(lib().ft_cache_classify(h, layer, ids, T, ctypes.byref(out) if out is not None else None, stream))


def ft_moe_forward(h: int, layer: int, mode: int, x: int, routes: int, w: int, T: int, y: int,
                   stream: int = 0) -> None:
    _check(lib().ft_moe_forward(h, layer, mode, x, routes, w, T, y, stream))


def ft_moe_forward_noalloc(h: int, layer: int, x: int, routes: int, w: int, T: int, y: int, stream: int = 0) -> None:
    _check(lib().ft_moe_forward_noalloc(h, layer, x, routes, w, T, y, stream))


def ft_cache_resize(h: int, num_slots: int) -> None:
    _check(lib().ft_cache_resize(h, num_slots))


def ft_cache_profile(h: int, records: int) -> FtProfile:
    out = FtProfile()
    _check(lib().ft_cache_profile(h, records, ctypes.byref(out)))
    return out


def ft_cache_set_profile(h: int, prof: FtProfile) -> None:
    _check(lib().ft_cache_set_profile(h, ctypes.byref(prof)))


def ft_cache_stats(h: int) -> FtStats:
    s = FtStats()
    _check(lib().ft_cache_stats(h, ctypes.byref(s)))
    return s


def ft_cache_set_timing(h: int, enable: bool) -> None:
    _check(lib().ft_cache_set_timing(h, 1 if enable else 0))


def ft_cache_timing(h: int) -> FtTiming:
    t = FtTiming()
    _check(lib().ft_cache_timing(h, ctypes.byref(t)))
    return t


def ft_cache_snapshot(h: int, n_ids: int, n_slots: int):
    sfi = np.empty(n_ids, np.int32)
    ios = np.empty(n_slots, np.int32)
    st = np.empty(n_slots, np.uint64)
    clk = np.zeros(1, np.uint64)
    _check(lib().ft_cache_snapshot(h, sfi.ctypes.data, ios.ctypes.data, st.ctypes.data, clk.ctypes.data))
    return sfi, ios, st, int(clk[0])


def ft_cache_read_slot(h: int, slot: int, nbytes: int) -> np.ndarray:
    out = np.empty(nbytes, np.uint8)
    _check(lib().ft_cache_read_slot(h, slot, out.ctypes.data))
    return out
