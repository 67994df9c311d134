"""Shared helpers of the GPU parity tests (inputs from synth, checks against oracle)."""
import numpy as np
import pytest
import torch

import synth
from oracle import formats as OF

gpu = pytest.mark.gpu


def cuda():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import moe_expert_execution_amd as M
    M.lib()    # fails loudly when the HIP library is missing
    return torch.device("cuda")


def dev_u16(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def bf16_bits_to_f64(t: torch.Tensor) -> np.ndarray:
    return OF.bf16_to_f64(t.cpu().numpy().view(np.uint16))


def make_bank(cfg, rec0=0, rec1=None):
    from moe_expert_execution_amd.tensors import PinnedBank
    if rec1 is None:
        rec1 = cfg.layers * cfg.E
    bank = PinnedBank((rec1 - rec0) * cfg.S)
    synth.bank(cfg, rec0, rec1, out=bank.records(cfg.S))
    return bank


def expert_fn(bank_records, cfg, layer, rec_base=0, maxsize=24):
    """e -> decoded (Wg, Wu, Wd) of layer `layer` (record index minus rec_base)."""
    import functools

    @functools.lru_cache(maxsize=maxsize)
    def f(e):
        return OF.decode_record(bank_records[layer * cfg.E + e - rec_base], cfg.fmt, cfg.d, cfg.f)
    return f


def oracle_layer_all_rows(x, ids, w, decode, threads=None):
    """The oracle layer output [T x d] (fp64) for every row, evaluated expert by
    expert as oracle.moe.expert_terms does: each routed expert's record is
    decoded once (`decode(e)` -> (Wg, Wu, Wd)) and oracle.moe.ffn is applied to
    all of its routed rows; experts run on a thread pool (NumPy releases the
    interpreter lock in the decode's array work and in BLAS) and the terms are
    summed in ascending j by oracle.moe.combine.  Same values as
    oracle.moe.moe_layer (pinned by a CPU test)."""
    from concurrent.futures import ThreadPoolExecutor
    import os
    from oracle import moe as OM
    ids = np.asarray(ids)
    x64 = OF.bf16_to_f64(x)
    T, k = ids.shape
    terms = np.zeros((T, k, x64.shape[1]), dtype=np.float64)

    def one(e):
        tt, jj = np.nonzero(ids == e)
        Wg, Wu, Wd = decode(int(e))
        return tt, jj, OM.ffn(x64[tt], Wg, Wu, Wd)

    if threads is None:
        threads = max(1, min(16, len(os.sched_getaffinity(0))))
    from threadpoolctl import threadpool_limits
    # one BLAS thread per pool thread: the pool is the parallelism
    with threadpool_limits(limits=1, user_api="blas"), ThreadPoolExecutor(threads) as ex:
        for tt, jj, v in ex.map(one, np.unique(ids)):
            terms[tt, jj] = v
    return OM.combine(terms, w)


def record_decoder(bank_records, cfg, layer, rec_base=0):
    """e -> decoded (Wg, Wu, Wd) of layer `layer`, decoded afresh on each call."""
    def f(e):
        return OF.decode_record(bank_records[layer * cfg.E + e - rec_base], cfg.fmt, cfg.d, cfg.f)
    return f


def oracle_rows(x, ids, w, experts, rows):
    """Oracle layer output for the token rows `rows` only (fp64)."""
    from oracle import moe as OM
    rows = np.asarray(rows)
    return OM.moe_layer(x[rows], ids[rows], w[rows], experts)


def assert_close_rel(got, ref, tol, what=""):
    """max |got - ref| <= tol * max |ref| (the layer's float parity bar)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    scale = np.abs(ref).max()
    err = np.abs(got - ref).max()
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    assert err <= tol * scale, f"{what}: max err {err:.3e} > {tol} * {scale:.3e}"
    return err / scale if scale else 0.0
