"""The combine's wait for the host branch is bounded.  The bound is forced
down from the host (FTMOE_HOST_WAIT_POLLS=1, read when a cache is created)
while every miss runs on the host (max_fetch 0: no fills), so the host
experts take far longer than the GPU part of each call: the calls still
complete, error flag 8 is raised, and the cache shuts down cleanly.  With the
default bound the same calls wait, raise nothing and match the oracle."""
import numpy as np

import moe_expert_execution_amd as M
import synth
from moe_expert_execution_amd.tensors import SlotCache
from oracle import route as OR

from gpu_util import assert_close_rel, cuda, expert_fn, gpu, make_bank, oracle_rows
from test_gpu_layer import TOL, run_cached


def _calls(cfg, sc, bank, check):
    recs = bank.records(cfg.S)
    ex = expert_fn(recs, cfg, 0, maxsize=24)
    wr = synth.router(cfg, 0)
    xs = synth.ar1_tokens(cfg, 0, 3)
    for s in range(3):
        x = xs[s:s + 1]
        ids, w, _ = OR.route(x, wr, cfg.k)
        y, routes = run_cached(sc, 0, x, ids, w)
        assert np.all(routes < 0), "max_fetch 0 keeps every miss on the host"
        if check:
            assert_close_rel(y, oracle_rows(x, ids, w, ex, range(1)), TOL["bf16"], f"step {s}")


@gpu
def test_host_wait_bound_raises_flag_8(monkeypatch):
    cuda()
    cfg = synth.CONFIGS["decode"].with_(layers=1, slots=64)
    bank = make_bank(cfg)
    try:
        monkeypatch.setenv("FTMOE_HOST_WAIT_POLLS", "1")
        sc = SlotCache(1, cfg.E, cfg.k, cfg.d, cfg.f, "bf16", bank.ptr, cfg.slots, 1, cfg.bp_mbps, cfg.bh_mbps, 0)
        monkeypatch.delenv("FTMOE_HOST_WAIT_POLLS")
        try:
            _calls(cfg, sc, bank, check=False)
            st = M.ft_cache_stats(sc.handle)
            assert st.error_flags & 8, st.error_flags
            assert st.cpu_experts == 3 * cfg.k and st.fills == 0
        finally:
            sc.close()
        sc = SlotCache(1, cfg.E, cfg.k, cfg.d, cfg.f, "bf16", bank.ptr, cfg.slots, 1, cfg.bp_mbps, cfg.bh_mbps, 0)
        try:
            _calls(cfg, sc, bank, check=True)
            assert M.ft_cache_stats(sc.handle).error_flags == 0
        finally:
            sc.close()
    finally:
        bank.close()
