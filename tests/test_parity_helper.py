"""The GPU tests' all-rows oracle evaluation (tests/gpu_util.py) gives the
oracle layer's values: it only spreads oracle.moe's per-expert work over
threads.  CPU only."""
import numpy as np
import pytest

import synth
from oracle import moe as OM, route as OR

from gpu_util import oracle_layer_all_rows, record_decoder


@pytest.mark.parametrize("fmt,d,f", [("bf16", 256, 128), ("fp8", 256, 256), ("mxfp4", 256, 128)])
def test_all_rows_equals_moe_layer(fmt, d, f):
    cfg = synth.CONFIGS["tiny"].with_(fmt=fmt, d=d, f=f, E=8, k=3, cfg_id=97)
    recs = synth.bank(cfg)
    x = synth.tokens(cfg, 37, 1)
    ids, w, _ = OR.route(x, synth.router(cfg, 0), cfg.k)
    dec = record_decoder(recs, cfg, 0)
    got = oracle_layer_all_rows(x, ids, w, dec, threads=4)
    ref = OM.moe_layer(x, ids, w, dec)
    assert got.shape == ref.shape == (37, d)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-15)
