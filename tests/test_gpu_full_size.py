"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times (automatic split count, the production decode kernel), plus
the debug variant for the logits.

The oracle encodes and decodes every sequence itself (it finishes these
sizes in seconds with all host threads), so every output, every logit and
every pool byte is compared, not a sample."""
import time

import numpy as np
import pytest

from long_context_decode_ada_amd import workloads as W
from oracle import oracle as O
from tests.parity_util import compare, gpu_run, oracle_run, planned_workloads, say

pytestmark = pytest.mark.gpu

FULL = ["gqa_t32k", "long_t128k", "ragged_b64", "mixed_tiers", "mixed_tiers_rdr"]


@pytest.fixture(scope="module")
def full_runs():
    held = {}

    def get(name):
        if name not in held:
            held.clear()            # keep one full-size workload in host memory at a time
            t0 = time.time()
            say("[full size] %s: generating" % name)
            if name == "mixed_tiers_rdr":
                # tiers and evictions planned by the controller (GPU and oracle plans equal)
                w, w_oracle = planned_workloads(W.rdr_inputs())
            else:
                w = w_oracle = W.make(name)
            say("[full size] %s: %d tokens, %d pages; GPU encode + decode (%.1fs)" %
                (name, w.n_tokens, w.num_pages, time.time() - t0))
            g = gpu_run(w)
            say("[full size] %s: oracle calibrate + encode + decode (%.1fs)" % (name, time.time() - t0))
            rng = O.calibrate(w_oracle.keys)
            o = oracle_run(w_oracle, rng)
            say("[full size] %s: ready (%.1fs)" % (name, time.time() - t0))
            held[name] = (w_oracle, g, o, rng)   # (the GPU plan's layout equals the oracle's)
        return held[name]
    return get


@pytest.mark.parametrize("name", FULL)
def test_full_size_encode_is_bit_exact(full_runs, name):
    w, g, o, rng = full_runs(name)
    assert np.array_equal(g["range"], rng)
    for k in ("kcode", "rcode", "v"):
        a, b = g["pools"][k], o["pools"][k]
        nd = int(np.count_nonzero(a != b))
        say("[%s full] %s mismatching bytes: %d of %d" % (name, k, nd, a.size))
        assert nd == 0
    assert g["errors"] == 0


@pytest.mark.parametrize("name", FULL)
def test_full_size_decode_matches_oracle(full_runs, name):
    w, g, o, rng = full_runs(name)
    compare(w, g, o, rng, label="%s full size" % name)
    if name in ("gqa_t32k", "long_t128k"):
        # the single-tier pools again with the query direction in binary32
        # (the precise mode, a few per cent slower on these pools)
        from long_context_decode_ada_amd import ska
        g32 = gpu_run(w, query_precision=ska.QDIR_F32)
        assert g32["errors"] == 0
        compare(w, g32, o, rng, label="%s full size, binary32 query direction" % name)
