"""The unfused three-kernel ablation (S and P materialised in global memory)
against the float64 oracle, and against the fused path, on the same seeded
inputs.  Same gate as the fused parity tests (atol = rtol = 2e-2 on O,
1e-3 max(1, |ref|) on LSE)."""
import math

import numpy as np
import pytest

from scaled_dot_product_attn_amd import inputs
from test_parity import check, log, rnd, run

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("c", [1, 2, 3, 4, 5])
def test_unfused_workload_parity(gpu, oracle_mod, c):
    w = inputs.WORKLOADS[c]
    log(f"unfused workload {c} {w.name}")
    q, k, v = w.qkv()
    o, lse = run(gpu, q, k, v, w.causal, w.scale, unfused=True)
    o_ref, l_ref = oracle_mod.attn_fwd(q, k, v, w.causal, w.scale)
    check(o, lse, o_ref, l_ref, "unfused " + w.name)


@pytest.mark.parametrize("D", [64, 128, 512])
@pytest.mark.parametrize("causal", [False, True])
def test_unfused_ragged(gpu, oracle_mod, D, causal):
    for S in (1, 5, 33, 64, 65, 130, 200):
        log(f"unfused ragged D={D} causal={causal} S={S}")
        q, k, v = (rnd(30_000 + 7 * S + D + t, (2, 3, S, D)) for t in range(3))
        sc = 1 / math.sqrt(D)
        o, lse = run(gpu, q, k, v, causal, sc, unfused=True)
        o_ref, l_ref = oracle_mod.attn_fwd(q, k, v, causal, sc)
        check(o, lse, o_ref, l_ref, f"unfused S={S} D={D} causal={causal}")


@pytest.mark.parametrize("S,D,causal", [(700, 64, True), (1500, 128, False), (2900, 64, True),
                                         (4200, 64, True)])
def test_unfused_long_rows(gpu, oracle_mod, S, D, causal):
    """Rows of every length class of the softmax step: held in registers in
    groups of up to 1024, 2048 and 4096 entries, and longer rows (two passes
    over S).  Every row of one head against the oracle."""
    log(f"unfused long rows S={S} D={D} causal={causal}")
    q, k, v = (rnd(31_000 + S + D + t, (1, 1, S, D)) for t in range(3))
    sc = 1 / math.sqrt(D)
    o, lse = run(gpu, q, k, v, causal, sc, unfused=True)
    o_ref, l_ref = oracle_mod.attn_fwd(q, k, v, causal, sc)
    check(o, lse, o_ref, l_ref, f"unfused S={S} D={D} causal={causal}")


def test_unfused_matches_fused(gpu):
    """The two paths differ only in where S lives: their outputs agree to fp16
    rounding (well inside the gate)."""
    for c in (2, 3):
        w = inputs.WORKLOADS[c]
        q, k, v = w.qkv()
        of, lf = run(gpu, q, k, v, w.causal, w.scale)
        ou, lu = run(gpu, q, k, v, w.causal, w.scale, unfused=True)
        assert np.max(np.abs(of.astype(np.float64) - ou)) < 4e-3
        assert np.max(np.abs(lf.astype(np.float64) - lu)) < 1e-4
