"""GPU parity of the D = 128 forward on shapes with many 128-row query tiles
(B*H*ceil(S/128) >= 512, or >= 256 when not causal), which attn_fwd runs on
the 128-row kernel: four
waves per tile, each owning 32 complete rows, keys in 32-key chunks, the
causal mask applied on each wave's diagonal chunk only.

Same gate as the other parity tests (O: 2e-2 + 2e-2|ref|, LSE:
1e-3 max(1, |ref|)) against the float64 oracle; the oracle checks a sample of
(batch, head) slices where the call has hundreds of them (heads are
independent), all of them where it is cheap.
"""
import math

import numpy as np
import pytest

from scaled_dot_product_attn_amd import inputs
from test_parity import LSE_TOL, O_TOL, check, log, rnd, run

pytestmark = pytest.mark.gpu

D = 128


def heads_for(S, B=1):
    """Heads per batch so that B*H*ceil(S/128) >= 512 (the 128-row kernel)."""
    t = -(-S // 128)
    return -(-512 // (B * t))


def routed(B, H, S, causal=True):
    return B * H * (-(-S // 128)) >= (512 if causal else 256)


def sample_check(oracle_mod, q, k, v, o, lse, causal, sc, what, n_pick=6):
    B, H = q.shape[:2]
    picks = sorted({(0, 0), (B - 1, H - 1), (B // 2, H // 2), (0, H - 1), (B - 1, 0),
                    (B // 3, (2 * H) // 3)})[:n_pick]
    for b, h in picks:
        sl = (slice(b, b + 1), slice(h, h + 1))
        o_ref, l_ref = oracle_mod.attn_fwd(q[sl], k[sl], v[sl], causal, sc)
        check(o[sl], lse[sl], o_ref, l_ref, f"{what} b={b} h={h}")


RAGGED = [1, 31, 32, 33, 65, 96, 127, 128, 129, 200, 257, 300]


@pytest.mark.parametrize("causal", [False, True])
def test_rows_ragged(gpu, oracle_mod, causal):
    for S in RAGGED:
        B, H = 1, heads_for(S)
        assert routed(B, H, S)
        log(f"rows kernel ragged S={S} H={H} causal={causal}")
        q, k, v = (rnd(30_000 + 7 * S + t, (B, H, S, D)) for t in range(3))
        sc = 1 / math.sqrt(D)
        o, lse = run(gpu, q, k, v, causal, sc)
        sample_check(oracle_mod, q, k, v, o, lse, causal, sc, f"S={S} causal={causal}")


def paired(B, H, S):
    t = -(-S // 128)
    return B * H * ((t + 1) // 2) >= 512


@pytest.mark.parametrize("B,H,S", [(1, 512, 200), (2, 128, 300), (1, 128, 1000), (4, 64, 512)])
def test_rows_paired_tiles(gpu, oracle_mod, B, H, S):
    """Causal calls with at least 512 pairs of 128-row tiles, where one
    workgroup runs tiles T-1-u and u of a head: even and odd tile counts (the
    middle tile alone), ragged last tiles; every row of the sampled heads
    against the oracle, and the call's bytes repeat."""
    assert routed(B, H, S) and paired(B, H, S)
    log(f"rows kernel paired B={B} H={H} S={S}")
    q, k, v = (rnd(36_000 + 11 * S + t, (B, H, S, D)) for t in range(3))
    sc = 1 / math.sqrt(D)
    o, lse = run(gpu, q, k, v, True, sc)
    sample_check(oracle_mod, q, k, v, o, lse, True, sc, f"paired B={B} H={H} S={S}", n_pick=3)
    o2, lse2 = run(gpu, q, k, v, True, sc)
    assert np.array_equal(o, o2) and np.array_equal(lse, lse2)


def test_rows_workload4_every_head(gpu, oracle_mod):
    """Workload 4 (B8 H32 S512) on the 128-row kernel, every one of the 256
    (batch, head) slices against the oracle."""
    w = inputs.WORKLOADS[4]
    assert routed(w.B, w.H, w.S)
    q, k, v = w.qkv()
    o, lse = run(gpu, q, k, v, w.causal, w.scale)
    o_ref, l_ref = oracle_mod.attn_fwd(q, k, v, w.causal, w.scale)
    check(o, lse, o_ref, l_ref, w.name)


def test_rows_pins(gpu, oracle_mod):
    """P2 (causal row 0 = V[0] bit-exact, LSE closed form), P3 (identical keys:
    prefix mean), P4 (scale 0: mean, LSE = ln n), P12 (large logits) and a
    negative scale, on the 128-row kernel."""
    B, H, S = 2, 128, 160
    assert routed(B, H, S)
    sc = 1 / math.sqrt(D)
    q, k, v = (rnd(31_000 + t, (B, H, S, D)) for t in range(3))
    o, lse = run(gpu, q, k, v, True, sc)
    assert np.array_equal(o[:, :, 0, :], v[:, :, 0, :])
    want = float(np.float32(sc)) * (q[:, :, 0].astype(np.float64) * k[:, :, 0]).sum(-1)
    assert np.max(np.abs(lse[:, :, 0] - want)) <= LSE_TOL * max(1.0, np.max(np.abs(want)))

    kk = np.broadcast_to(rnd(31_010, (B, H, 1, D)), (B, H, S, D)).copy()
    v64 = v.astype(np.float64)
    for causal in (False, True):
        o, lse = run(gpu, q, kk, v, causal, sc)
        n = np.arange(1, S + 1) if causal else np.full(S, S)
        mean = (np.cumsum(v64, axis=2) / n[:, None]) if causal else \
            np.broadcast_to(v64.mean(2, keepdims=True), v64.shape)
        l_want = float(np.float32(sc)) * (q.astype(np.float64) * kk).sum(-1) + np.log(n)
        check(o, lse, mean, l_want, f"identical keys causal={causal}")
        o, lse = run(gpu, q, k, v, causal, 0.0)
        check(o, lse, mean, np.broadcast_to(np.log(n), lse.shape), f"scale 0 causal={causal}")
        for s2 in (8 / math.sqrt(D), -0.2):
            o, lse = run(gpu, q, k, v, causal, s2)
            sample_check(oracle_mod, q, k, v, o, lse, causal, s2, f"scale {s2:.3g} causal={causal}")


def test_rows_future_independence_and_repeat(gpu):
    """P10: changing K, V rows after i0 leaves rows <= i0 bit-identical; and
    the same inputs give the same output bytes."""
    B, H, S = 1, 256, 300
    assert routed(B, H, S)
    q, k, v = (rnd(32_000 + t, (B, H, S, D)) for t in range(3))
    i0 = 141
    k2, v2 = k.copy(), v.copy()
    k2[:, :, i0 + 1:] = rnd(32_100, k2[:, :, i0 + 1:].shape)
    v2[:, :, i0 + 1:] = rnd(32_200, v2[:, :, i0 + 1:].shape)
    o, lse = run(gpu, q, k, v, True, 1 / math.sqrt(D))
    o2, lse2 = run(gpu, q, k2, v2, True, 1 / math.sqrt(D))
    assert np.array_equal(o[:, :, :i0 + 1], o2[:, :, :i0 + 1])
    assert np.array_equal(lse[:, :, :i0 + 1], lse2[:, :, :i0 + 1])
    o3, lse3 = run(gpu, q, k, v, True, 1 / math.sqrt(D))
    assert np.array_equal(o, o3) and np.array_equal(lse, lse3)


def test_rows_value_identity(gpu):
    """P1 with S = D = 128: V = I makes O the probability matrix."""
    S = 128
    B, H = 1, heads_for(S)
    q, k = rnd(33_000, (B, H, S, S)), rnd(33_001, (B, H, S, S))
    v = np.broadcast_to(np.eye(S, dtype=np.float16), (B, H, S, S)).copy()
    for causal in (False, True):
        p, _ = run(gpu, q, k, v, causal, 1 / math.sqrt(S))
        p = p.astype(np.float64)
        assert np.all(p >= 0)
        assert np.max(np.abs(p.sum(-1) - 1.0)) <= S * 2.0 ** -11 + O_TOL
        if causal:
            assert np.all(np.triu(p, 1) == 0.0)


def test_rows_head_dim_coverage(gpu, oracle_mod):
    """P9 on the 128-row kernel."""
    B, H, S = 1, 256, 192
    for half in (0, 1):
        q, k, v = (rnd(34_000 + 10 * half + t, (B, H, S, D)) for t in range(3))
        lo = slice(0, D // 2) if half == 0 else slice(D // 2, D)
        q[..., lo] = 0
        k[..., lo] = 0
        sc = 2 / math.sqrt(D)
        o, lse = run(gpu, q, k, v, True, sc)
        sample_check(oracle_mod, q, k, v, o, lse, True, sc, f"coverage half={half}")


def test_rows_slice_alone_matches_within_gate(gpu, oracle_mod):
    """P11 across the dispatch threshold: a (b, h) slice of a call routed to
    the 128-row kernel, launched alone, runs the 64-row kernel; the two agree
    to rounding (each within the gate of the oracle) and, for a slice of a
    call that is itself routed, bit for bit."""
    B, H, S = 1, 256, 200
    assert routed(B, H, S) and not routed(1, 1, S)
    q, k, v = (rnd(35_000 + t, (B, H, S, D)) for t in range(3))
    sc = 1 / math.sqrt(D)
    o, lse = run(gpu, q, k, v, True, sc)
    h = 77
    o1, l1 = run(gpu, q[:, h:h + 1], k[:, h:h + 1], v[:, h:h + 1], True, sc)
    o_ref, l_ref = oracle_mod.attn_fwd(q[:, h:h + 1], k[:, h:h + 1], v[:, h:h + 1], True, sc)
    check(o[:, h:h + 1], lse[:, h:h + 1], o_ref, l_ref, "slice of the routed call")
    check(o1, l1, o_ref, l_ref, "slice alone")
    # the same slice inside another routed call (different neighbours) is bit-exact
    q2, k2, v2 = q.copy(), k.copy(), v.copy()
    for t in (q2, k2, v2):
        t[:, :h] = rnd(35_100, t[:, :h].shape)
    o2, l2 = run(gpu, q2, k2, v2, True, sc)
    assert np.array_equal(o[:, h:h + 1], o2[:, h:h + 1])
    assert np.array_equal(lse[:, h:h + 1], l2[:, h:h + 1])


@pytest.mark.parametrize("B,H,S", [(1, 32, 1024), (1, 128, 200), (2, 8, 2048), (1, 255, 100),
                                   (1, 256, 100)])
def test_rows_noncausal_from_256_tiles(gpu, oracle_mod, B, H, S):
    """Non-causal calls take the 128-row kernel from 256 tiles of 128 rows
    (one per CU) and the 64-row kernel below: both sides of the boundary,
    sampled heads against the oracle, and the call's bytes repeat."""
    log(f"non-causal B={B} H={H} S={S} routed={routed(B, H, S, causal=False)}")
    q, k, v = (rnd(37_000 + 13 * S + H + t, (B, H, S, D)) for t in range(3))
    sc = 1 / math.sqrt(D)
    o, lse = run(gpu, q, k, v, False, sc)
    sample_check(oracle_mod, q, k, v, o, lse, False, sc, f"non-causal B={B} H={H} S={S}", n_pick=3)
    o2, lse2 = run(gpu, q, k, v, False, sc)
    assert np.array_equal(o, o2) and np.array_equal(lse, lse2)
