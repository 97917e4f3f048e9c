"""GPU parity: the HIP path (through the C ABI) against the float64 oracle on
the same seeded inputs.

Gate (the pages' own, "An Optimal Mapper Meets a Real GPU", section "Ground
rules": FP16 in / FP32 accumulate, atol = rtol = 2e-2 against a reference
SDPA), applied element-wise in allclose form:
    O   : |O_gpu - O_ref|     <= 2e-2 + 2e-2 |O_ref|
    LSE : |LSE_gpu - LSE_ref| <= 1e-3 max(1, |LSE_ref|)
The reference is unrounded float64.
"""
import math
import sys

import numpy as np
import pytest

from scaled_dot_product_attn_amd import inputs

pytestmark = pytest.mark.gpu

O_TOL = 2e-2
LSE_TOL = 1e-3


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def to_dev(x):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def run(gpu, q, k, v, causal, scale, unfused=False):
    import torch
    fn = gpu.fwd_unfused if unfused else gpu.fwd
    o, lse = fn(to_dev(q), to_dev(k), to_dev(v), causal=causal, scale=scale)
    torch.cuda.synchronize()
    return o.cpu().numpy(), lse.cpu().numpy()


def check(o, lse, o_ref, l_ref, what=""):
    o64 = o.astype(np.float64)
    assert np.all(np.isfinite(o64)) and np.all(np.isfinite(lse)), f"{what}: non-finite output"
    d_o = np.abs(o64 - o_ref)
    bad_o = d_o > O_TOL + O_TOL * np.abs(o_ref)
    d_l = np.abs(lse.astype(np.float64) - l_ref)
    bad_l = d_l > LSE_TOL * np.maximum(1.0, np.abs(l_ref))
    log(f"{what}: max|dO| {d_o.max():.3g}  max|dLSE| {d_l.max():.3g}  "
        f"violations O {int(bad_o.sum())} LSE {int(bad_l.sum())}")
    assert not bad_o.any(), f"{what}: {int(bad_o.sum())} O violations, max {d_o.max():.3g}"
    assert not bad_l.any(), f"{what}: {int(bad_l.sum())} LSE violations, max {d_l.max():.3g}"


def rnd(seed, shape, sigma=1.0):
    return inputs.normal_f16(seed, shape, sigma)


# ------------------------------------------------------------ the workloads

@pytest.mark.parametrize("c", [1, 2, 3, 4, 5])
def test_workload_parity(gpu, oracle_mod, c):
    w = inputs.WORKLOADS[c]
    log(f"workload {c} {w.name}")
    q, k, v = w.qkv()
    o, lse = run(gpu, q, k, v, w.causal, w.scale)
    o_ref, l_ref = oracle_mod.attn_fwd(q, k, v, w.causal, w.scale)
    check(o, lse, o_ref, l_ref, w.name)


# ------------------------------------------------------- ragged and tiny S

RAGGED = [1, 2, 3, 17, 31, 33, 63, 64, 65, 127, 128, 129, 200, 257, 300]


@pytest.mark.parametrize("D", [64, 128, 512])
@pytest.mark.parametrize("causal", [False, True])
def test_ragged_lengths(gpu, oracle_mod, D, causal):
    for S in RAGGED:
        if D == 512 and S > 129:
            continue
        log(f"ragged D={D} causal={causal} S={S}")
        shape = (1, 2, S, D)
        q, k, v = (rnd(10_000 + 7 * S + D + t, shape) for t in range(3))
        sc = 1 / math.sqrt(D)
        o, lse = run(gpu, q, k, v, causal, sc)
        o_ref, l_ref = oracle_mod.attn_fwd(q, k, v, causal, sc)
        check(o, lse, o_ref, l_ref, f"S={S} D={D} causal={causal}")


@pytest.mark.parametrize("D", [64, 128, 512])
def test_batch_heads_layout(gpu, oracle_mod, D):
    """Several batches and heads, odd S: every (b, h) slice lands in place."""
    shape = (3, 5, 77, D)
    q, k, v = (rnd(11_000 + D + t, shape) for t in range(3))
    for causal in (False, True):
        o, lse = run(gpu, q, k, v, causal, 0.1)
        o_ref, l_ref = oracle_mod.attn_fwd(q, k, v, causal, 0.1)
        check(o, lse, o_ref, l_ref, f"B3 H5 S77 D{D} causal={causal}")


@pytest.mark.parametrize("B,H,S", [(1, 2, 300), (2, 3, 449), (1, 4, 1000), (1, 1, 65),
                                   (1, 3, 576)])
def test_d512_causal_tile_counts(gpu, oracle_mod, B, H, S):
    """D = 512 causal at odd and even counts of 64-row query tiles, ragged
    last tiles and several heads: every row against the oracle, and the
    call's bytes repeat."""
    shape = (B, H, S, 512)
    q, k, v = (rnd(13_000 + S + H + t, shape) for t in range(3))
    sc = 1 / math.sqrt(512)
    log(f"D=512 causal B={B} H={H} S={S}")
    o, lse = run(gpu, q, k, v, True, sc)
    o_ref, l_ref = oracle_mod.attn_fwd(q, k, v, True, sc)
    check(o, lse, o_ref, l_ref, f"D=512 causal B={B} H={H} S={S}")
    o2, lse2 = run(gpu, q, k, v, True, sc)
    assert np.array_equal(o, o2) and np.array_equal(lse, lse2)


def test_d512_many_tiles(gpu, oracle_mod):
    """D = 512 fused with at least 256 tiles of 64 rows (B2 H8 S1024, causal
    and not): the 64-row, four-wave form (fewer tiles take 32-row tiles of
    two waves); sampled heads against the oracle, and the bytes equal a
    split-KV call with one split (the same kernel, one chunk per tile)."""
    import torch
    B, H, S, D = 2, 8, 1024, 512
    assert B * H * (S // 64) >= 256
    q, k, v = (rnd(14_000 + t, (B, H, S, D), 0.5) for t in range(3))
    sc = float(np.float32(1 / math.sqrt(D)))
    for causal in (True, False):
        log(f"D=512 many tiles causal={causal}")
        o, lse = run(gpu, q, k, v, causal, sc)
        for b, h in ((0, 0), (1, 7), (1, 3)):
            sl = (slice(b, b + 1), slice(h, h + 1))
            o_ref, l_ref = oracle_mod.attn_fwd(q[sl], k[sl], v[sl], causal, sc)
            check(o[sl], lse[sl], o_ref, l_ref, f"D=512 B2 H8 S1024 causal={causal} b={b} h={h}")
        o1, l1 = gpu.fwd_splitkv(to_dev(q), to_dev(k), to_dev(v), causal=causal, scale=sc,
                                 splits=1)
        torch.cuda.synchronize()
        assert np.array_equal(o1.cpu().numpy(), o) and np.array_equal(l1.cpu().numpy(), lse)


# ---------------------------------- grids of more than one wave of workgroups

# More 64-row query tiles than 2 x 256 (two workgroups on each of the 256
# CUs), so that workgroups start as others finish.  Cases: one tile per head,
# odd tile counts, B*H a multiple of 8 and not, both head dims, both masks,
# ragged S.
MULTIWAVE = [
    (1, 520, 64, 64, False),
    (1, 520, 64, 128, True),
    (3, 7, 1590, 64, False),
    (2, 16, 1030, 128, True),
    (1, 24, 1400, 64, True),
    (1, 40, 900, 128, False),
]


@pytest.mark.parametrize("B,H,S,D,causal", MULTIWAVE)
def test_multiwave_grids(gpu, oracle_mod, B, H, S, D, causal):
    assert B * H * ((S + 63) // 64) > 512
    shape = (B, H, S, D)
    seed = 12_000 + S + D + H
    q, k, v = (rnd(seed + t, shape) for t in range(3))
    sc = 1 / math.sqrt(D)
    log(f"multi-wave B={B} H={H} S={S} D={D} causal={causal}")
    o, lse = run(gpu, q, k, v, causal, sc)
    # heads are independent: the oracle checks a sample of (batch, head) pairs
    picks = sorted({(0, 0), (B - 1, H - 1), (B // 2, H // 2), (0, H - 1), (B - 1, 0)})
    if S <= 64:
        picks = [(b, h) for b in range(B) for h in range(H)]
    for b, h in picks:
        sl = (slice(b, b + 1), slice(h, h + 1))
        o_ref, l_ref = oracle_mod.attn_fwd(q[sl], k[sl], v[sl], causal, sc)
        check(o[sl], lse[sl], o_ref, l_ref, f"multi-wave {shape} causal={causal} b={b} h={h}")


def test_multiwave_repeat_bit_identical(gpu):
    shape = (2, 16, 1030, 128)
    q, k, v = (rnd(12_500 + t, shape) for t in range(3))
    o1, l1 = run(gpu, q, k, v, True, 0.088)
    o2, l2 = run(gpu, q, k, v, True, 0.088)
    assert inputs.sha256(o1) == inputs.sha256(o2)
    assert inputs.sha256(l1) == inputs.sha256(l2)


# ------------------------------------------------------------------ the pins

@pytest.mark.parametrize("S", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_value_identity_gives_probabilities(gpu, S, causal):
    """P1: V = I makes O the probability matrix: rows sum to 1 (within fp16
    rounding of P and O), entries >= 0, future keys exactly 0."""
    q, k = rnd(12_000 + S, (1, 2, S, S)), rnd(12_001 + S, (1, 2, S, S))
    v = np.broadcast_to(np.eye(S, dtype=np.float16), (1, 2, S, S)).copy()
    p, _ = run(gpu, q, k, v, causal, 1 / math.sqrt(S))
    p = p.astype(np.float64)
    assert np.all(p >= 0)
    assert np.max(np.abs(p.sum(-1) - 1.0)) <= S * 2.0 ** -11 + O_TOL
    if causal:
        for h in range(2):
            assert np.all(np.triu(p[0, h], 1) == 0.0)


def test_causal_row_zero_is_v0(gpu):
    """P2: under causal masking row 0 sees key 0 only: O[0] = V[0] bit-exact,
    LSE[0] = scale q0.k0."""
    for D in (64, 128, 512):
        q, k, v = (rnd(13_000 + D + t, (2, 3, 96, D)) for t in range(3))
        sc = 1 / math.sqrt(D)
        o, lse = run(gpu, q, k, v, True, sc)
        assert np.array_equal(o[:, :, 0, :], v[:, :, 0, :]), f"D={D}"
        want = float(np.float32(sc)) * (q[:, :, 0].astype(np.float64) * k[:, :, 0]).sum(-1)
        assert np.max(np.abs(lse[:, :, 0] - want)) <= LSE_TOL * max(1.0, np.max(np.abs(want)))


def test_identical_keys_give_mean(gpu, oracle_mod):
    """P3: every key equal -> O is the mean of V (prefix mean when causal)."""
    for D in (64, 128, 512):
        B, H, S = 1, 2, 160
        q, v = rnd(14_000 + D, (B, H, S, D)), rnd(14_001 + D, (B, H, S, D))
        k = np.broadcast_to(rnd(14_002 + D, (B, H, 1, D)), (B, H, S, D)).copy()
        for causal in (False, True):
            o, lse = run(gpu, q, k, v, causal, 1 / math.sqrt(D))
            v64 = v.astype(np.float64)
            n = np.arange(1, S + 1) if causal else np.full(S, S)
            mean = (np.cumsum(v64, axis=2) / n[:, None]) if causal else \
                np.broadcast_to(v64.mean(2, keepdims=True), v64.shape)
            check(o, lse, mean, oracle_mod.attn_fwd(q, k, v, causal, 1 / math.sqrt(D))[1],
                  f"identical keys D={D} causal={causal}")


def test_scale_zero(gpu):
    """P4: scale = 0 -> uniform weights: O = (prefix) mean of V, LSE = ln(n)."""
    for D in (64, 128, 512):
        B, H, S = 1, 2, 130
        q, k, v = (rnd(15_000 + D + t, (B, H, S, D)) for t in range(3))
        for causal in (False, True):
            o, lse = run(gpu, q, k, v, causal, 0.0)
            v64 = v.astype(np.float64)
            n = np.arange(1, S + 1) if causal else np.full(S, S)
            mean = (np.cumsum(v64, axis=2) / n[:, None]) if causal else \
                np.broadcast_to(v64.mean(2, keepdims=True), v64.shape)
            l_ref = np.broadcast_to(np.log(n), lse.shape)
            check(o, lse, mean, l_ref, f"scale 0 D={D} causal={causal}")


def test_single_key(gpu):
    """P8: S = 1 -> O = V, LSE = scale q.k."""
    for D in (64, 128, 512):
        q, k, v = (rnd(16_000 + D + t, (1, 2, 1, D)) for t in range(3))
        sc = 1 / math.sqrt(D)
        for causal in (False, True):
            o, lse = run(gpu, q, k, v, causal, sc)
            assert np.array_equal(o, v)
            want = float(np.float32(sc)) * (q.astype(np.float64) * k).sum(-1)
            assert np.max(np.abs(lse - want)) <= LSE_TOL


@pytest.mark.parametrize("D", [64, 128, 512])
def test_head_dim_coverage(gpu, oracle_mod, D):
    """P9: Q and K zero on one half of the head dim and random on the other
    (then the mirror image).  A kernel that drops part of the head dim in
    Q K^T fails by far more than the tolerance (the STAGE_D.md notes describe
    exactly such a bug: only 64 of 128+ dims entered the QK product)."""
    B, H, S = 1, 2, 192
    for half in (0, 1):
        q, k, v = (rnd(17_000 + D + 10 * half + t, (B, H, S, D)) for t in range(3))
        lo, hi = (slice(0, D // 2), slice(D // 2, D)) if half == 0 else \
            (slice(D // 2, D), slice(0, D // 2))
        q[..., lo] = 0
        k[..., lo] = 0
        sc = 2 / math.sqrt(D)
        o, lse = run(gpu, q, k, v, True, sc)
        o_ref, l_ref = oracle_mod.attn_fwd(q, k, v, True, sc)
        check(o, lse, o_ref, l_ref, f"coverage D={D} half={half}")


def test_future_independence(gpu):
    """P10: changing K, V rows after i0 leaves rows <= i0 bit-identical."""
    for D in (64, 128, 512):
        q, k, v = (rnd(18_000 + D + t, (1, 2, 300, D)) for t in range(3))
        i0 = 137
        k2, v2 = k.copy(), v.copy()
        k2[:, :, i0 + 1:] = rnd(18_100 + D, k2[:, :, i0 + 1:].shape)
        v2[:, :, i0 + 1:] = rnd(18_200 + D, v2[:, :, i0 + 1:].shape)
        o, lse = run(gpu, q, k, v, True, 1 / math.sqrt(D))
        o2, lse2 = run(gpu, q, k2, v2, True, 1 / math.sqrt(D))
        assert np.array_equal(o[:, :, :i0 + 1], o2[:, :, :i0 + 1])
        assert np.array_equal(lse[:, :, :i0 + 1], lse2[:, :, :i0 + 1])


def test_slice_consistency(gpu):
    """P11: one (b, h) launched alone equals its slice of the full call,
    bit-exact."""
    for D in (64, 128, 512):
        q, k, v = (rnd(19_000 + D + t, (2, 3, 200, D)) for t in range(3))
        for causal in (False, True):
            o, lse = run(gpu, q, k, v, causal, 1 / math.sqrt(D))
            o1, l1 = run(gpu, q[1:2, 2:3], k[1:2, 2:3], v[1:2, 2:3], causal, 1 / math.sqrt(D))
            assert np.array_equal(o[1:2, 2:3], o1) and np.array_equal(lse[1:2, 2:3], l1)


def test_linearity_in_v_and_key_permutation(gpu):
    """P13 on the GPU: O is linear in V for fixed Q, K (the probabilities do
    not depend on V), and permuting the key/value rows jointly leaves a
    non-causal result unchanged; both within the parity tolerance (the GPU
    rounds P and O to fp16, and the sums run in a different order)."""
    for D in (64, 128, 512):
        shape = (1, 2, 190, D)
        q, k = (rnd(19_500 + D + t, shape) for t in range(2))
        # V1 and V2 on the grid 2^-8 within [-4, 4], so that V1 + V2 (grid 2^-8
        # within [-8, 8], 11 significant bits) is exact in fp16
        def grid(seed):
            x = rnd(seed, shape).astype(np.float64)
            return np.clip(np.round(x * 256) / 256, -4, 4).astype(np.float16)
        v1, v2 = grid(19_600 + D), grid(19_700 + D)
        v12 = (v1.astype(np.float32) + v2.astype(np.float32)).astype(np.float16)
        assert np.array_equal(v12.astype(np.float32), v1.astype(np.float32) + v2.astype(np.float32))
        sc = 1 / math.sqrt(D)
        for causal in (False, True):
            o1, l1 = run(gpu, q, k, v1, causal, sc)
            o2, l2 = run(gpu, q, k, v2, causal, sc)
            o12, l12 = run(gpu, q, k, v12, causal, sc)
            lhs = o12.astype(np.float64)
            rhs = o1.astype(np.float64) + o2.astype(np.float64)
            assert np.all(np.abs(lhs - rhs) <= O_TOL + O_TOL * np.abs(rhs)), f"linearity D={D}"
            # the log-sum-exp does not see V at all
            assert np.array_equal(l1, l2) and np.array_equal(l1, l12)
        perm = np.random.default_rng(19_800 + D).permutation(shape[2])
        o, l = run(gpu, q, k, v1, False, sc)
        op, lp = run(gpu, q, k[:, :, perm], v1[:, :, perm], False, sc)
        assert np.all(np.abs(op.astype(np.float64) - o) <= O_TOL + O_TOL * np.abs(o))
        assert np.all(np.abs(lp.astype(np.float64) - l) <= LSE_TOL * np.maximum(1, np.abs(l)))


def test_large_logits(gpu, oracle_mod):
    """P12: scale = 8/sqrt(D) (logit spreads of tens): finite and in parity."""
    for D in (64, 128, 512):
        q, k, v = (rnd(20_000 + D + t, (1, 2, 256, D)) for t in range(3))
        sc = 8 / math.sqrt(D)
        for causal in (False, True):
            o, lse = run(gpu, q, k, v, causal, sc)
            o_ref, l_ref = oracle_mod.attn_fwd(q, k, v, causal, sc)
            check(o, lse, o_ref, l_ref, f"large logits D={D} causal={causal}")


def test_negative_scale(gpu, oracle_mod):
    for D in (64, 128, 512):
        q, k, v = (rnd(21_000 + D + t, (1, 2, 150, D)) for t in range(3))
        for causal in (False, True):
            o, lse = run(gpu, q, k, v, causal, -0.2)
            o_ref, l_ref = oracle_mod.attn_fwd(q, k, v, causal, -0.2)
            check(o, lse, o_ref, l_ref, f"negative scale D={D} causal={causal}")


def test_repeat_runs_bit_identical(gpu):
    """Determinism: the same inputs give the same output bytes."""
    w = inputs.WORKLOADS[3]
    q, k, v = w.qkv()
    o1, l1 = run(gpu, q, k, v, w.causal, w.scale)
    o2, l2 = run(gpu, q, k, v, w.causal, w.scale)
    assert inputs.sha256(o1) == inputs.sha256(o2)
    assert inputs.sha256(l1) == inputs.sha256(l2)
