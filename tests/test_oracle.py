"""Pins for the float64 oracle, checked against things other than itself:
exact-arithmetic brute force, closed forms and invariants of the softmax, and
PyTorch's own float64 SDPA on the CPU (the pages gate their kernels against
PyTorch SDPA: "An Optimal Mapper Meets a Real GPU", section "Ground rules").

Each pin is a function ``pin(impl) -> (ok, detail)`` over an implementation
``impl(q, k, v, causal, scale) -> (O, LSE)``, so the same pins are also run
against deliberately wrong variants of the oracle to show that every planted
mistake fails at least one of them.
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

from scaled_dot_product_attn_amd import inputs
from oracle import brute


def rnd(seed, shape, sigma=1.0):
    return inputs.normal_f16(seed, shape, sigma)


def torch_reference(q, k, v, causal, scale):
    """PyTorch float64 SDPA for O, torch.logsumexp over masked logits for LSE."""
    q64, k64, v64 = (torch.from_numpy(x.astype(np.float64)) for x in (q, k, v))
    sc = float(np.float32(scale))
    o = torch.nn.functional.scaled_dot_product_attention(
        q64, k64, v64, is_causal=bool(causal), scale=sc)
    s = sc * (q64 @ k64.transpose(-1, -2))
    if causal:
        S = q.shape[2]
        mask = torch.ones(S, S, dtype=torch.bool).triu(1)
        s = s.masked_fill(mask, float("-inf"))
    lse = torch.logsumexp(s, dim=-1)
    return o.numpy(), lse.numpy()


# --------------------------------------------------------------------- pins

def pin_brute_force(impl):
    """P5: agreement with exact-Fraction logits + fsum on tiny shapes."""
    worst = 0.0
    for seed, (B, H, S, D) in enumerate([(1, 1, 1, 1), (1, 3, 5, 4), (2, 1, 8, 8),
                                         (1, 2, 17, 2), (2, 3, 3, 8)]):
        q, k, v = (rnd(100 + 3 * seed + t, (B, H, S, D)) for t in range(3))
        for causal in (False, True):
            o, lse = impl(q, k, v, causal, 0.37)
            ob, lb = brute.attn_fwd(q, k, v, causal, 0.37)
            eo = np.max(np.abs(o - ob)) / max(1.0, np.max(np.abs(ob)))
            el = np.max(np.abs(lse - lb) / np.maximum(1.0, np.abs(lb)))
            worst = max(worst, eo, el)
    return worst < 1e-12, f"max rel err {worst:.3g}"


def pin_torch_sdpa(impl):
    """PyTorch float64 SDPA (a library routine the oracle does not use)."""
    worst = 0.0
    for seed, (B, H, S, D) in enumerate([(2, 3, 37, 16), (1, 2, 130, 64)]):
        q, k, v = (rnd(200 + 3 * seed + t, (B, H, S, D)) for t in range(3))
        for causal in (False, True):
            sc = 1 / math.sqrt(D)
            o, lse = impl(q, k, v, causal, sc)
            ot, lt = torch_reference(q, k, v, causal, sc)
            worst = max(worst, np.max(np.abs(o - ot)), np.max(np.abs(lse - lt)))
    return worst < 1e-11, f"max abs err {worst:.3g}"


def pin_value_identity_rows(impl):
    """P1: with V = I (S = D) the output is the probability matrix: rows sum
    to 1, entries are >= 0, and under causal masking the strict upper
    triangle is exactly 0."""
    worst = 0.0
    for S in (64, 128):
        q, k = rnd(300 + S, (1, 2, S, S)), rnd(301 + S, (1, 2, S, S))
        v = np.broadcast_to(np.eye(S, dtype=np.float16), (1, 2, S, S)).copy()
        for causal in (False, True):
            p, _ = impl(q, k, v, causal, 1 / math.sqrt(S))
            if np.any(p < 0):
                return False, "negative probability"
            worst = max(worst, np.max(np.abs(p.sum(-1) - 1.0)))
            if causal and np.any(np.triu(p[0, 0], 1) != 0.0):
                return False, "weight on a future key"
    return worst <= 1e-13, f"max |row sum - 1| {worst:.3g}"


def pin_causal_row_zero(impl):
    """P2: under causal masking row 0 sees only key 0, so O[0] = V[0] exactly
    and LSE[0] = scale * q0.k0 (evaluated exactly here, then rounded)."""
    q, k, v = (rnd(400 + t, (2, 3, 40, 32)) for t in range(3))
    sc = 0.125
    o, lse = impl(q, k, v, True, sc)
    if not np.array_equal(o[:, :, 0, :], v[:, :, 0, :].astype(np.float64)):
        return False, "O[0] != V[0]"
    worst = 0.0
    for b in range(2):
        for h in range(3):
            ex = Fraction(sc) * sum(Fraction(float(a)) * Fraction(float(c))
                                    for a, c in zip(q[b, h, 0], k[b, h, 0]))
            worst = max(worst, abs(lse[b, h, 0] - float(ex)))
    return worst <= 1e-12, f"LSE[0] err {worst:.3g}"


def pin_identical_keys(impl):
    """P3: with every key equal the weights are uniform over the visible
    keys: O is the mean of V (prefix mean if causal) and
    LSE_i = scale * q_i.k + ln(number of visible keys)."""
    B, H, S, D = 1, 2, 48, 16
    q, v = rnd(500, (B, H, S, D)), rnd(501, (B, H, S, D))
    krow = rnd(502, (B, H, 1, D))
    k = np.broadcast_to(krow, (B, H, S, D)).copy()
    sc = 0.3
    worst = 0.0
    for causal in (False, True):
        o, lse = impl(q, k, v, causal, sc)
        v64 = v.astype(np.float64)
        for i in range(S):
            n = i + 1 if causal else S
            mean = v64[:, :, :n, :].mean(axis=2)
            worst = max(worst, np.max(np.abs(o[:, :, i, :] - mean)))
            dot = (q[:, :, i, :].astype(np.float64) * krow[:, :, 0, :]).sum(-1)
            want = float(np.float32(sc)) * dot + math.log(n)
            worst = max(worst, np.max(np.abs(lse[:, :, i] - want)))
    return worst <= 1e-12, f"max err {worst:.3g}"


def pin_scale_zero(impl):
    """P4: scale = 0 makes every visible weight 1: O is the (prefix) mean of V
    and LSE = ln(number of visible keys), exactly."""
    B, H, S, D = 1, 3, 33, 8
    q, k, v = (rnd(600 + t, (B, H, S, D)) for t in range(3))
    worst = 0.0
    for causal in (False, True):
        o, lse = impl(q, k, v, causal, 0.0)
        for i in range(S):
            n = i + 1 if causal else S
            if np.any(lse[:, :, i] != math.log(n)):
                return False, f"LSE[{i}] != ln({n})"
            worst = max(worst, np.max(np.abs(o[:, :, i] - v[:, :, :n].astype(np.float64).mean(2))))
    return worst <= 1e-12, f"max err {worst:.3g}"


def pin_single_key(impl):
    """P8: S = 1 gives O = V and LSE = scale * q.k."""
    worst = 0.0
    for D in (64, 128, 512):
        q, k, v = (rnd(700 + D + t, (1, 2, 1, D)) for t in range(3))
        sc = 1 / math.sqrt(D)
        for causal in (False, True):
            o, lse = impl(q, k, v, causal, sc)
            if not np.array_equal(o, v.astype(np.float64)):
                return False, "O != V at S = 1"
            want = float(np.float32(sc)) * (q.astype(np.float64) * k).sum(-1)
            worst = max(worst, np.max(np.abs(lse - want)))
    return worst <= 1e-12, f"LSE err {worst:.3g}"


def pin_two_keys_logistic(impl):
    """Two keys, non-causal: the weight on key 0 is the logistic function of
    s0 - s1 (scipy.special.expit), and LSE = logaddexp(s0, s1)."""
    from scipy.special import expit
    q, k, v = (rnd(800 + t, (1, 4, 2, 8)) for t in range(3))
    sc = 0.7
    o, lse = impl(q, k, v, False, sc)
    q64, k64, v64 = (x.astype(np.float64) for x in (q, k, v))
    s = float(np.float32(sc)) * np.einsum("bhid,bhjd->bhij", q64, k64)
    w0 = expit(s[..., 0] - s[..., 1])
    want = w0[..., None] * v64[:, :, None, 0, :] + (1 - w0)[..., None] * v64[:, :, None, 1, :]
    e = max(np.max(np.abs(o - want)), np.max(np.abs(lse - np.logaddexp(s[..., 0], s[..., 1]))))
    return e <= 1e-12, f"err {e:.3g}"


PINS = [pin_brute_force, pin_torch_sdpa, pin_value_identity_rows,
        pin_causal_row_zero, pin_identical_keys, pin_scale_zero,
        pin_single_key, pin_two_keys_logistic]


@pytest.fixture(scope="module")
def impl(oracle_mod):
    return lambda q, k, v, causal, scale: oracle_mod.attn_fwd(q, k, v, causal, scale)


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_oracle_pin(pin, impl):
    ok, detail = pin(impl)
    assert ok, detail


@pytest.mark.parametrize("mistake", [1, 2, 3, 4, 5, 6])
def test_pins_catch_planted_mistake(mistake, oracle_mod):
    """Each planted mistake in the oracle fails at least one pin."""
    def wrong(q, k, v, causal, scale):
        return oracle_mod.attn_fwd(q, k, v, causal, scale, planted_mistake=mistake)
    failed = [p.__name__ for p in PINS if not p(wrong)[0]]
    assert failed, f"mistake {mistake} passed every pin"


# ------------------------------------------------------- more invariants

def test_half_to_double_exhaustive(oracle_mod):
    bits = np.arange(65536, dtype=np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([oracle_mod.half_to_double(int(b)) for b in bits])
    finite = np.isfinite(ref)
    assert np.array_equal(got[finite], ref[finite])
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    assert np.array_equal(got[np.isinf(ref)], ref[np.isinf(ref)])


def test_thread_count_invariance(oracle_mod):
    q, k, v = (rnd(900 + t, (2, 4, 96, 64)) for t in range(3))
    o1, l1 = oracle_mod.attn_fwd(q, k, v, True, 0.125, nthreads=1)
    o8, l8 = oracle_mod.attn_fwd(q, k, v, True, 0.125, nthreads=8)
    assert np.array_equal(o1, o8) and np.array_equal(l1, l8)


def test_future_independence(oracle_mod):
    """P10: changing keys/values after row i0 leaves rows <= i0 bit-identical."""
    q, k, v = (rnd(1000 + t, (1, 2, 64, 32)) for t in range(3))
    i0 = 40
    k2, v2 = k.copy(), v.copy()
    k2[:, :, i0 + 1:] = rnd(1003, k2[:, :, i0 + 1:].shape)
    v2[:, :, i0 + 1:] = rnd(1004, v2[:, :, i0 + 1:].shape)
    o, l = oracle_mod.attn_fwd(q, k, v, True, 0.2)
    o2, l2 = oracle_mod.attn_fwd(q, k2, v2, True, 0.2)
    assert np.array_equal(o[:, :, :i0 + 1], o2[:, :, :i0 + 1])
    assert np.array_equal(l[:, :, :i0 + 1], l2[:, :, :i0 + 1])
    assert not np.array_equal(o[:, :, i0 + 1:], o2[:, :, i0 + 1:])


def test_linearity_in_v(oracle_mod):
    """P13: O is linear in V.  Small-integer V keeps V1 + V2 exact in fp16."""
    q, k = rnd(1100, (1, 2, 50, 16)), rnd(1101, (1, 2, 50, 16))
    g = np.random.default_rng(1102)
    v1 = g.integers(-8, 9, (1, 2, 50, 16)).astype(np.float16)
    v2 = g.integers(-8, 9, (1, 2, 50, 16)).astype(np.float16)
    for causal in (False, True):
        oa, _ = oracle_mod.attn_fwd(q, k, v1, causal, 0.25)
        ob, _ = oracle_mod.attn_fwd(q, k, v2, causal, 0.25)
        oc, _ = oracle_mod.attn_fwd(q, k, (v1 + v2).astype(np.float16), causal, 0.25)
        assert np.max(np.abs(oc - (oa + ob))) < 1e-12


def test_key_permutation_equivariance(oracle_mod):
    """P13: non-causal attention does not depend on the order of the keys."""
    q, k, v = (rnd(1200 + t, (1, 2, 64, 32)) for t in range(3))
    perm = np.random.default_rng(1203).permutation(64)
    o, l = oracle_mod.attn_fwd(q, k, v, False, 0.2)
    o2, l2 = oracle_mod.attn_fwd(q, k[:, :, perm], v[:, :, perm], False, 0.2)
    assert np.max(np.abs(o - o2)) < 1e-12 and np.max(np.abs(l - l2)) < 1e-12


def test_large_logits_stay_finite(oracle_mod):
    """P12: scale = 8/sqrt(D) gives logit spreads of tens; subtracting the row
    max keeps every exp finite."""
    q, k, v = (rnd(1300 + t, (1, 2, 128, 128)) for t in range(3))
    sc = 8 / math.sqrt(128)
    o, l = oracle_mod.attn_fwd(q, k, v, True, sc)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(l))
    ot, lt = torch_reference(q, k, v, True, sc)
    assert np.max(np.abs(o - ot)) < 1e-10 and np.max(np.abs(l - lt)) < 1e-10


def test_logits_match_exact_and_subtiles_add(oracle_mod):
    """P6: full-width logits equal the exact ones; the two half-width sub-tile
    logits S_0 (d < D/2) and S_1 (d >= D/2) add to S in logit space (the
    head-dim-512 notes, lesson "2. External k_sub Merge is Mathematically
    Impossible" and "6. The k_tile Parameter")."""
    q, k = rnd(1400, (1, 1, 6, 8)), rnd(1401, (1, 1, 6, 8))
    ex = brute.exact_logits(q[0, 0], k[0, 0], 0.5, True)
    s = oracle_mod.logits(q, k, True, 0.5)
    for i in range(6):
        for j in range(6):
            if ex[i][j] is None:
                assert s[0, 0, i, j] == -np.inf
            else:
                assert abs(s[0, 0, i, j] - float(ex[i][j])) <= 1e-15 * max(1, abs(float(ex[i][j])))
    # exact sub-tile sums (Fractions): S_0 + S_1 == S with no rounding at all
    qa, kb = brute._exact(q[0, 0]), brute._exact(k[0, 0])
    for i in range(6):
        for j in range(i + 1):
            s0 = sum(a * b for a, b in zip(qa[i][:4], kb[j][:4]))
            s1 = sum(a * b for a, b in zip(qa[i][4:], kb[j][4:]))
            assert Fraction(0.5) * (s0 + s1) == ex[i][j]


def test_head_dim_512_subtile_logits(oracle_mod):
    """P6 at the head-dim-512 workload's inputs (first two heads)."""
    w = inputs.WORKLOADS[5]
    q, k, _ = w.qkv()
    q, k = q[:, :2, :256], k[:, :2, :256]
    s = oracle_mod.logits(q, k, True, w.scale)
    s0 = oracle_mod.logits(q, k, True, w.scale, 0, 256)
    s1 = oracle_mod.logits(q, k, True, w.scale, 256, 512)
    vis = np.isfinite(s)
    assert np.array_equal(vis, np.isfinite(s0)) and np.array_equal(vis, np.isfinite(s1))
    bound = 1e-13 * w.scale * np.einsum("bhid,bhjd->bhij", np.abs(q.astype(np.float64)),
                                         np.abs(k.astype(np.float64)))
    assert np.all(np.abs(s0[vis] + s1[vis] - s[vis]) <= bound[vis] + 1e-300)


def test_wrong_merge_negative_control(oracle_mod):
    """P7: merging softmax(S_0)V and softmax(S_1)V with the LSE-weighted
    formula for disjoint key sets does NOT give softmax(S_0 + S_1)V.  The
    difference is far above the 2e-2 gate, so parity tests would catch a
    kernel that merged sub-tiles after the softmax."""
    w = inputs.WORKLOADS[5]
    q, k, v = w.qkv()
    q, k, v = q[:, :2, :512], k[:, :2, :512], v[:, :2, :512]
    o_ref, l_ref = oracle_mod.attn_fwd(q, k, v, True, w.scale)
    s0 = oracle_mod.logits(q, k, True, w.scale, 0, 256)
    s1 = oracle_mod.logits(q, k, True, w.scale, 256, 512)
    o0, l0 = oracle_mod.softmax_av(s0, v)
    o1, l1 = oracle_mod.softmax_av(s1, v)
    # the same oracle from full-width logits agrees with the direct path
    o_full, l_full = oracle_mod.softmax_av(oracle_mod.logits(q, k, True, w.scale), v)
    assert np.max(np.abs(o_full - o_ref)) < 1e-12 and np.max(np.abs(l_full - l_ref)) < 1e-12
    mx = np.maximum(l0, l1)
    a0, a1 = np.exp(l0 - mx), np.exp(l1 - mx)
    o_wrong = (a0[..., None] * o0 + a1[..., None] * o1) / (a0 + a1)[..., None]
    l_wrong = mx + np.log(a0 + a1)
    # the parity gate (|d| <= 2e-2 + 2e-2 |ref| on O, 1e-3 max(1,|ref|) on LSE)
    viol = np.abs(o_wrong - o_ref) > 2e-2 + 2e-2 * np.abs(o_ref)
    assert viol.sum() > 1000 and np.max(np.abs(o_wrong - o_ref)) > 5 * 2e-2
    assert np.max(np.abs(l_wrong - l_ref) / np.maximum(1, np.abs(l_ref))) > 100 * 1e-3
