"""GPU parity of the backward (dQ, dK, dV of sum(dO * O)) against the float64
oracle on the same seeded inputs.

The GPU backward consumes the GPU forward's O (fp16) and LSE; the oracle
recomputes everything in float64 from Q, K, V and dO alone.

Gate.  The pages give no tolerance for gradients; this one follows from the
arithmetic.  The kernels round P and dS to fp16 before the products that use
them and round the results to fp16, each a relative error of at most
u = 2^-11; dO.O uses the fp16 O.  Summed over the rows of a product these
errors stay within a few u of each output's magnitude, so per tensor X:
    element-wise : |X_gpu - X_ref| <= 2e-2 |X_ref| + 2e-2 rms(X_ref)
    tensor-wise  : ||X_gpu - X_ref||_F <= 5e-3 ||X_ref||_F      (about 10 u)
The element-wise form is the forward's atol = rtol = 2e-2 with atol scaled by
the tensor's RMS, since gradients are not of unit size.
"""
import numpy as np
import pytest

from scaled_dot_product_attn_amd import inputs
from test_parity import log, rnd, to_dev

pytestmark = pytest.mark.gpu

EL_TOL = 2e-2
FRO_TOL = 5e-3


def run_bwd(gpu, q, k, v, do, causal, scale):
    import torch
    qd, kd, vd, dod = (to_dev(x) for x in (q, k, v, do))
    o, lse = gpu.fwd(qd, kd, vd, causal=causal, scale=scale)
    dq, dk, dv = gpu.bwd(qd, kd, vd, o, lse, dod, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return tuple(t.cpu().numpy() for t in (dq, dk, dv))


def check_grads(got, ref, what, zero_bound=0.0):
    """zero_bound: the largest |X_gpu| accepted where the reference tensor is
    identically zero (only fp32 rounding remains there)."""
    for name, x, r in zip(("dQ", "dK", "dV"), got, ref):
        x64 = x.astype(np.float64)
        assert np.all(np.isfinite(x64)), f"{what} {name}: non-finite output"
        if not r.any():
            log(f"{what} {name}: reference is zero, max|X| {np.abs(x64).max():.3g}")
            assert np.all(np.abs(x64) <= zero_bound), f"{what} {name}: max {np.abs(x64).max()}"
            continue
        d = np.abs(x64 - r)
        rms = float(np.sqrt(np.mean(r * r)))
        bad = d > EL_TOL * np.abs(r) + EL_TOL * rms
        fro = float(np.linalg.norm(d) / max(np.linalg.norm(r), 1e-300))
        log(f"{what} {name}: rms {rms:.3g} max|d| {d.max():.3g} rel-fro {fro:.3g} "
            f"violations {int(bad.sum())}")
        assert not bad.any(), f"{what} {name}: {int(bad.sum())} violations, max {d.max():.3g}"
        if rms > 0:
            assert fro <= FRO_TOL, f"{what} {name}: relative Frobenius error {fro:.3g}"


def problem(seed, B, H, S, D, sigma=1.0):
    return tuple(rnd(seed + t, (B, H, S, D), sigma) for t in range(4))


@pytest.mark.parametrize("B,H,S,D,causal", [
    (1, 2, 200, 64, True), (1, 2, 200, 128, True), (2, 2, 129, 128, False),
    (1, 3, 64, 64, False), (1, 1, 1, 128, True), (1, 1, 1, 64, False),
    (1, 2, 257, 64, False), (1, 1, 33, 128, True), (2, 1, 320, 128, True),
    (1, 2, 65, 64, True),
    # D = 512: the materialised form (S, dP, dS, P^T, dS^T in the workspace)
    (1, 2, 200, 512, True), (1, 1, 129, 512, False), (2, 1, 64, 512, True),
    (1, 1, 1, 512, True), (1, 1, 33, 512, False)])
def test_bwd_small(gpu, oracle_mod, B, H, S, D, causal):
    seed = 70_000 + 97 * S + D + int(causal)
    q, k, v, do = problem(seed, B, H, S, D)
    scale = 1.0 / np.sqrt(D)
    log(f"bwd small B={B} H={H} S={S} D={D} causal={causal} seed={seed}")
    got = run_bwd(gpu, q, k, v, do, causal, scale)
    ref = oracle_mod.attn_bwd(q, k, v, do, causal, scale)
    zero_bound = 0.0
    if S == 1:
        # One key: P = 1, so dS = dO.v - dO.O = 0 exactly (O = v), and dQ = dK = 0.
        # The kernels form both dot products in fp32 in different orders, so
        # |dS| <= 2 D 2^-24 sum|dO * v| and |dQ| <= scale |dS| max|k|.
        f = [x.astype(np.float64) for x in (q, k, v, do)]
        ds = 2 * D * 2.0 ** -24 * np.abs(f[3] * f[2]).sum()
        zero_bound = scale * ds * max(np.abs(f[1]).max(), np.abs(f[0]).max())
    check_grads(got, ref, f"S={S} D={D} causal={causal}", zero_bound)


@pytest.mark.parametrize("c", [1, 2, 3, 4, 5])
def test_bwd_workload_shapes(gpu, oracle_mod, c):
    """The forward workloads' shapes and inputs, with dO drawn like Q; the GPU
    runs the full problem and the oracle checks a sample of (batch, head)
    pairs (heads are independent, so slicing the inputs is exact)."""
    w = inputs.WORKLOADS[c]
    q, k, v = w.qkv()
    do = rnd(w.seed_base + 50, q.shape)
    log(f"bwd workload {w.name}")
    got = run_bwd(gpu, q, k, v, do, w.causal, w.scale)
    B, H = q.shape[:2]
    picks = sorted({(0, 0), (B - 1, H - 1), (B // 2, H // 3), (0, H - 1)})
    for b, h in picks:
        sl = (slice(b, b + 1), slice(h, h + 1))
        ref = oracle_mod.attn_bwd(q[sl], k[sl], v[sl], do[sl], w.causal, w.scale)
        check_grads(tuple(g[sl] for g in got), ref, f"{w.name} b={b} h={h}")


@pytest.mark.parametrize("scale", [-0.2, 0.0, 0.4])
def test_bwd_scales(gpu, oracle_mod, scale):
    """A negative scale (applied by flipping signs), a zero scale (uniform P,
    dQ = dK = 0 exactly) and a large one (peaked rows)."""
    q, k, v, do = problem(71_000, 1, 2, 190, 128)
    log(f"bwd scale={scale}")
    got = run_bwd(gpu, q, k, v, do, True, scale)
    ref = oracle_mod.attn_bwd(q, k, v, do, True, scale)
    if scale == 0.0:
        assert not got[0].any() and not got[1].any()
        x, r = got[2].astype(np.float64), ref[2]
        assert np.all(np.abs(x - r) <= EL_TOL * np.abs(r) + EL_TOL * np.sqrt(np.mean(r * r)))
    else:
        check_grads(got, ref, f"scale={scale}")


def test_bwd_dk_sums_to_zero(gpu):
    """Every row of dS sums to zero (sum_j P_ij dP_ij = dO_i . O_i), so the key
    gradients of a head sum to zero: a property that holds at any size, here
    B=1 H=32 S=1024 D=128 causal in full."""
    w = inputs.WORKLOADS[3]
    q, k, v = w.qkv()
    do = rnd(w.seed_base + 50, q.shape)
    _, dk, _ = run_bwd(gpu, q, k, v, do, w.causal, w.scale)
    dk = dk.astype(np.float64)
    tot = np.abs(dk.sum(axis=2))            # [B, H, D]
    mag = np.abs(dk).sum(axis=2)
    log(f"sum_j dK_j: max {tot.max():.3g}, relative to sum|dK| {float((tot / mag).max()):.3g}")
    assert np.all(tot <= 5e-3 * mag)


@pytest.mark.parametrize("D", [64, 512])
def test_bwd_repeat_is_bit_identical(gpu, D):
    q, k, v, do = problem(72_000, 2, 3, 300, D)
    a = run_bwd(gpu, q, k, v, do, True, 0.125)
    b = run_bwd(gpu, q, k, v, do, True, 0.125)
    for x, y in zip(a, b):
        assert np.array_equal(x.view(np.uint16), y.view(np.uint16))


def test_bwd_d512_dk_sums_to_zero(gpu):
    """The zero-sum property of the key gradients at workload 5's shape
    (B=1 H=8 S=1024 D=512 causal) in full."""
    w = inputs.WORKLOADS[5]
    q, k, v = w.qkv()
    do = rnd(w.seed_base + 50, q.shape)
    _, dk, _ = run_bwd(gpu, q, k, v, do, w.causal, w.scale)
    dk = dk.astype(np.float64)
    tot = np.abs(dk.sum(axis=2))
    mag = np.abs(dk).sum(axis=2)
    log(f"D=512 sum_j dK_j: relative to sum|dK| {float((tot / mag).max()):.3g}")
    assert np.all(tot <= 5e-3 * mag)
