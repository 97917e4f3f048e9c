"""Pins for the oracle's backward pass (gradients of sum(dO * O) with respect
to q, k and v).  CPU only.

- PyTorch's float64 autograd through its SDPA (an independent implementation
  of the same definition);
- translation invariance: adding one vector to every key shifts each row's
  logits uniformly, so the key gradients sum to zero, sum_j dK[j] = 0;
- scale = 0: dQ = dK = 0 exactly and dV[j] = sum_{i sees j} dO[i] / n_i, with
  n_i the visible keys of row i;
- each planted mistake fails the autograd pin.
"""
import numpy as np
import pytest
import torch

from scaled_dot_product_attn_amd import inputs


def problem(seed, B, H, S, D, sigma=1.0):
    return tuple(inputs.normal_f16(seed + t, (B, H, S, D), sigma) for t in range(4))


def autograd(q, k, v, do, causal, scale):
    Q, K, V = (torch.from_numpy(x.astype(np.float64)).requires_grad_() for x in (q, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(
        Q, K, V, is_causal=causal, scale=float(np.float32(scale)))
    (o * torch.from_numpy(do.astype(np.float64))).sum().backward()
    return Q.grad.numpy(), K.grad.numpy(), V.grad.numpy()


@pytest.mark.parametrize("B,H,S,D", [(1, 1, 1, 4), (1, 2, 7, 8), (2, 1, 33, 16), (1, 2, 100, 64)])
@pytest.mark.parametrize("causal", [False, True])
def test_backward_matches_torch_autograd(oracle_mod, B, H, S, D, causal):
    q, k, v, do = problem(5000 + S + D, B, H, S, D)
    scale = 1 / np.sqrt(D)
    got = oracle_mod.attn_bwd(q, k, v, do, causal, scale)
    ref = autograd(q, k, v, do, causal, scale)
    for name, a, b in zip(("dq", "dk", "dv"), got, ref):
        assert np.allclose(a, b, rtol=1e-10, atol=1e-12), name


@pytest.mark.parametrize("causal", [False, True])
def test_key_gradients_sum_to_zero(oracle_mod, causal):
    q, k, v, do = problem(5100, 2, 2, 90, 32)
    _, dk, _ = oracle_mod.attn_bwd(q, k, v, do, causal, 0.3)
    tot = dk.sum(axis=2)
    assert np.all(np.abs(tot) <= 1e-12 * np.abs(dk).sum(axis=2) + 1e-300)


@pytest.mark.parametrize("causal", [False, True])
def test_scale_zero_closed_form(oracle_mod, causal):
    B, H, S, D = 1, 2, 40, 8
    q, k, v, do = problem(5200, B, H, S, D)
    dq, dk, dv = oracle_mod.attn_bwd(q, k, v, do, causal, 0.0)
    assert np.all(dq == 0) and np.all(dk == 0)
    g = do.astype(np.float64)
    expect = np.zeros_like(dv)
    for i in range(S):
        n = i + 1 if causal else S
        expect[:, :, :n] += g[:, :, i:i + 1] / n
    assert np.allclose(dv, expect, rtol=1e-13, atol=1e-15)


def test_thread_count_invariance(oracle_mod):
    q, k, v, do = problem(5300, 2, 3, 50, 16)
    a = oracle_mod.attn_bwd(q, k, v, do, True, 0.25, nthreads=1)
    b = oracle_mod.attn_bwd(q, k, v, do, True, 0.25, nthreads=4)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


@pytest.mark.parametrize("mistake", [1, 2, 3, 4])
def test_pins_catch_planted_mistakes(oracle_mod, mistake):
    q, k, v, do = problem(5400, 1, 2, 30, 16)
    got = oracle_mod.attn_bwd(q, k, v, do, True, 0.4, planted_mistake=mistake)
    ref = autograd(q, k, v, do, True, 0.4)
    assert not all(np.allclose(a, b, rtol=1e-6, atol=1e-8) for a, b in zip(got, ref))
