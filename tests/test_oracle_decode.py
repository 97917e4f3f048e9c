"""Pins for the oracle's decode form: Sq query rows against Sk keys, with the
causal mask aligned bottom-right (key j visible to query i iff
j <= i + Sk - Sq), the reading a cache of past keys implies; the pages
("Validating Memory-Optimal Transformer Kernels on Real Hardware", section 5,
the decode kernel) give no alignment.  CPU only.

Each pin is independent of the oracle's own code: exact Fractions, PyTorch's
float64 SDPA with an explicit mask, and properties of the definition (the
last Sq rows of a square causal problem; one query sees every key).  The
planted top-left alignment fails them.
"""
import numpy as np
import pytest
import torch

from oracle import brute
from scaled_dot_product_attn_amd import inputs


def rnd(seed, shape, sigma=1.0):
    return inputs.normal_f16(seed, shape, sigma)


def problem(seed, B, H, Sq, Sk, D, sigma=1.0):
    q = rnd(seed, (B, H, Sq, D), sigma)
    k = rnd(seed + 1, (B, H, Sk, D), sigma)
    v = rnd(seed + 2, (B, H, Sk, D), sigma)
    return q, k, v


def torch_ref(q, k, v, causal, scale):
    """PyTorch float64 SDPA with an explicit bottom-right boolean mask."""
    Q, K, V = (torch.from_numpy(x.astype(np.float64)) for x in (q, k, v))
    Sq, Sk = Q.shape[2], K.shape[2]
    sc = float(np.float32(scale))
    mask = None
    if causal:
        i = torch.arange(Sq)[:, None]
        j = torch.arange(Sk)[None, :]
        mask = j <= i + (Sk - Sq)
    o = torch.nn.functional.scaled_dot_product_attention(Q, K, V, attn_mask=mask, scale=sc)
    logits = sc * (Q @ K.transpose(-1, -2))
    if mask is not None:
        logits = logits.masked_fill(~mask, float("-inf"))
    return o.numpy(), torch.logsumexp(logits, -1).numpy()


SHAPES = [(1, 1, 1, 1, 1), (1, 2, 1, 5, 3), (2, 1, 3, 7, 4), (1, 1, 2, 2, 8), (1, 3, 4, 9, 2)]


@pytest.mark.parametrize("B,H,Sq,Sk,D", SHAPES)
@pytest.mark.parametrize("causal", [False, True])
def test_decode_matches_exact_fractions(oracle_mod, B, H, Sq, Sk, D, causal):
    q, k, v = problem(31 + Sq + 7 * Sk + D, B, H, Sq, Sk, D)
    o, lse = oracle_mod.attn_fwd_kv(q, k, v, causal, 0.37)
    o_b, l_b = brute.attn_fwd(q, k, v, causal, 0.37)
    assert np.allclose(o, o_b, rtol=1e-12, atol=1e-13)
    assert np.allclose(lse, l_b, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("Sq,Sk", [(1, 64), (5, 200), (64, 130), (100, 100), (33, 1000)])
@pytest.mark.parametrize("causal", [False, True])
def test_decode_matches_torch_sdpa(oracle_mod, Sq, Sk, causal):
    q, k, v = problem(500 + Sq + Sk, 1, 2, Sq, Sk, 64)
    scale = 1 / np.sqrt(64)
    o, lse = oracle_mod.attn_fwd_kv(q, k, v, causal, scale)
    o_t, l_t = torch_ref(q, k, v, causal, scale)
    assert np.allclose(o, o_t, rtol=1e-11, atol=1e-12)
    assert np.allclose(lse, l_t, rtol=1e-11, atol=1e-12)


def test_decode_rows_are_the_tail_of_the_square_problem(oracle_mod):
    """With bottom-right alignment, Sq queries against Sk keys are exactly the
    last Sq rows of the Sk x Sk causal problem."""
    S, Sq, D = 150, 7, 32
    q, k, v = problem(77, 1, 2, S, S, D)
    o_full, l_full = oracle_mod.attn_fwd(q, k, v, True, 0.2)
    o, lse = oracle_mod.attn_fwd_kv(q[:, :, S - Sq:], k, v, True, 0.2)
    assert np.array_equal(o, o_full[:, :, S - Sq:])
    assert np.array_equal(lse, l_full[:, :, S - Sq:])


def test_single_query_sees_every_key(oracle_mod):
    q, k, v = problem(91, 2, 2, 1, 300, 16)
    o_c, l_c = oracle_mod.attn_fwd_kv(q, k, v, True, 0.25)
    o_n, l_n = oracle_mod.attn_fwd_kv(q, k, v, False, 0.25)
    assert np.array_equal(o_c, o_n) and np.array_equal(l_c, l_n)


def test_causal_more_queries_than_keys_rejected(oracle_mod):
    q, k, v = problem(3, 1, 1, 5, 4, 8)
    with pytest.raises(RuntimeError):
        oracle_mod.attn_fwd_kv(q, k, v, True, 0.5)
    oracle_mod.attn_fwd_kv(q, k, v, False, 0.5)  # fine without a mask


@pytest.mark.parametrize("mistake", [1, 7])
def test_pins_catch_misaligned_mask(oracle_mod, mistake):
    """A mask off by one, or aligned top-left, fails the torch pin."""
    Sq, Sk = 5, 40
    q, k, v = problem(123, 1, 2, Sq, Sk, 16)
    o, lse = oracle_mod.attn_fwd_kv(q, k, v, True, 0.3, planted_mistake=mistake)
    o_t, l_t = torch_ref(q, k, v, True, 0.3)
    assert not (np.allclose(o, o_t, rtol=1e-6, atol=1e-6) and
                np.allclose(lse, l_t, rtol=1e-6, atol=1e-6))
