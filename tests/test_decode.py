"""GPU parity of the decode form (Sq query rows against Sk keys, causal mask
aligned bottom-right) against the float64 oracle's decode form, with the same
gate as the square path (O: 2e-2 + 2e-2|ref|, LSE: 1e-3 max(1, |ref|))."""
import numpy as np
import pytest

from scaled_dot_product_attn_amd import inputs
from test_parity import check, log, rnd, to_dev

pytestmark = pytest.mark.gpu


def run_dec(gpu, q, k, v, causal, scale, splits=None):
    import torch
    o, lse = gpu.fwd_decode(to_dev(q), to_dev(k), to_dev(v), causal=causal, scale=scale,
                            splits=splits)
    torch.cuda.synchronize()
    return o.cpu().numpy(), lse.cpu().numpy()


def problem(seed, B, H, Sq, Sk, D, sigma=1.0):
    return (rnd(seed, (B, H, Sq, D), sigma), rnd(seed + 1, (B, H, Sk, D), sigma),
            rnd(seed + 2, (B, H, Sk, D), sigma))


@pytest.mark.parametrize("c", [1, 3])
def test_decode_workloads(gpu, oracle_mod, c):
    w = inputs.DECODE_WORKLOADS[c]
    log(f"decode workload {w.name}")
    q, k, v = w.qkv()
    o, lse = run_dec(gpu, q, k, v, w.causal, w.scale)
    o_ref, l_ref = oracle_mod.attn_fwd_kv(q, k, v, w.causal, w.scale)
    check(o, lse, o_ref, l_ref, w.name)


def test_decode_long_cache_sampled_heads(gpu, oracle_mod):
    """Sk = 65536 at full size; the oracle checks 4 of the 32 heads."""
    w = inputs.DECODE_WORKLOADS[2]
    q, k, v = w.qkv()
    o, lse = run_dec(gpu, q, k, v, w.causal, w.scale)
    heads = [0, 9, 22, 31]
    o_ref, l_ref = oracle_mod.attn_fwd_kv(q[:, heads], k[:, heads], v[:, heads], w.causal, w.scale)
    check(o[:, heads], lse[:, heads], o_ref, l_ref, w.name + " heads 0,9,22,31")


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_decode_shapes_and_splits(gpu, oracle_mod, D, causal):
    for (Sq, Sk) in [(1, 1), (1, 63), (1, 65), (3, 3), (5, 1000), (64, 700), (65, 700),
                     (130, 2000), (200, 200)]:
        for splits in (1, 3, 64):
            q, k, v = problem(3000 + Sq + Sk + D, 1, 2, Sq, Sk, D)
            scale = float(np.float32(1 / np.sqrt(D)))
            o, lse = run_dec(gpu, q, k, v, causal, scale, splits)
            o_ref, l_ref = oracle_mod.attn_fwd_kv(q, k, v, causal, scale)
            check(o, lse, o_ref, l_ref, f"D={D} causal={causal} Sq={Sq} Sk={Sk} splits={splits}")


def test_decode_batch_heads_layout(gpu, oracle_mod):
    q, k, v = problem(4100, 2, 3, 7, 517, 128, 0.5)
    o, lse = run_dec(gpu, q, k, v, True, 0.1, 5)
    o_ref, l_ref = oracle_mod.attn_fwd_kv(q, k, v, True, 0.1)
    check(o, lse, o_ref, l_ref, "B=2 H=3 Sq=7 Sk=517")


def test_decode_square_matches_fused(gpu):
    """With Sq = Sk the decode form is attn_fwd's problem (different kernels,
    so within the gate rather than bit for bit)."""
    import torch
    w = inputs.WORKLOADS[3]
    q, k, v = (to_dev(x) for x in w.qkv())
    o1, l1 = gpu.fwd_decode(q, k, v, causal=True, scale=w.scale, splits=4)
    o2, l2 = gpu.fwd(q, k, v, causal=True, scale=w.scale)
    torch.cuda.synchronize()
    d = (o1.float() - o2.float()).abs()
    assert d.max().item() <= 2e-2, d.max().item()
    assert (l1 - l2).abs().max().item() <= 1e-3 * max(1.0, l2.abs().max().item())


def test_decode_repeat_bit_identical(gpu):
    import torch
    w = inputs.DECODE_WORKLOADS[3]
    q, k, v = (to_dev(x) for x in w.qkv())
    outs = []
    for _ in range(3):
        o, l = gpu.fwd_decode(q, k, v, causal=True, scale=w.scale, splits=16)
        torch.cuda.synchronize()
        outs.append((o.clone(), l.clone()))
    for o, l in outs[1:]:
        assert torch.equal(o, outs[0][0]) and torch.equal(l, outs[0][1])
