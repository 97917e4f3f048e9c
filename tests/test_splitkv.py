"""GPU parity of the split-KV forward against the float64 oracle (D = 512:
its own chunked kernel; D = 64, 128: the decode kernel with Sq = Sk).

Every query tile's key range is cut into chunks that leave partial states in
a workspace and are merged in chunk order by a second kernel.  The merge is
over disjoint key sets, so the result is the softmax over all keys up to
rounding: the same gate as the fused path (O: 2e-2 + 2e-2|ref|, LSE:
1e-3 max(1, |ref|)), and with splits = 1 the same kernel writes every tile
directly, so its bytes equal the fused call's.
"""
import numpy as np
import pytest

from scaled_dot_product_attn_amd import inputs
from test_parity import check, log, rnd, to_dev

pytestmark = pytest.mark.gpu


def run_split(gpu, q, k, v, causal, scale, splits):
    import torch
    o, lse = gpu.fwd_splitkv(to_dev(q), to_dev(k), to_dev(v), causal=causal, scale=scale,
                             splits=splits)
    torch.cuda.synchronize()
    return o.cpu().numpy(), lse.cpu().numpy()


# None: the binding's default count (splitkv_splits), the one bench.py times
@pytest.mark.parametrize("splits", [2, 3, 4, 7, None])
def test_splitkv_workload5(gpu, oracle_mod, splits):
    w = inputs.WORKLOADS[5]
    if splits is None:
        assert gpu.splitkv_splits(w.B, w.H, w.S, w.causal) == 3
    log(f"split-KV {w.name} splits={splits}")
    q, k, v = w.qkv()
    o, lse = run_split(gpu, q, k, v, w.causal, w.scale, splits)
    o_ref, l_ref = oracle_mod.attn_fwd(q, k, v, w.causal, w.scale)
    check(o, lse, o_ref, l_ref, f"{w.name} splits={splits}")


@pytest.mark.parametrize("causal", [False, True])
def test_splitkv_ragged(gpu, oracle_mod, causal):
    for S in (1, 33, 65, 200, 333):
        for splits in (2, 3, 16):
            B, H, D = 1, 2, 512
            q, k, v = (rnd(700 + 10 * S + t, (B, H, S, D)) for t in range(3))
            scale = float(np.float32(1 / np.sqrt(D)))
            o, lse = run_split(gpu, q, k, v, causal, scale, splits)
            o_ref, l_ref = oracle_mod.attn_fwd(q, k, v, causal, scale)
            check(o, lse, o_ref, l_ref, f"S={S} causal={causal} splits={splits}")


def test_splitkv_batch_heads(gpu, oracle_mod):
    B, H, S, D = 2, 3, 300, 512
    q, k, v = (rnd(900 + t, (B, H, S, D), 0.5) for t in range(3))
    scale = float(np.float32(1 / np.sqrt(D)))
    o, lse = run_split(gpu, q, k, v, True, scale, 4)
    o_ref, l_ref = oracle_mod.attn_fwd(q, k, v, True, scale)
    check(o, lse, o_ref, l_ref, "B=2 H=3 S=300 splits=4")


def test_splitkv_one_split_equals_fused(gpu):
    import torch
    w = inputs.WORKLOADS[5]
    q, k, v = (to_dev(x) for x in w.qkv())
    o1, l1 = gpu.fwd_splitkv(q, k, v, causal=True, scale=w.scale, splits=1)
    o2, l2 = gpu.fwd(q, k, v, causal=True, scale=w.scale)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_splitkv_repeat_bit_identical(gpu):
    import torch
    w = inputs.WORKLOADS[5]
    q, k, v = (to_dev(x) for x in w.qkv())
    outs = []
    for _ in range(3):
        o, l = gpu.fwd_splitkv(q, k, v, causal=True, scale=w.scale, splits=4)
        torch.cuda.synchronize()
        outs.append((o.clone(), l.clone()))
    for o, l in outs[1:]:
        assert torch.equal(o, outs[0][0]) and torch.equal(l, outs[0][1])


def test_splitkv_shared_workspace(gpu):
    """D = 512: one workspace, left as the previous call wrote it, serves
    calls of different shapes and split counts in turn, and each gives the
    bytes of a call on a workspace of its own: no call reads what it did not
    write in that call."""
    import torch
    shapes = [(1, 8, 1024, True, 3), (2, 3, 300, True, 4), (1, 2, 333, False, 16),
              (1, 8, 1024, True, 7), (1, 1, 65, True, 2)]
    need = max(gpu.splitkv_workspace_bytes(B, H, S, 512, c, sp) for B, H, S, c, sp in shapes)
    shared = torch.full((need,), 0x7f, dtype=torch.uint8, device="cuda")
    for rep in range(2):
        for i, (B, H, S, causal, splits) in enumerate(shapes):
            log(f"shared workspace rep={rep} B={B} H={H} S={S} causal={causal} splits={splits}")
            q, k, v = (to_dev(rnd(1300 + 10 * i + t, (B, H, S, 512), 0.5)) for t in range(3))
            scale = float(np.float32(1 / np.sqrt(512)))
            o1, l1 = gpu.fwd_splitkv(q, k, v, causal=causal, scale=scale, splits=splits,
                                     workspace=shared)
            o2, l2 = gpu.fwd_splitkv(q, k, v, causal=causal, scale=scale, splits=splits)
            torch.cuda.synchronize()
            assert torch.equal(o1, o2) and torch.equal(l1, l2)


# D = 64, 128: workloads 1 and 2, every split count from 1 to one chunk per
# 64-key tile, and the default
@pytest.mark.parametrize("c", [1, 2])
def test_splitkv_small_d_workloads(gpu, oracle_mod, c):
    w = inputs.WORKLOADS[c]
    q, k, v = w.qkv()
    o_ref, l_ref = oracle_mod.attn_fwd(q, k, v, w.causal, w.scale)
    for splits in (1, 2, 3, -(-w.S // 64), None):
        log(f"split-KV {w.name} splits={splits}")
        o, lse = run_split(gpu, q, k, v, w.causal, w.scale, splits)
        check(o, lse, o_ref, l_ref, f"{w.name} splits={splits}")


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_splitkv_small_d_ragged(gpu, oracle_mod, D, causal):
    for S in (1, 63, 65, 200, 333):
        for splits in (2, 5):
            B, H = 2, 3
            q, k, v = (rnd(1300 + 10 * S + D + t, (B, H, S, D)) for t in range(3))
            scale = float(np.float32(1 / np.sqrt(D)))
            o, lse = run_split(gpu, q, k, v, causal, scale, splits)
            o_ref, l_ref = oracle_mod.attn_fwd(q, k, v, causal, scale)
            check(o, lse, o_ref, l_ref, f"D={D} S={S} causal={causal} splits={splits}")


def test_splitkv_small_d_equals_decode(gpu):
    """With Sq = Sk the split-KV call is the decode call: same bytes."""
    import torch
    B, H, S, D = 1, 4, 256, 128
    q, k, v = (to_dev(rnd(1500 + t, (B, H, S, D))) for t in range(3))
    o1, l1 = gpu.fwd_splitkv(q, k, v, causal=True, splits=3)
    o2, l2 = gpu.fwd_decode(q, k, v, causal=True, splits=3)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
