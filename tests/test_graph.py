"""HIP graph capture of every path: a graph of several calls on
different inputs, replayed several times with eager work and
synchronisations in between, gives the eager outputs bit for bit on every
replay.  (bench.py times its K steps as one such graph.)"""
import numpy as np
import pytest

from scaled_dot_product_attn_amd import inputs

pytestmark = pytest.mark.gpu


def _inputs(seed, shape, n):
    import torch
    return [tuple(torch.from_numpy(inputs.normal_f16(seed + 10 * i + t, shape)).cuda()
                  for t in range(3)) for i in range(n)]


# fused: the 64-row D = 128 kernel; fused_rows: the 128-row kernel with
# tiles in pairs (>= 512 pairs of 128-row tiles); fused512: D = 512 on
# 32-row tiles of two waves
@pytest.mark.parametrize("path", ["fused", "fused_rows", "fused512", "unfused", "decode",
                                  "splitkv"])
def test_graph_replays_match_eager(gpu, path):
    import torch
    if path == "decode":
        B, H, Sq, Sk, D, causal, sc = 1, 4, 2, 700, 128, True, 0.088
        sets = [(q[:, :, :Sq].contiguous(), k, v) for q, k, v in _inputs(90_000, (B, H, Sk, D), 3)]
        splits = gpu.decode_splits(B, H, Sq, Sk)
        ws = torch.empty(max(gpu.decode_workspace_bytes(B, H, Sq, Sk, D, causal, splits), 1),
                         dtype=torch.uint8, device="cuda")
        qshape = (B, H, Sq, D)
    elif path == "splitkv":
        B, H, S, D, causal, sc, splits = 1, 2, 300, 512, True, 0.044, 3
        sets = _inputs(93_000, (B, H, S, D), 3)
        ws = torch.empty(gpu.splitkv_workspace_bytes(B, H, S, D, causal, splits),
                         dtype=torch.uint8, device="cuda")
        qshape = (B, H, S, D)
    elif path == "fused_rows":
        B, H, S, D, causal, sc = 1, 512, 200, 128, True, 0.088
        assert B * H * ((-(-S // 128) + 1) // 2) >= 512
        sets = _inputs(94_000, (B, H, S, D), 3)
        qshape = (B, H, S, D)
    elif path == "fused512":
        B, H, S, D, causal, sc = 1, 2, 300, 512, True, 0.044
        sets = _inputs(95_000, (B, H, S, D), 3)
        qshape = (B, H, S, D)
    else:
        B, H, S, D, causal, sc = 2, 3, 300, 128, True, 0.088
        sets = _inputs(91_000, (B, H, S, D), 3)
        ws = torch.empty(gpu.unfused_workspace_bytes(B, H, S), dtype=torch.uint8, device="cuda")
        qshape = (B, H, S, D)
    outs = [(torch.empty(qshape, dtype=torch.float16, device="cuda"),
             torch.empty(qshape[:3], dtype=torch.float32, device="cuda")) for _ in sets]

    def call(i):
        q, k, v = sets[i]
        o, lse = outs[i]
        if path in ("fused", "fused_rows", "fused512"):
            gpu.fwd(q, k, v, causal=causal, scale=sc, out=o, lse=lse)
        elif path == "unfused":
            gpu.fwd_unfused(q, k, v, causal=causal, scale=sc, out=o, lse=lse, workspace=ws)
        elif path == "splitkv":
            gpu.fwd_splitkv(q, k, v, causal=causal, scale=sc, splits=splits, out=o, lse=lse,
                            workspace=ws)
        else:
            gpu.fwd_decode(q, k, v, causal=causal, scale=sc, splits=splits, out=o, lse=lse,
                           workspace=ws)

    for i in range(len(sets)):
        call(i)
    torch.cuda.synchronize()
    eager = [(o.clone(), lse.clone()) for o, lse in outs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(len(sets)):
            call(i)
    for rep in range(4):
        for o, lse in outs:
            o.fill_(float("nan"))
            lse.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for (o, lse), (eo, el) in zip(outs, eager):
            assert torch.equal(o, eo), f"{path}: O differs on replay {rep}"
            assert torch.equal(lse, el), f"{path}: LSE differs on replay {rep}"
        # eager work between replays
        call(0)
        torch.cuda.synchronize()


def test_graph_backward_replays_match_eager(gpu):
    """The backward (two launches sharing a workspace) captured over several
    input sets and replayed: every replay gives the eager dQ, dK, dV bit for
    bit, with eager calls and synchronisations in between."""
    import torch
    B, H, S, D, causal, sc = 2, 3, 300, 128, True, 0.088
    sets = []
    for i, (q, k, v) in enumerate(_inputs(92_000, (B, H, S, D), 3)):
        do = torch.from_numpy(inputs.normal_f16(92_500 + i, (B, H, S, D))).cuda()
        o, lse = gpu.fwd(q, k, v, causal=causal, scale=sc)
        sets.append((q, k, v, o, lse, do))
    torch.cuda.synchronize()
    ws = torch.empty(gpu.bwd_workspace_bytes(B, H, S), dtype=torch.uint8, device="cuda")
    grads = [tuple(torch.empty((B, H, S, D), dtype=torch.float16, device="cuda") for _ in range(3))
             for _ in sets]

    def call(i):
        q, k, v, o, lse, do = sets[i]
        dq, dk, dv = grads[i]
        gpu.bwd(q, k, v, o, lse, do, causal=causal, scale=sc, dq=dq, dk=dk, dv=dv, workspace=ws)

    for i in range(len(sets)):
        call(i)
    torch.cuda.synchronize()
    eager = [tuple(t.clone() for t in g3) for g3 in grads]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(len(sets)):
            call(i)
    for rep in range(4):
        for g3 in grads:
            for t in g3:
                t.fill_(float("nan"))
        ws.fill_(0xFF)  # a stale workspace must not leak into the result
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for g3, e3 in zip(grads, eager):
            for name, t, e in zip(("dQ", "dK", "dV"), g3, e3):
                assert torch.equal(t, e), f"backward: {name} differs on replay {rep}"
        call(1)
        torch.cuda.synchronize()
