"""HIP graph capture of the forward paths: a graph of several calls on
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


@pytest.mark.parametrize("path", ["fused", "unfused", "decode"])
def test_graph_replays_match_eager(gpu, path):
    import torch
    if path == "decode":
        B, H, Sq, Sk, D, causal, sc = 1, 4, 2, 700, 128, True, 0.088
        sets = [(q[:, :, :Sq].contiguous(), k, v) for q, k, v in _inputs(90_000, (B, H, Sk, D), 3)]
        splits = gpu.decode_splits(B, H, Sq, Sk)
        ws = torch.empty(max(gpu.decode_workspace_bytes(B, H, Sq, Sk, D, causal, splits), 1),
                         dtype=torch.uint8, device="cuda")
        qshape = (B, H, Sq, D)
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
        if path == "fused":
            gpu.fwd(q, k, v, causal=causal, scale=sc, out=o, lse=lse)
        elif path == "unfused":
            gpu.fwd_unfused(q, k, v, causal=causal, scale=sc, out=o, lse=lse, workspace=ws)
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
