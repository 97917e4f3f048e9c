"""attn_fwd_decode_noalloc against attn_fwd_decode through the C ABI: the same
kernels with the workspace in the library's static per-GPU array instead of a
caller buffer, so the outputs must be the same bytes.  Two calls in a row,
the second smaller (the array keeps the first call's contents), plus the
oracle's gate on each, and an oversized call refused before any launch."""
import math
import sys

import numpy as np
import pytest

from scaled_dot_product_attn_amd import inputs

pytestmark = pytest.mark.gpu


def log(msg):
    print(msg, file=sys.stderr, flush=True)


CASES = [
    # (B, H, Sq, Sk, D, causal): the first needs ~8.5 MB of scratch, the second less
    (1, 32, 1, 4096, 128, True),
    (2, 3, 5, 1000, 64, False),
]


def _inputs(case, seed):
    B, H, Sq, Sk, D, causal = case
    q = inputs.normal_f16(seed, (B, H, Sq, D))
    k = inputs.normal_f16(seed + 1, (B, H, Sk, D))
    v = inputs.normal_f16(seed + 2, (B, H, Sk, D))
    return q, k, v


def test_noalloc_matches_workspace_entry_point(gpu, oracle_mod):
    import torch
    for i, case in enumerate(CASES):
        B, H, Sq, Sk, D, causal = case
        q, k, v = _inputs(case, 40_000 + 10 * i)
        qd, kd, vd = (torch.from_numpy(x).cuda() for x in (q, k, v))
        splits = gpu.decode_splits(B, H, Sq, Sk)
        need = gpu.decode_workspace_bytes(B, H, Sq, Sk, D, causal, splits)
        log(f"no-alloc decode {case} splits={splits} workspace={need} bytes")
        assert 0 < need <= gpu.DECODE_NOALLOC_SCRATCH_BYTES
        sc = 1 / math.sqrt(D)
        o1, l1 = gpu.fwd_decode(qd, kd, vd, causal=causal, scale=sc, splits=splits)
        o2, l2 = gpu.fwd_decode_noalloc(qd, kd, vd, causal=causal, scale=sc, splits=splits)
        torch.cuda.synchronize()
        o1, l1, o2, l2 = (t.cpu().numpy() for t in (o1, l1, o2, l2))
        assert np.array_equal(o1, o2) and np.array_equal(l1, l2), case
        o_ref, l_ref = oracle_mod.attn_fwd_kv(q, k, v, causal, sc)
        d_o = np.abs(o2.astype(np.float64) - o_ref)
        d_l = np.abs(l2.astype(np.float64) - l_ref)
        assert np.all(d_o <= 2e-2 + 2e-2 * np.abs(o_ref)), case
        assert np.all(d_l <= 1e-3 * np.maximum(1.0, np.abs(l_ref))), case


def test_noalloc_refuses_oversize(gpu):
    import torch
    B, H, Sq, Sk, D = 1, 64, 1, 65536, 128
    need = gpu.decode_workspace_bytes(B, H, Sq, Sk, D, True, 64)
    assert need > gpu.DECODE_NOALLOC_SCRATCH_BYTES
    q = torch.zeros(B, H, Sq, D, dtype=torch.float16, device="cuda")
    kv = torch.zeros(B, H, Sk, D, dtype=torch.float16, device="cuda")
    with pytest.raises(gpu.AttnError) as e:
        gpu.fwd_decode_noalloc(q, kv, kv, causal=True, splits=64)
    assert e.value.code == -9
