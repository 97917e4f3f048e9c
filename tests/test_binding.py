"""The Python binding refuses host memory and mismatched devices before it
calls into the library: every check here raises before any launch, so no
kernel ever sees a host pointer."""
import pytest

pytestmark = pytest.mark.gpu


def _gpu_qkv(S=64, D=128, Sk=None):
    import torch
    q = torch.zeros(1, 2, S, D, dtype=torch.float16, device="cuda")
    kv = torch.zeros(1, 2, Sk or S, D, dtype=torch.float16, device="cuda")
    return q, kv, kv.clone()


def test_host_workspace_is_refused(gpu):
    import torch
    q, k, v = _gpu_qkv(S=256)
    host_ws = torch.empty(1 << 24, dtype=torch.uint8)
    with pytest.raises(ValueError, match="workspace"):
        gpu.fwd_unfused(q, k, v, causal=True, workspace=host_ws)
    with pytest.raises(ValueError, match="workspace"):
        gpu.bwd(q, k, v, q.clone(), torch.zeros(1, 2, 256, device="cuda"), q.clone(),
                causal=True, workspace=host_ws)
    q5, k5, v5 = _gpu_qkv(S=256, D=512)
    with pytest.raises(ValueError, match="workspace"):
        gpu.fwd_splitkv(q5, k5, v5, causal=True, splits=4, workspace=host_ws)
    qd, kd, vd = _gpu_qkv(S=1, Sk=4096)
    with pytest.raises(ValueError, match="workspace"):
        gpu.fwd_decode(qd, kd, vd, causal=True, splits=8, workspace=host_ws)
    # a non-contiguous device workspace is refused too
    strided = torch.empty(1 << 25, dtype=torch.uint8, device="cuda")[::2]
    with pytest.raises(ValueError, match="contiguous"):
        gpu.fwd_unfused(q, k, v, causal=True, workspace=strided)


def test_host_outputs_are_refused(gpu):
    import torch
    q, k, v = _gpu_qkv()
    with pytest.raises(ValueError):
        gpu.fwd(q, k, v, causal=True, out=torch.empty(q.shape, dtype=torch.float16))
    with pytest.raises(ValueError):
        gpu.fwd(q, k, v, causal=True, lse=torch.empty(q.shape[:3], dtype=torch.float32))
    qd, kd, vd = _gpu_qkv(S=1, Sk=256)
    with pytest.raises(ValueError):
        gpu.fwd_decode(qd, kd, vd, causal=True, out=torch.empty(qd.shape, dtype=torch.float16))
    with pytest.raises(ValueError):
        gpu.fwd_decode(qd, kd, vd, causal=True,
                       lse=torch.empty(qd.shape[:3], dtype=torch.float32))
    with pytest.raises(ValueError):
        gpu.fwd_decode(qd, kd.cpu(), vd, causal=True)
