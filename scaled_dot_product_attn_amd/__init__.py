"""Fused scaled-dot-product attention forward for AMD Instinct MI355X.

A thin ctypes binding over libattn.so (include/attn.h).  It only marshals
arguments: every step of the computation runs in the library's HIP kernels.
PyTorch provides device memory and the current stream.  There is no fallback:
if the library is missing the calls raise.
"""
from __future__ import annotations

import ctypes
import math
import os

from .build import LIB_PATH

__all__ = ["AttnError", "fwd", "fwd_unfused", "unfused_workspace_bytes", "fwd_splitkv",
           "splitkv_workspace_bytes", "splitkv_splits", "fwd_decode", "fwd_decode_noalloc", "decode_workspace_bytes", "decode_splits",
           "DECODE_NOALLOC_SCRATCH_BYTES", "bwd", "bwd_workspace_bytes", "head_dim_supported", "load_library", "LIB_PATH",
           "SYMBOLS"]

# Every symbol include/attn.h declares.
SYMBOLS = ("attn_fwd", "attn_fwd_unfused", "attn_fwd_unfused_workspace_bytes",
           "attn_fwd_splitkv", "attn_fwd_splitkv_workspace_bytes",
           "attn_fwd_decode", "attn_fwd_decode_workspace_bytes", "attn_fwd_decode_noalloc",
           "attn_bwd", "attn_bwd_workspace_bytes", "attn_bwd_workspace_bytes_d",
           "attn_head_dim_supported", "attn_status_string", "attn_last_hip_error")

ATTN_ERR_LAUNCH = -5
ATTN_ERR_SCRATCH = -9
# capacity of the static scratch array behind fwd_decode_noalloc (attn.h)
DECODE_NOALLOC_SCRATCH_BYTES = 32 << 20


class AttnError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"attn error {code}: {msg}")
        self.code = code


_lib = None


def load_library(path: str = LIB_PATH):
    """Load libattn.so (built by build.py / __graft_entry__.build())."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with "
                          "`python -m scaled_dot_product_attn_amd.build`")
    # Bring up torch's HIP runtime before the library registers its kernels:
    # a library loaded ahead of torch's lazy GPU initialisation gets
    # hipErrorNoDevice (100) from every launch.  On a machine without a GPU
    # this only counts devices, and the library still loads for its
    # argument-checking entry points.
    import torch
    if torch.cuda.is_available():
        torch.cuda.init()
    L = ctypes.CDLL(path)
    P, I, F, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    L.attn_fwd.argtypes = [P, P, P, P, P, I, I, I, I, I, F, P]
    L.attn_fwd.restype = I
    L.attn_fwd_unfused.argtypes = [P, P, P, P, P, I, I, I, I, I, F, P, Z, P]
    L.attn_fwd_unfused.restype = I
    L.attn_fwd_unfused_workspace_bytes.argtypes = [I, I, I]
    L.attn_fwd_unfused_workspace_bytes.restype = Z
    L.attn_fwd_splitkv.argtypes = [P, P, P, P, P, I, I, I, I, I, F, I, P, Z, P]
    L.attn_fwd_splitkv.restype = I
    L.attn_fwd_splitkv_workspace_bytes.argtypes = [I, I, I, I, I, I]
    L.attn_fwd_splitkv_workspace_bytes.restype = Z
    L.attn_fwd_decode.argtypes = [P, P, P, P, P, I, I, I, I, I, I, F, I, P, Z, P]
    L.attn_fwd_decode.restype = I
    L.attn_fwd_decode_noalloc.argtypes = [P, P, P, P, P, I, I, I, I, I, I, F, I, P]
    L.attn_fwd_decode_noalloc.restype = I
    L.attn_fwd_decode_workspace_bytes.argtypes = [I, I, I, I, I, I, I]
    L.attn_fwd_decode_workspace_bytes.restype = Z
    L.attn_bwd.argtypes = [P, P, P, P, P, P, P, P, P, I, I, I, I, I, F, P, Z, P]
    L.attn_bwd.restype = I
    L.attn_bwd_workspace_bytes.argtypes = [I, I, I]
    L.attn_bwd_workspace_bytes.restype = Z
    L.attn_bwd_workspace_bytes_d.argtypes = [I, I, I, I]
    L.attn_bwd_workspace_bytes_d.restype = Z
    L.attn_head_dim_supported.argtypes = [I]
    L.attn_head_dim_supported.restype = I
    L.attn_status_string.argtypes = [I]
    L.attn_status_string.restype = ctypes.c_char_p
    L.attn_last_hip_error.argtypes = []
    L.attn_last_hip_error.restype = I
    _lib = L
    return L


def _check(code: int):
    if code != 0:
        L = load_library()
        msg = L.attn_status_string(code).decode()
        if code == ATTN_ERR_LAUNCH:
            msg += f" (hipError {L.attn_last_hip_error()})"
        raise AttnError(code, msg)


def head_dim_supported(D: int) -> bool:
    return bool(load_library().attn_head_dim_supported(D))


def unfused_workspace_bytes(B: int, H: int, S: int) -> int:
    return int(load_library().attn_fwd_unfused_workspace_bytes(B, H, S))


def _workspace(workspace, need, device):
    """The workspace tensor to pass (allocated when None and needed), checked
    to be contiguous device memory on `device`.  Returns (pointer, bytes)."""
    import torch
    if workspace is None:
        if need == 0:
            return None, 0
        workspace = torch.empty(need, dtype=torch.uint8, device=device)
    if not isinstance(workspace, torch.Tensor):
        raise TypeError("workspace must be a torch.Tensor")
    if workspace.device != device:
        raise ValueError(f"workspace must be on {device}, got {workspace.device}")
    if not workspace.is_contiguous():
        raise ValueError("workspace must be contiguous")
    return workspace.data_ptr(), workspace.numel() * workspace.element_size()


def _prepare(q, k, v, out, lse, scale):
    import torch
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch.Tensor")
        if t.dtype != torch.float16:
            raise TypeError(f"{name} must be float16, got {t.dtype}")
        if t.device.type != "cuda":
            raise ValueError(f"{name} must be on a GPU device")
        if t.dim() != 4:
            raise ValueError(f"{name} must be [B, H, S, D]")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if not (q.shape == k.shape == v.shape):
        raise ValueError(f"q, k, v shapes differ: {q.shape} {k.shape} {v.shape}")
    if not (q.device == k.device == v.device):
        raise ValueError("q, k, v must be on the same device")
    B, H, S, D = q.shape
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape or out.dtype != torch.float16 or not out.is_contiguous() \
            or out.device != q.device:
        raise ValueError("out must be a contiguous float16 tensor shaped like q")
    if lse is None:
        lse = torch.empty((B, H, S), dtype=torch.float32, device=q.device)
    elif lse.shape != (B, H, S) or lse.dtype != torch.float32 or not lse.is_contiguous() \
            or lse.device != q.device:
        raise ValueError("lse must be a contiguous float32 tensor [B, H, S]")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    stream = torch.cuda.current_stream(q.device).cuda_stream
    return B, H, S, D, out, lse, float(scale), stream


def fwd(q, k, v, *, causal: bool, scale: float | None = None, out=None, lse=None):
    """Fused forward.  q, k, v: contiguous fp16 [B, H, S, D] on the GPU.
    Returns (o fp16 [B, H, S, D], lse fp32 [B, H, S]).  Enqueued on the
    current stream; asynchronous."""
    L = load_library()
    B, H, S, D, out, lse, scale, stream = _prepare(q, k, v, out, lse, scale)
    _check(L.attn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                      lse.data_ptr(), B, H, S, D, int(bool(causal)), scale, stream))
    return out, lse


def fwd_unfused(q, k, v, *, causal: bool, scale: float | None = None, out=None,
                lse=None, workspace=None):
    """Unfused three-kernel forward (ablation).  ``workspace``: a uint8 GPU
    tensor of at least unfused_workspace_bytes(B, H, S) bytes; allocated with
    torch when not given."""
    L = load_library()
    B, H, S, D, out, lse, scale, stream = _prepare(q, k, v, out, lse, scale)
    wptr, wbytes = _workspace(workspace, unfused_workspace_bytes(B, H, S), q.device)
    _check(L.attn_fwd_unfused(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                              lse.data_ptr(), B, H, S, D, int(bool(causal)), scale,
                              wptr, wbytes, stream))
    return out, lse


def splitkv_workspace_bytes(B: int, H: int, S: int, D: int, causal: bool, splits: int) -> int:
    return int(load_library().attn_fwd_splitkv_workspace_bytes(B, H, S, D, int(bool(causal)),
                                                                splits))


def splitkv_splits(B: int, H: int, S: int, causal: bool, max_units: int = 282,
                   D: int = 512) -> int:
    """A default split count for fwd_splitkv.  D = 64, 128: decode_splits
    with Sq = Sk = S.  D = 512: the largest count (up to 16) whose (batch,
    head, query tile, chunk) work units still run in about one wave on the
    256 CUs of an MI355X (one workgroup per CU, 10% over allowed).  A query
    tile of 64 rows sees nkt 32-key tiles (all ceil(S/32), or those up to its
    last row when causal) and is cut into ceil(nkt / C) chunks,
    C = ceil(ceil(S/32) / splits).  At B1 H8 S1024 causal it picks 3 (256
    units), measured faster than 2 (192 units) and 4 (320 units)."""
    if D in (64, 128):
        return decode_splits(B, H, S, S)
    nmax = -(-S // 32)
    tq = -(-S // 64)
    best = 1
    for splits in range(1, 17):
        c = -(-nmax // splits)
        units = 0
        for qt in range(tq):
            kv_end = min(S, 64 * (qt + 1)) if causal else S
            units += -(-(-(-kv_end // 32)) // c)
        if B * H * units <= max_units:
            best = splits
    return best


def fwd_splitkv(q, k, v, *, causal: bool, splits: int | None = None, scale: float | None = None,
                out=None, lse=None, workspace=None):
    """Split-KV forward: every query tile's key range in chunks (D = 512: of
    at most ceil(ceil(S/32) / splits) 32-key tiles; D = 64, 128: the decode
    kernel with Sq = Sk, 64-key tiles), merged in chunk order.
    ``splits`` defaults to splitkv_splits(B, H, S, causal, D=D).
    ``workspace``: a uint8 GPU tensor of at least splitkv_workspace_bytes(...)
    bytes; allocated with torch when not given and needed."""
    L = load_library()
    B, H, S, D, out, lse, scale, stream = _prepare(q, k, v, out, lse, scale)
    if splits is None:
        splits = splitkv_splits(B, H, S, causal, D=D)
    wptr, wbytes = _workspace(workspace, splitkv_workspace_bytes(B, H, S, D, causal, splits),
                              q.device)
    _check(L.attn_fwd_splitkv(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                              lse.data_ptr(), B, H, S, D, int(bool(causal)), scale, int(splits),
                              wptr, wbytes, stream))
    return out, lse


def decode_workspace_bytes(B: int, H: int, Sq: int, Sk: int, D: int, causal: bool,
                           splits: int) -> int:
    return int(load_library().attn_fwd_decode_workspace_bytes(B, H, Sq, Sk, D,
                                                               int(bool(causal)), splits))


def decode_splits(B: int, H: int, Sq: int, Sk: int, target_units: int = 256,
                  max_chunk_tiles: int = 64) -> int:
    """A default chunk count: enough (batch, head, query tile, chunk) units to
    give every CU of an MI355X (256) one workgroup, doubled while a chunk
    would still span more than max_chunk_tiles 64-key tiles, and at most one
    chunk per 64-key tile.  Measured (B1 H32 Sq1 D128): 8 splits beat 16 at
    Sk = 4096 (18.6 vs 22.2 us) and 16384 (47.0 vs 50.7 us); 16 beat 8 at
    65536 (193.7 vs 203.4 us)."""
    q_tiles = -(-Sq // 64)
    k_tiles = -(-Sk // 64)
    splits = max(1, -(-target_units // (B * H * q_tiles)))
    while -(-k_tiles // splits) > max_chunk_tiles and splits < k_tiles:
        splits *= 2
    return max(1, min(k_tiles, splits))


def _decode_args(q, k, v, out, lse, scale, splits, causal):
    import torch
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch.Tensor")
        if t.dtype != torch.float16:
            raise TypeError(f"{name} must be float16, got {t.dtype}")
        if t.device.type != "cuda" or t.dim() != 4 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous 4-D GPU tensor")
    B, H, Sq, D = q.shape
    Sk = k.shape[2]
    if k.shape != v.shape or k.shape[0] != B or k.shape[1] != H or k.shape[3] != D:
        raise ValueError(f"k, v must be [B, H, Sk, D] matching q: {q.shape} {k.shape} {v.shape}")
    if not (q.device == k.device == v.device):
        raise ValueError("q, k, v must be on the same device")
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape or out.dtype != torch.float16 or not out.is_contiguous() \
            or out.device != q.device:
        raise ValueError("out must be a contiguous float16 tensor shaped like q, on q's device")
    if lse is None:
        lse = torch.empty((B, H, Sq), dtype=torch.float32, device=q.device)
    elif lse.shape != (B, H, Sq) or lse.dtype != torch.float32 or not lse.is_contiguous() \
            or lse.device != q.device:
        raise ValueError("lse must be a contiguous float32 tensor [B, H, Sq] on q's device")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if splits is None:
        splits = decode_splits(B, H, Sq, Sk)
    stream = torch.cuda.current_stream(q.device).cuda_stream
    return B, H, Sq, Sk, D, out, lse, float(scale), int(splits), stream


def fwd_decode(q, k, v, *, causal: bool, splits: int | None = None,
               scale: float | None = None, out=None, lse=None, workspace=None):
    """Decode form: q [B, H, Sq, D] against k, v [B, H, Sk, D] (contiguous fp16
    on the GPU, D = 64 or 128); causal aligned bottom-right.  Returns
    (o fp16 [B, H, Sq, D], lse fp32 [B, H, Sq])."""
    B, H, Sq, Sk, D, out, lse, scale, splits, stream = _decode_args(q, k, v, out, lse, scale,
                                                                    splits, causal)
    L = load_library()
    wptr, wbytes = _workspace(workspace, decode_workspace_bytes(B, H, Sq, Sk, D, causal, splits),
                              q.device)
    _check(L.attn_fwd_decode(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                             lse.data_ptr(), B, H, Sq, Sk, D, int(bool(causal)), scale,
                             splits, wptr, wbytes, stream))
    return out, lse


def fwd_decode_noalloc(q, k, v, *, causal: bool, splits: int | None = None,
                       scale: float | None = None, out=None, lse=None):
    """fwd_decode without a workspace: the library's static per-GPU scratch
    array (DECODE_NOALLOC_SCRATCH_BYTES) holds the chunks' partial states, and
    the C entry point allocates nothing (pass out and lse to keep torch from
    allocating them).  Calls that overlap on one GPU race on the array."""
    B, H, Sq, Sk, D, out, lse, scale, splits, stream = _decode_args(q, k, v, out, lse, scale,
                                                                    splits, causal)
    L = load_library()
    _check(L.attn_fwd_decode_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                     lse.data_ptr(), B, H, Sq, Sk, D, int(bool(causal)), scale,
                                     splits, stream))
    return out, lse


def bwd_workspace_bytes(B: int, H: int, S: int, D: int = 128) -> int:
    return int(load_library().attn_bwd_workspace_bytes_d(B, H, S, D))


def bwd(q, k, v, o, lse, do, *, causal: bool, scale: float | None = None, dq=None, dk=None,
        dv=None, workspace=None):
    """Backward of fwd (D = 64, 128 or 512): q, k, v, o, do contiguous fp16
    [B, H, S, D] and lse fp32 [B, H, S] on one GPU, o and lse from fwd with the
    same causal and scale.  Returns (dq, dk, dv), fp16 [B, H, S, D].
    Enqueued on the current stream; asynchronous."""
    import torch
    B, H, S, D, _, _, scale, stream = _prepare(q, k, v, o, lse, scale)
    if not isinstance(do, torch.Tensor) or do.dtype != torch.float16 or \
            do.shape != q.shape or not do.is_contiguous() or do.device != q.device:
        raise ValueError("do must be a contiguous float16 tensor shaped like q")
    grads = []
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        if t is None:
            t = torch.empty_like(q)
        elif t.shape != q.shape or t.dtype != torch.float16 or not t.is_contiguous() \
                or t.device != q.device:
            raise ValueError(f"{name} must be a contiguous float16 tensor shaped like q")
        grads.append(t)
    L = load_library()
    wptr, wbytes = _workspace(workspace, bwd_workspace_bytes(B, H, S, D), q.device)
    _check(L.attn_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                      do.data_ptr(), grads[0].data_ptr(), grads[1].data_ptr(),
                      grads[2].data_ptr(), B, H, S, D, int(bool(causal)), scale,
                      wptr, wbytes, stream))
    return tuple(grads)
