"""The C ABI on the CPU: libattn.so loads, exports every symbol that
include/attn.h declares, and rejects bad arguments with the documented
status codes before any HIP call (no kernel is launched here)."""
import ctypes
import math
import os
import re

import pytest

import scaled_dot_product_attn_amd as attn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(attn.LIB_PATH):
        from scaled_dot_product_attn_amd import build
        build.build()
    return attn.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_\w+)\s*\(", text)))


def declared_codes():
    return {m[0]: int(m[1]) for m in
            re.findall(r"#define\s+(ATTN_\w+)\s+(-?\d+)", open(HEADER).read())}


def test_every_declared_symbol_is_exported(L):
    names = declared_functions()
    assert set(names) == set(attn.SYMBOLS)
    for name in names:
        assert hasattr(L, name), name


def test_status_strings(L):
    for name, code in declared_codes().items():
        s = L.attn_status_string(code).decode()
        assert s and s != "unknown status", name
    assert L.attn_status_string(12345).decode() == "unknown status"


def test_head_dims(L):
    assert [d for d in range(1, 1025) if L.attn_head_dim_supported(d)] == [64, 128, 512]


C = declared_codes()
# distinct fake addresses, never dereferenced: validation rejects first
Q, K, V, O, LSE = (0x10000000 * (i + 1) for i in range(5))


def call(L, q=Q, k=K, v=V, o=O, lse=LSE, B=1, H=2, S=64, D=64, causal=1, scale=0.125):
    return L.attn_fwd(q, k, v, o, lse, B, H, S, D, causal, scale, None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), "ATTN_ERR_NULL"), (dict(k=None), "ATTN_ERR_NULL"),
    (dict(v=None), "ATTN_ERR_NULL"), (dict(o=None), "ATTN_ERR_NULL"),
    (dict(lse=None), "ATTN_ERR_NULL"),
    (dict(B=0), "ATTN_ERR_SHAPE"), (dict(H=-1), "ATTN_ERR_SHAPE"),
    (dict(S=0), "ATTN_ERR_SHAPE"), (dict(D=0), "ATTN_ERR_SHAPE"),
    (dict(B=1 << 16, H=1 << 16, S=1), "ATTN_ERR_SHAPE"),
    (dict(B=1, H=1 << 20, S=1 << 12), "ATTN_ERR_SHAPE"),
    (dict(D=96), "ATTN_ERR_HEAD_DIM"), (dict(D=256), "ATTN_ERR_HEAD_DIM"),
    (dict(scale=math.nan), "ATTN_ERR_SCALE"), (dict(scale=math.inf), "ATTN_ERR_SCALE"),
    (dict(scale=-math.inf), "ATTN_ERR_SCALE"),
    (dict(o=Q), "ATTN_ERR_ALIAS"), (dict(lse=V + 100), "ATTN_ERR_ALIAS"),
    (dict(lse=O), "ATTN_ERR_ALIAS"),
])
def test_fused_validation(L, kw, code):
    assert call(L, **kw) == C[code]


def test_unfused_validation(L):
    need = L.attn_fwd_unfused_workspace_bytes(2, 3, 100)
    assert need == 2 * 3 * 100 * 128 * 6  # rows padded to 128 (a multiple of 64)
    assert L.attn_fwd_unfused_workspace_bytes(0, 3, 100) == 0
    W = 0x90000000
    args = (Q, K, V, O, LSE, 2, 3, 100, 128, 1, 0.1)
    assert L.attn_fwd_unfused(*args, None, need, None) == C["ATTN_ERR_WORKSPACE"]
    assert L.attn_fwd_unfused(*args, W, need - 1, None) == C["ATTN_ERR_WORKSPACE"]
    assert L.attn_fwd_unfused(*args, Q, need, None) == C["ATTN_ERR_ALIAS"]
    bad = (Q, K, V, O, LSE, 2, 3, 100, 100, 1, 0.1)
    assert L.attn_fwd_unfused(*bad, W, need, None) == C["ATTN_ERR_HEAD_DIM"]


def test_last_hip_error_starts_clear(L):
    assert L.attn_last_hip_error() == 0


def test_python_binding_rejects_cpu_tensors(L):
    import torch
    q = torch.zeros(1, 1, 4, 64, dtype=torch.float16)
    with pytest.raises(ValueError):
        attn.fwd(q, q, q, causal=True)
    with pytest.raises(TypeError):
        attn.fwd(q.float(), q, q, causal=True)


def splitkv_units(S, causal, splits):
    """Work units (query tile, key chunk) of one (batch, head): 64-row query
    tiles, 32-key tiles, chunks of at most ceil(ceil(S/32) / splits) tiles."""
    T = -(-S // 64)
    C = -(-(-(-S // 32)) // splits)
    units = 0
    for qt in range(T):
        kv_end = min(S, (qt + 1) * 64) if causal else S
        units += -(-(-(-kv_end // 32)) // C)
    return units, T


@pytest.mark.parametrize("S,causal,splits", [(1024, 1, 4), (1024, 0, 4), (1024, 1, 1),
                                             (300, 1, 3), (65, 0, 16), (1, 1, 8)])
def test_splitkv_workspace_bytes(L, S, causal, splits):
    units, T = splitkv_units(S, causal, splits)
    slot = 64 * 512 * 2 + 2 * 64 * 4   # fp16 O_c / l_c, then m and l in fp32
    expect = 0 if units == T else 2 * 3 * units * slot
    assert L.attn_fwd_splitkv_workspace_bytes(2, 3, S, 512, causal, splits) == expect
    if (S, causal, splits) == (1024, 1, 4):
        assert units == 40  # 1,1,1,1,2,2,2,2,3,3,3,3,4,4,4,4 chunks per query tile


def test_splitkv_validation(L):
    # D = 64, 128: the decode kernel with Sq = Sk, same workspace
    for D in (64, 128):
        n = L.attn_fwd_splitkv_workspace_bytes(1, 8, 1024, D, 1, 4)
        assert n > 0 and n == L.attn_fwd_decode_workspace_bytes(1, 8, 1024, 1024, D, 1, 4)
    assert L.attn_fwd_splitkv_workspace_bytes(1, 8, 1024, 512, 1, 0) == 0
    need = L.attn_fwd_splitkv_workspace_bytes(1, 2, 1024, 512, 1, 4)
    assert need > 0
    W = 0x90000000
    args = (Q, K, V, O, LSE, 1, 2, 1024, 512, 1, 0.1)
    assert L.attn_fwd_splitkv(*args, 4, None, need, None) == C["ATTN_ERR_WORKSPACE"]
    assert L.attn_fwd_splitkv(*args, 4, W, need - 1, None) == C["ATTN_ERR_WORKSPACE"]
    assert L.attn_fwd_splitkv(*args, 4, Q, need, None) == C["ATTN_ERR_ALIAS"]
    assert L.attn_fwd_splitkv(*args, 0, W, need, None) == C["ATTN_ERR_SPLITS"]
    d96 = (Q, K, V, O, LSE, 1, 2, 1024, 96, 1, 0.1)
    assert L.attn_fwd_splitkv(*d96, 4, W, need, None) == C["ATTN_ERR_HEAD_DIM"]
    d128 = (Q, K, V, O, LSE, 1, 2, 1024, 128, 1, 0.1)
    need128 = L.attn_fwd_splitkv_workspace_bytes(1, 2, 1024, 128, 1, 4)
    assert L.attn_fwd_splitkv(*d128, 4, W, need128 - 1, None) == C["ATTN_ERR_WORKSPACE"]
    assert L.attn_fwd_splitkv(*d128, 0, W, need128, None) == C["ATTN_ERR_SPLITS"]
    nul = (None, K, V, O, LSE, 1, 2, 1024, 512, 1, 0.1)
    assert L.attn_fwd_splitkv(*nul, 4, W, need, None) == C["ATTN_ERR_NULL"]


def decode_units(Sq, Sk, causal, splits):
    """Work units of one (batch, head) in the decode form: 64-row query tiles,
    64-key tiles, chunks of at most ceil(ceil(Sk/64) / splits) tiles, each
    tile's key range ending at its last row's visible key (bottom-right)."""
    Tq = -(-Sq // 64)
    C = -(-(-(-Sk // 64)) // splits)
    units = 0
    for qt in range(Tq):
        kv_end = min(Sk, min(Sq, (qt + 1) * 64) - 1 + (Sk - Sq) + 1) if causal else Sk
        units += -(-(-(-kv_end // 64)) // C)
    return units, Tq


@pytest.mark.parametrize("Sq,Sk,D,causal,splits", [(1, 4096, 128, 1, 8), (4, 8192, 64, 0, 3),
                                                   (130, 2000, 128, 1, 5), (64, 64, 64, 1, 1),
                                                   (200, 200, 128, 1, 4)])
def test_decode_workspace_bytes(L, Sq, Sk, D, causal, splits):
    units, Tq = decode_units(Sq, Sk, causal, splits)
    expect = 0 if units == Tq else 2 * 3 * units * (64 * D + 128) * 4
    assert L.attn_fwd_decode_workspace_bytes(2, 3, Sq, Sk, D, causal, splits) == expect


def test_decode_validation(L):
    need = L.attn_fwd_decode_workspace_bytes(1, 2, 1, 4096, 128, 1, 8)
    assert need == 1 * 2 * 8 * (64 * 128 + 128) * 4
    W = 0x90000000
    def dec(q=Q, k=K, v=V, o=O, lse=LSE, B=1, H=2, Sq=1, Sk=4096, D=128, causal=1,
            scale=0.1, splits=8, ws=W, wb=need):
        return L.attn_fwd_decode(q, k, v, o, lse, B, H, Sq, Sk, D, causal, scale, splits,
                                 ws, wb, None)
    assert dec(ws=None) == C["ATTN_ERR_WORKSPACE"]
    assert dec(wb=need - 1) == C["ATTN_ERR_WORKSPACE"]
    assert dec(ws=Q) == C["ATTN_ERR_ALIAS"]
    assert dec(splits=0) == C["ATTN_ERR_SPLITS"]
    assert dec(D=512) == C["ATTN_ERR_HEAD_DIM"]
    assert dec(Sq=5, Sk=4) == C["ATTN_ERR_SHAPE"]        # causal needs Sq <= Sk
    assert dec(Sk=0) == C["ATTN_ERR_SHAPE"]
    assert dec(q=None) == C["ATTN_ERR_NULL"]
    assert dec(scale=math.nan) == C["ATTN_ERR_SCALE"]
    assert dec(lse=O) == C["ATTN_ERR_ALIAS"]
    # one chunk per query tile needs no workspace
    assert L.attn_fwd_decode_workspace_bytes(1, 2, 1, 4096, 128, 1, 1) == 0


def test_bwd_workspace_bytes(L):
    assert L.attn_bwd_workspace_bytes(2, 3, 1000) == 2 * 3 * 1000 * 4
    assert L.attn_bwd_workspace_bytes(0, 3, 1000) == 0
    for D in (64, 128):
        assert L.attn_bwd_workspace_bytes_d(2, 3, 1000, D) == 2 * 3 * 1000 * 4
    # D = 512: S, dP (fp32), dS, P^T, dS^T (fp16) of S x Sp, Sp = S rounded up
    # to 64, plus one float per row
    sp = 1024
    assert L.attn_bwd_workspace_bytes_d(2, 3, 1000, 512) == 6 * (1000 * sp * 14 + 1000 * 4)
    assert L.attn_bwd_workspace_bytes_d(0, 3, 1000, 512) == 0


def test_bwd_validation(L):
    B, H, S, D = 1, 2, 1024, 128
    nt = B * H * S * D * 2
    # fake, disjoint device addresses: validation never dereferences them
    base = 0x80000000
    q, k, v, o, do, dq, dk, dv = (base + i * nt for i in range(8))
    lse = base + 8 * nt
    ws = lse + B * H * S * 4
    need = L.attn_bwd_workspace_bytes(B, H, S)
    def bwd(q=q, k=k, v=v, o=o, lse=lse, do=do, dq=dq, dk=dk, dv=dv, B=B, H=H, S=S, D=D,
            causal=1, scale=0.1, ws=ws, wb=need):
        return L.attn_bwd(q, k, v, o, lse, do, dq, dk, dv, B, H, S, D, causal, scale, ws, wb,
                          None)
    assert bwd(q=None) == C["ATTN_ERR_NULL"]
    assert bwd(do=None) == C["ATTN_ERR_NULL"]
    assert bwd(dv=None) == C["ATTN_ERR_NULL"]
    assert bwd(S=0) == C["ATTN_ERR_SHAPE"]
    # D = 512 needs its larger workspace
    assert bwd(D=512) == C["ATTN_ERR_WORKSPACE"]
    assert bwd(D=96) == C["ATTN_ERR_HEAD_DIM"]
    assert bwd(scale=math.inf) == C["ATTN_ERR_SCALE"]
    assert bwd(ws=None) == C["ATTN_ERR_WORKSPACE"]
    assert bwd(wb=need - 1) == C["ATTN_ERR_WORKSPACE"]
    assert bwd(dq=k) == C["ATTN_ERR_ALIAS"]          # output over an input
    assert bwd(dk=dq) == C["ATTN_ERR_ALIAS"]         # outputs over each other
    assert bwd(dv=dq + 2) == C["ATTN_ERR_ALIAS"]     # partial overlap
    assert bwd(ws=o) == C["ATTN_ERR_ALIAS"]          # workspace over an input
    assert bwd(ws=dk) == C["ATTN_ERR_ALIAS"]         # workspace over an output
    assert bwd(lse=dv) == C["ATTN_ERR_ALIAS"]


def test_default_split_counts():
    """Host heuristics for the default split counts: about one wave of
    workgroups on 256 CUs (decode: doubled while a chunk would exceed 64 key
    tiles), at least 1, at most one chunk per key tile."""
    import scaled_dot_product_attn_amd as a
    assert a.splitkv_splits(1, 8, 1024, True) == 3      # 256 work units
    assert a.splitkv_splits(4, 16, 2048, True) == 1     # already many query tiles
    assert a.splitkv_splits(1, 1, 333, True) == 16      # tiny: the cap
    assert a.decode_splits(1, 32, 1, 4096) == 8
    assert a.decode_splits(1, 32, 1, 16384) == 8
    assert a.decode_splits(1, 32, 1, 65536) == 16
    assert a.decode_splits(8, 32, 4, 8192) == 2
    assert a.decode_splits(1, 1, 1, 64) == 1            # one key tile


def test_slice_of_4gib_is_rejected(L):
    """Buffer descriptors address one (batch, head) slice with 32-bit byte
    offsets, so every entry point rejects a slice of 4 GiB or more before any
    launch (the largest accepted slice is one row less)."""
    big = 0x1_0000_0000_0000  # fake, far apart: validation never dereferences them
    q, k, v, o, lse = (big * (i + 1) for i in range(5))
    fw = lambda S, D: L.attn_fwd(q, k, v, o, lse, 1, 1, S, D, 1, 0.1, None)
    assert fw(1 << 24, 128) == C["ATTN_ERR_SHAPE"]          # 16M rows x 256 B = 4 GiB
    assert fw(1 << 22, 512) == C["ATTN_ERR_SHAPE"]          # 4M rows x 1 KB
    assert fw(1 << 25, 64) == C["ATTN_ERR_SHAPE"]
    W = big * 7
    assert L.attn_fwd_unfused(q, k, v, o, lse, 1, 1, 1 << 22, 512, 1, 0.1, W, 1 << 62,
                              None) == C["ATTN_ERR_SHAPE"]
    dec = lambda Sq, Sk: L.attn_fwd_decode(q, k, v, o, lse, 1, 1, Sq, Sk, 128, 1, 0.1, 1,
                                           W, 1 << 62, None)
    assert dec(1, 1 << 24) == C["ATTN_ERR_SHAPE"]           # the K/V cache slice
    bwd = L.attn_bwd(q, k, v, o, lse, big * 6, big * 8, big * 9, big * 10, 1, 1, 1 << 24, 128,
                     1, 0.1, W, 1 << 62, None)
    assert bwd == C["ATTN_ERR_SHAPE"]


def test_unit_counts_do_not_wrap(L):
    """The (query tile, key chunk) unit count of a long causal row with many
    splits exceeds 2^31; the library counts it in 64 bits, so the workspace
    size is exact and the launch is refused instead of running a wrapped
    grid."""
    S, splits = (1 << 22) - 64, 1 << 20      # D = 512: just under a 4 GiB slice
    units, T = splitkv_units(S, 1, splits)
    assert units > 2**31
    slot = 64 * 512 * 2 + 2 * 64 * 4
    assert L.attn_fwd_splitkv_workspace_bytes(1, 1, S, 512, 1, splits) == units * slot
    big = 0x1_0000_0000_0000
    q, k, v, o, lse = (big * (i + 1) for i in range(5))
    assert L.attn_fwd_splitkv(q, k, v, o, lse, 1, 1, S, 512, 1, 0.1, splits, big * 7,
                              units * slot, None) == C["ATTN_ERR_SHAPE"]
    Sq = Sk = (1 << 24) - 64                 # D = 128, decode form, 64-key tiles
    du, Tq = decode_units(Sq, Sk, 1, 1 << 20)
    assert du > 2**31
    assert L.attn_fwd_decode_workspace_bytes(1, 1, Sq, Sk, 128, 1, 1 << 20) == \
        du * (64 * 128 + 128) * 4
    assert L.attn_fwd_decode(q, k, v, o, lse, 1, 1, Sq, Sk, 128, 1, 0.1, 1 << 20, big * 7,
                             1 << 62, None) == C["ATTN_ERR_SHAPE"]


def test_decode_noalloc_validation(L):
    """attn_fwd_decode_noalloc: the decode checks, and ATTN_ERR_SCRATCH for a
    call whose workspace would exceed the static array, all before any HIP
    call."""
    cap = 32 << 20
    big = 0x1_0000_0000_0000  # fake, far apart: validation never dereferences them
    q_, k_, v_, o_, l_ = (big * (i + 1) for i in range(5))
    def nd(q=q_, k=k_, v=v_, o=o_, lse=l_, B=1, H=64, Sq=1, Sk=65536, D=128, causal=1,
           scale=0.1, splits=64):
        return L.attn_fwd_decode_noalloc(q, k, v, o, lse, B, H, Sq, Sk, D, causal, scale,
                                         splits, None)
    assert L.attn_fwd_decode_workspace_bytes(1, 64, 1, 65536, 128, 1, 64) > cap
    assert nd() == C["ATTN_ERR_SCRATCH"]
    assert nd(q=None) == C["ATTN_ERR_NULL"]
    assert nd(D=512) == C["ATTN_ERR_HEAD_DIM"]
    assert nd(Sq=5, Sk=4) == C["ATTN_ERR_SHAPE"]
    assert nd(splits=0) == C["ATTN_ERR_SPLITS"]
    assert nd(scale=math.nan) == C["ATTN_ERR_SCALE"]
    assert nd(lse=o_) == C["ATTN_ERR_ALIAS"]
    s = L.attn_status_string(C["ATTN_ERR_SCRATCH"]).decode()
    assert "scratch" in s
    assert attn.DECODE_NOALLOC_SCRATCH_BYTES == cap
