// C ABI of the attention forward (declared in include/attn.h).
//
// Every entry point validates its arguments before touching HIP, so the
// error paths run (and are tested) on machines without a GPU.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "attn.h"
#include "kernels.h"

namespace {

thread_local int g_last_hip_error = 0;

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return x < y + nb && y < x + na;
}

// Buffer descriptors address one (batch, head) slice with 32-bit offsets.
constexpr long long kMaxSliceBytes = 1LL << 32;

// Shared argument checks of the fused and unfused forward.
int validate(const void* q, const void* k, const void* v, const void* o,
             const float* lse, int B, int H, int S, int D, float scale) {
    if (!q || !k || !v || !o || !lse) return ATTN_ERR_NULL;
    if (B < 1 || H < 1 || S < 1 || D < 1) return ATTN_ERR_SHAPE;
    // Kernels index rows with 32-bit ints and launch B*H*ceil(S/32) groups at most.
    const long long bh = (long long)B * H;
    if (bh > INT32_MAX || (long long)S > INT32_MAX / 2 || bh * S > INT32_MAX ||
        bh * ((S + 31) / 32) > INT32_MAX || (long long)S * D * 2 >= kMaxSliceBytes)
        return ATTN_ERR_SHAPE;
    if (!attn_head_dim_supported(D)) return ATTN_ERR_HEAD_DIM;
    if (!isfinite(scale)) return ATTN_ERR_SCALE;
    const size_t nt = (size_t)bh * S * D * 2, nl = (size_t)bh * S * 4;
    if (overlaps(o, nt, q, nt) || overlaps(o, nt, k, nt) || overlaps(o, nt, v, nt) ||
        overlaps(lse, nl, q, nt) || overlaps(lse, nl, k, nt) || overlaps(lse, nl, v, nt) ||
        overlaps(lse, nl, o, nt))
        return ATTN_ERR_ALIAS;
    return ATTN_OK;
}

// Argument checks shared by the two decode entry points (everything but the
// workspace).
int validate_decode(const void* q, const void* k, const void* v, const void* o,
                    const float* lse, int B, int H, int Sq, int Sk, int D, int causal,
                    float scale, int splits) {
    if (!q || !k || !v || !o || !lse) return ATTN_ERR_NULL;
    if (B < 1 || H < 1 || Sq < 1 || Sk < 1 || D < 1) return ATTN_ERR_SHAPE;
    const long long bh = (long long)B * H;
    if (bh > INT32_MAX || bh * Sq > INT32_MAX / 2 || bh * Sk > INT32_MAX / 2 ||
        (causal && Sq > Sk) || (long long)Sq * D * 2 >= kMaxSliceBytes ||
        (long long)Sk * D * 2 >= kMaxSliceBytes)
        return ATTN_ERR_SHAPE;
    if (D != 64 && D != 128) return ATTN_ERR_HEAD_DIM;
    if (!isfinite(scale)) return ATTN_ERR_SCALE;
    if (splits < 1) return ATTN_ERR_SPLITS;
    if (bh * attn::decode_units(Sq, Sk, causal != 0, splits) > INT32_MAX ||
        bh * ((Sq + 63) / 64) * 8 > INT32_MAX)
        return ATTN_ERR_SHAPE;
    const size_t nq = (size_t)bh * Sq * D * 2, nk = (size_t)bh * Sk * D * 2,
                 nl = (size_t)bh * Sq * 4;
    if (overlaps(o, nq, q, nq) || overlaps(o, nq, k, nk) || overlaps(o, nq, v, nk) ||
        overlaps(lse, nl, q, nq) || overlaps(lse, nl, k, nk) || overlaps(lse, nl, v, nk) ||
        overlaps(lse, nl, o, nq))
        return ATTN_ERR_ALIAS;
    return ATTN_OK;
}

int launched(hipError_t e) {
    g_last_hip_error = (int)e;
    return e == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

}  // namespace

extern "C" {

int attn_head_dim_supported(int D) { return D == 64 || D == 128 || D == 512; }

int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
             int B, int H, int S, int D, int causal, float scale, void* stream) {
    const int st = validate(q, k, v, o, lse, B, H, S, D, scale);
    if (st != ATTN_OK) return st;
    const attn::FwdArgs a{q, k, v, o, lse, B, H, S, D, causal != 0, scale, stream};
    if (D == 512) return launched(attn::launch_fused_d512(a));
    // D = 128 with enough 128-row query tiles: the 128-row kernel (half the
    // staged bytes per FLOP, no key merge); otherwise the 64-row kernel,
    // whose waves split the keys of a tile and so keep every CU busy on fewer
    // rows.  Enough: causal, two tiles for each of the 256 CUs (with fewer,
    // the heaviest tiles of the triangle run alone and the 64-row kernel's
    // heavy/light pairs are faster); non-causal, one per CU (equal tiles).
    if (D == 128 && (long long)B * H * ((S + 127) / 128) >= (causal ? 512 : 256))
        return launched(attn::launch_fused_rows_d128(a));
    return launched(attn::launch_fused_pipe_d64_d128(a));
}

size_t attn_fwd_unfused_workspace_bytes(int B, int H, int S) {
    if (B < 1 || H < 1 || S < 1) return 0;
    // S as fp32 plus P as fp16, each [B, H, S, Sp], Sp = S rounded up to 64
    return (size_t)B * H * S * attn::unfused_row_stride(S) * (4 + 2);
}

int attn_fwd_unfused(const void* q, const void* k, const void* v, void* o,
                     float* lse, int B, int H, int S, int D, int causal,
                     float scale, void* workspace, size_t workspace_bytes,
                     void* stream) {
    const int st = validate(q, k, v, o, lse, B, H, S, D, scale);
    if (st != ATTN_OK) return st;
    // the Q K^T kernel's grid: (batch, head, 64-row query tile, chunk of 4 key tiles)
    const long long tq = (S + 63) / 64;
    if ((long long)B * H * tq * ((tq + 3) / 4) > INT32_MAX) return ATTN_ERR_SHAPE;
    const size_t need = attn_fwd_unfused_workspace_bytes(B, H, S);
    if (!workspace || workspace_bytes < need) return ATTN_ERR_WORKSPACE;
    const size_t nt = (size_t)B * H * S * D * 2, nl = (size_t)B * H * S * 4;
    if (overlaps(workspace, need, q, nt) || overlaps(workspace, need, k, nt) ||
        overlaps(workspace, need, v, nt) || overlaps(workspace, need, o, nt) ||
        overlaps(workspace, need, lse, nl))
        return ATTN_ERR_ALIAS;
    const attn::FwdArgs a{q, k, v, o, lse, B, H, S, D, causal != 0, scale, stream};
    return launched(attn::launch_unfused(a, workspace));
}

size_t attn_fwd_splitkv_workspace_bytes(int B, int H, int S, int D, int causal, int splits) {
    // D = 64, 128: the decode kernel with Sq = Sk = S (its bottom-right causal
    // alignment is then attn_fwd's)
    if (D == 64 || D == 128) return attn_fwd_decode_workspace_bytes(B, H, S, S, D, causal, splits);
    if (B < 1 || H < 1 || S < 1 || D != 512 || splits < 1) return 0;
    const int T = (S + 63) / 64;
    if (attn::splitkv_d512_units(S, causal != 0, splits) == T) return 0;  // nothing is split
    return attn::splitkv_d512_workspace_floats(B, H, S, causal != 0, splits) * sizeof(float);
}

int attn_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse,
                     int B, int H, int S, int D, int causal, float scale, int splits,
                     void* workspace, size_t workspace_bytes, void* stream) {
    if (D == 64 || D == 128)
        return attn_fwd_decode(q, k, v, o, lse, B, H, S, S, D, causal, scale, splits, workspace,
                               workspace_bytes, stream);
    const int st = validate(q, k, v, o, lse, B, H, S, D, scale);
    if (st != ATTN_OK) return st;
    if (D != 512) return ATTN_ERR_HEAD_DIM;
    if (splits < 1) return ATTN_ERR_SPLITS;
    // one workgroup per (batch, head, work unit), and per 8 rows in the merge
    if ((long long)B * H * attn::splitkv_d512_units(S, causal != 0, splits) > INT32_MAX ||
        (long long)B * H * ((S + 63) / 64) * 8 > INT32_MAX)
        return ATTN_ERR_SHAPE;
    const size_t need = attn_fwd_splitkv_workspace_bytes(B, H, S, D, causal, splits);
    if (need > 0) {
        if (!workspace || workspace_bytes < need) return ATTN_ERR_WORKSPACE;
        const size_t nt = (size_t)B * H * S * D * 2, nl = (size_t)B * H * S * 4;
        if (overlaps(workspace, need, q, nt) || overlaps(workspace, need, k, nt) ||
            overlaps(workspace, need, v, nt) || overlaps(workspace, need, o, nt) ||
            overlaps(workspace, need, lse, nl))
            return ATTN_ERR_ALIAS;
    }
    const attn::FwdArgs a{q, k, v, o, lse, B, H, S, D, causal != 0, scale, stream};
    return launched(attn::launch_splitkv_d512(a, splits, need > 0 ? workspace : nullptr));
}

size_t attn_fwd_decode_workspace_bytes(int B, int H, int Sq, int Sk, int D, int causal,
                                       int splits) {
    if (B < 1 || H < 1 || Sq < 1 || Sk < 1 || (D != 64 && D != 128) || splits < 1) return 0;
    return attn::decode_workspace_floats(B, H, Sq, Sk, D, causal != 0, splits) * sizeof(float);
}

int attn_fwd_decode(const void* q, const void* k, const void* v, void* o, float* lse,
                    int B, int H, int Sq, int Sk, int D, int causal, float scale, int splits,
                    void* workspace, size_t workspace_bytes, void* stream) {
    const int st = validate_decode(q, k, v, o, lse, B, H, Sq, Sk, D, causal, scale, splits);
    if (st != ATTN_OK) return st;
    const long long bh = (long long)B * H;
    const size_t nq = (size_t)bh * Sq * D * 2, nk = (size_t)bh * Sk * D * 2,
                 nl = (size_t)bh * Sq * 4;
    const size_t need = attn_fwd_decode_workspace_bytes(B, H, Sq, Sk, D, causal, splits);
    if (need > 0) {
        if (!workspace || workspace_bytes < need) return ATTN_ERR_WORKSPACE;
        if (overlaps(workspace, need, q, nq) || overlaps(workspace, need, k, nk) ||
            overlaps(workspace, need, v, nk) || overlaps(workspace, need, o, nq) ||
            overlaps(workspace, need, lse, nl))
            return ATTN_ERR_ALIAS;
    }
    const attn::DecArgs a{q, k, v, o, lse, B, H, Sq, Sk, D, causal != 0, scale, splits,
                          need > 0 ? workspace : nullptr, stream};
    return launched(attn::launch_decode(a));
}

int attn_fwd_decode_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                            int B, int H, int Sq, int Sk, int D, int causal, float scale,
                            int splits, void* stream) {
    const int st = validate_decode(q, k, v, o, lse, B, H, Sq, Sk, D, causal, scale, splits);
    if (st != ATTN_OK) return st;
    const size_t need = attn_fwd_decode_workspace_bytes(B, H, Sq, Sk, D, causal, splits);
    if (need > ATTN_DECODE_NOALLOC_SCRATCH_BYTES) return ATTN_ERR_SCRATCH;
    void* scratch = nullptr;
    if (need > 0) {
        const hipError_t e = attn::decode_scratch(&scratch);
        if (e != hipSuccess) return launched(e);
    }
    const attn::DecArgs a{q, k, v, o, lse, B, H, Sq, Sk, D, causal != 0, scale, splits,
                          scratch, stream};
    return launched(attn::launch_decode(a));
}

size_t attn_bwd_workspace_bytes(int B, int H, int S) {
    if (B < 1 || H < 1 || S < 1) return 0;
    return (size_t)B * H * S * sizeof(float);  // dO . O per row
}

size_t attn_bwd_workspace_bytes_d(int B, int H, int S, int D) {
    if (D == 512) {
        if (B < 1 || H < 1 || S < 1) return 0;
        return attn::bwd512_workspace_bytes(B, H, S);
    }
    return attn_bwd_workspace_bytes(B, H, S);
}

int attn_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
             const void* dout, void* dq, void* dk, void* dv, int B, int H, int S, int D,
             int causal, float scale, void* workspace, size_t workspace_bytes, void* stream) {
    if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv) return ATTN_ERR_NULL;
    if (B < 1 || H < 1 || S < 1 || D < 1) return ATTN_ERR_SHAPE;
    const long long bh = (long long)B * H;
    // rows are indexed with 32-bit ints; one workgroup per (batch, head, 64-row tile)
    if (bh > INT32_MAX || (long long)S > INT32_MAX / 2 || bh * S > INT32_MAX / 2 ||
        bh * ((S + 63) / 64) > INT32_MAX || (long long)S * D * 2 >= kMaxSliceBytes)
        return ATTN_ERR_SHAPE;
    if (D != 64 && D != 128 && D != 512) return ATTN_ERR_HEAD_DIM;
    if (!isfinite(scale)) return ATTN_ERR_SCALE;
    if (D == 512) {
        // the materialised form's grids: Q K^T (query tile, 4-key-tile chunk)
        // and the dS pass (query tile, key tile), per (batch, head)
        const long long tq = (S + 63) / 64;
        if (bh * tq * tq > INT32_MAX) return ATTN_ERR_SHAPE;
    }
    const size_t need = attn_bwd_workspace_bytes_d(B, H, S, D);
    if (!workspace || workspace_bytes < need) return ATTN_ERR_WORKSPACE;
    const size_t nt = (size_t)bh * S * D * 2, nl = (size_t)bh * S * 4;
    const void* in[7] = {q, k, v, o, dout, lse, workspace};
    const size_t in_n[7] = {nt, nt, nt, nt, nt, nl, need};
    void* out[3] = {dq, dk, dv};
    for (int i = 0; i < 3; ++i) {
        for (int j = 0; j < 7; ++j)
            if (overlaps(out[i], nt, in[j], in_n[j])) return ATTN_ERR_ALIAS;
        for (int j = i + 1; j < 3; ++j)
            if (overlaps(out[i], nt, out[j], nt)) return ATTN_ERR_ALIAS;
    }
    for (int j = 0; j < 6; ++j)
        if (overlaps(workspace, need, in[j], in_n[j])) return ATTN_ERR_ALIAS;
    const attn::BwdArgs a{q, k, v, o, lse, dout, dq, dk, dv, B, H, S, D,
                          causal != 0, scale, workspace, stream};
    return launched(D == 512 ? attn::launch_bwd512(a) : attn::launch_bwd(a));
}

const char* attn_status_string(int status) {
    switch (status) {
        case ATTN_OK: return "ok";
        case ATTN_ERR_NULL: return "a required pointer is NULL";
        case ATTN_ERR_SHAPE:
            return "B, H and S must be >= 1, the sizes must fit 32-bit row indices and one "
                   "(batch, head) slice must stay under 4 GiB";
        case ATTN_ERR_HEAD_DIM: return "unsupported head dimension (supported: 64, 128, 512)";
        case ATTN_ERR_SCALE: return "scale must be finite";
        case ATTN_ERR_LAUNCH: return "HIP kernel launch failed (see attn_last_hip_error)";
        case ATTN_ERR_WORKSPACE:
            return "workspace is NULL or smaller than the entry point's *_workspace_bytes size";
        case ATTN_ERR_ALIAS: return "an output buffer overlaps another buffer";
        case ATTN_ERR_SPLITS: return "splits must be >= 1";
        case ATTN_ERR_SCRATCH:
            return "the call needs more workspace than the static scratch array holds "
                   "(ATTN_DECODE_NOALLOC_SCRATCH_BYTES): use attn_fwd_decode with a workspace";
        default: return "unknown status";
    }
}

int attn_last_hip_error(void) { return g_last_hip_error; }

}  // extern "C"
