// Internal interface between the C ABI (api.cpp) and the HIP kernels.
#pragma once
#include <hip/hip_runtime.h>

namespace attn {

struct FwdArgs {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    float* lse;
    int B, H, S, D;
    int causal;
    float scale;
    void* stream;
};

// Fused single-kernel forward, D = 64 or 128: one workgroup of four waves per
// query tile, two per CU, K/V tiles loaded straight into LDS, the next tile's
// Q K^T overlapped with the current tile's softmax.
hipError_t launch_fused_pipe_d64_d128(const FwdArgs& a);
// Fused single-kernel forward, D = 128, for shapes with many query tiles: one
// workgroup of four waves per 128-row query tile, two per CU, every wave
// owning 32 complete rows and walking the keys in 32-key chunks.
hipError_t launch_fused_rows_d128(const FwdArgs& a);
// Fused single-kernel forward, D = 512 (head-dim halves summed in logit space).
hipError_t launch_fused_d512(const FwdArgs& a);
// Split-KV forward, D = 512: every query tile's key range cut into chunks of
// at most ceil(ceil(S/32) / splits) 32-key tiles, partial states in
// `workspace`, merged by a second kernel.
hipError_t launch_splitkv_d512(const FwdArgs& a, int splits, void* workspace);
// Floats of workspace that launch_splitkv_d512 needs, and its number of work
// units per (batch, head).
size_t splitkv_d512_workspace_floats(int B, int H, int S, int causal, int splits);
long long splitkv_d512_units(int S, int causal, int splits);
// Decode form: Sq query rows against Sk keys (causal aligned bottom-right),
// D = 64 or 128, key ranges in chunks of at most ceil(ceil(Sk/64) / splits)
// 64-key tiles, partial states in `workspace` merged by a second kernel.
struct DecArgs {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    float* lse;
    int B, H, Sq, Sk, D;
    int causal;
    float scale;
    int splits;
    void* workspace;
    void* stream;
};
hipError_t launch_decode(const DecArgs& a);
// The decode workspace that needs no allocation: a static device array of
// ATTN_DECODE_NOALLOC_SCRATCH_BYTES, one per GPU.  *ptr = its address on the
// current device (looked up once per device, then cached).
hipError_t decode_scratch(void** ptr);
// Work units per (batch, head) and workspace floats (0 when no query tile is
// split) of launch_decode.
long long decode_units(int Sq, int Sk, int causal, int splits);
size_t decode_workspace_floats(int B, int H, int Sq, int Sk, int D, int causal, int splits);
// Unfused ablation: QK -> S (fp32, workspace), softmax -> P (fp16, workspace)
// and LSE, PV -> O.  Three launches on a.stream.
hipError_t launch_unfused(const FwdArgs& a, void* workspace);
// Row stride (elements) of the unfused workspace matrices: S rounded up to 64.
int unfused_row_stride(int S);

// Backward, D = 64 or 128: dQ, dK, dV (fp16) from Q, K, V, the forward's O
// and LSE, and dO.  `workspace` holds B H S floats (dO.O per row).  Two
// launches on a.stream, no atomics.
struct BwdArgs {
    const void* q;
    const void* k;
    const void* v;
    const void* o;
    const float* lse;
    const void* dout;
    void* dq;
    void* dk;
    void* dv;
    int B, H, S, D;
    int causal;
    float scale;
    void* workspace;
    void* stream;
};
hipError_t launch_bwd(const BwdArgs& a);
// Backward, D = 512, with S, dP, dS, P^T and dS^T materialised in `workspace`
// (bwd512_workspace_bytes), built from the unfused ablation's kernels.
size_t bwd512_workspace_bytes(int B, int H, int S);
hipError_t launch_bwd512(const BwdArgs& a);

}  // namespace attn
