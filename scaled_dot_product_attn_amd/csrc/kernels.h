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

// Fused single-kernel forward, D = 64 or 128: two query tiles per workgroup
// of eight waves (causal pairs t, T-1-t).
hipError_t launch_fused_pair8_d64_d128(const FwdArgs& a);
// Fused single-kernel forward, D = 512 (head-dim halves summed in logit space).
hipError_t launch_fused_d512(const FwdArgs& a);
// Unfused ablation: QK -> S (fp32, workspace), softmax -> P (fp16, workspace)
// and LSE, PV -> O.  Three launches on a.stream.
hipError_t launch_unfused(const FwdArgs& a, void* workspace);
// Row stride (elements) of the unfused workspace matrices: S rounded up to 64.
int unfused_row_stride(int S);

}  // namespace attn
