// Fused scaled-dot-product attention forward for gfx950 (CDNA4), D in {64, 128}.
//
//   O = softmax(scale * Q K^T + causal mask) V,   LSE = log sum_j exp(scale q.k_j)
//
// fp16 Q/K/V/O, fp32 accumulation and fp32 LSE.  The score matrix never leaves
// the chip: one kernel keeps the scores in registers ("An Optimal Mapper Meets
// a Real GPU", section "Ground rules": the alternative to a multi-kernel
// pipeline with global workspaces is one fused kernel with register-resident
// scores), and rescales the running output when a later key tile raises the
// row maximum (the "O rescale (kt>0)" step of the STAGE_D.md notes).
//
// Work decomposition
//   * one workgroup = 4 waves = 128 query rows of one (batch, head); each wave
//     owns 32 consecutive rows for the whole key loop.
//   * keys stream in tiles of 64 through double-buffered LDS: K row-major,
//     V transposed.  Global loads for tile j+1 are in flight while tile j is
//     computed.  Under causal masking tiles past the diagonal are never loaded
//     and 32-key blocks a wave cannot see are skipped.
//   * S^T = K Q^T on v_mfma_f32_32x32x16_f16 (A = 32 keys x 16 dims from LDS,
//     B = Q^T fragment held in VGPRs for the whole loop).  In the 32x32
//     accumulator a lane holds one query column and 16 keys, so the row max
//     needs one exchange between the two 32-lane halves and the per-row
//     statistics m, l live in the lane that owns the query.
//   * O^T += V^T P^T on the same MFMA: P^T (fp16, round-to-nearest-even) is the
//     B operand straight from the softmax registers, and V^T comes from LDS in
//     a key order that matches the accumulator layout (keys 4..7 and 8..11 of
//     each 16-key group swapped), so no lane shuffles are needed.
//   * exp2 on v_exp_f32 with scale*log2(e) folded into one FMA; the O^T
//     rescale is per lane.
//
// MFMA lane layouts used (32x32x16, wave64, g = lane / 32, n = lane % 32):
//   A[m][k]: lane holds m = n, k = 8g .. 8g+7
//   B[k][n]: lane holds n = n, k = 8g .. 8g+7
//   C[m][n]: register r holds m = 8(r/4) + 4g + r%4, n = n
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace attn {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kNegInf = -__builtin_inff();
constexpr float kLn2 = 0.693147180559945309417f;

template <int D>
struct Cfg {
    static constexpr int NW = 4;             // waves per workgroup
    static constexpr int NT = NW * 64;       // threads per workgroup
    static constexpr int BM = 32 * NW;       // query rows per workgroup
    static constexpr int BN = 64;            // keys per tile
    static constexpr int KSTR = D + 8;       // K row stride in LDS (halfs); +16 B
    static constexpr int VSTR = BN + 8;      // V^T row stride in LDS (halfs)
    static constexpr int K_HALFS = BN * KSTR;
    static constexpr int V_HALFS = D * VSTR;
    static constexpr int STAGE = K_HALFS + V_HALFS;
    static constexpr int LDS_BYTES = 2 * STAGE * 2;
    static constexpr int CPR = D / 8;                 // 16-byte chunks per row
    static constexpr int KCH = BN * CPR / NT;         // K chunks per thread
    static constexpr int VR = BN * D / 8 / NT;        // keys per thread (V^T)
    static constexpr int VKG = BN / VR;               // key groups per d-block
    static_assert(KCH * NT == BN * CPR, "K tile must split evenly");
    static_assert(VR == 2 || VR == 4, "V transpose handles 2 or 4 keys");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
};

// Position of key x (0..63) inside a V^T row: bits 2 and 3 swapped, so that
// the 8 keys a lane half feeds to one PV MFMA step are contiguous.
__device__ __forceinline__ int vt_pos(int x) {
    return (x & ~12) | ((x & 4) << 1) | ((x & 8) >> 1);
}

__device__ __forceinline__ float xor32(float x) {
    return __shfl_xor(x, 32, 64);
}

template <int D, bool CAUSAL>
__global__ void __launch_bounds__(256, 2)
fwd_kernel(const _Float16* __restrict__ Q, const _Float16* __restrict__ K,
           const _Float16* __restrict__ V, _Float16* __restrict__ O,
           float* __restrict__ LSE, int BH, int S, float c_scale, uint32_t qsign)
{
    using C = Cfg<D>;
    __shared__ __attribute__((aligned(16))) _Float16 lds[2 * C::STAGE];

    const int T = (S + C::BM - 1) / C::BM;
    const int bh = blockIdx.x % BH;
    int qt = blockIdx.x / BH;
    if (CAUSAL) qt = T - 1 - qt;  // longest rows first
    const int q0 = qt * C::BM;
    const size_t base = (size_t)bh * S * D;

    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6;
    const int g = lane >> 5, n = lane & 31;
    const int row = q0 + 32 * w + n;        // the query this lane owns
    const int r_lo = q0 + 32 * w, r_hi = r_lo + 31;

    // Q^T fragments for the whole key loop: lane holds Q[row][16kk + 8g .. +7].
    half8 qf[D / 16];
    {
        const bool ok = row < S;
        const u32x4* src = reinterpret_cast<const u32x4*>(Q + base + (size_t)(ok ? row : 0) * D);
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) {
            u32x4 x = ok ? src[2 * kk + g] : u32x4{0, 0, 0, 0};
            x ^= qsign;  // exact negation when the scale is negative
            qf[kk] = __builtin_bit_cast(half8, x);
        }
    }

    const int kv_end = CAUSAL ? min(S, q0 + C::BM) : S;
    const int nT = (kv_end + C::BN - 1) / C::BN;

    // Staging registers for the next tile.
    u32x4 kreg[C::KCH];
    u32x4 vreg[C::VR];
    const int vkb = tid % C::VKG, vdb = tid / C::VKG;

    auto gload = [&](int j0) {
#pragma unroll
        for (int u = 0; u < C::KCH; ++u) {
            const int ci = tid + C::NT * u;
            const int r = ci / C::CPR, c8 = ci % C::CPR;
            const int key = j0 + r;
            kreg[u] = key < S ? *reinterpret_cast<const u32x4*>(K + base + (size_t)key * D + 8 * c8)
                              : u32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int v = 0; v < C::VR; ++v) {
            const int key = j0 + vkb * C::VR + v;
            vreg[v] = key < S ? *reinterpret_cast<const u32x4*>(V + base + (size_t)key * D + 8 * vdb)
                              : u32x4{0, 0, 0, 0};
        }
    };

    auto lstore = [&](int buf) {
        _Float16* Ks = lds + buf * C::STAGE;
        _Float16* Vt = Ks + C::K_HALFS;
#pragma unroll
        for (int u = 0; u < C::KCH; ++u) {
            const int ci = tid + C::NT * u;
            const int r = ci / C::CPR, c8 = ci % C::CPR;
            *reinterpret_cast<u32x4*>(Ks + r * C::KSTR + 8 * c8) = kreg[u];
        }
        // Transpose VR keys x 8 dims into 8 rows of V^T.
        const int pos = vt_pos(vkb * C::VR);
#pragma unroll
        for (int dd = 0; dd < 8; ++dd) {
            const int wi = dd >> 1;
            const bool hi = dd & 1;
            uint32_t pk[C::VR / 2];
#pragma unroll
            for (int v = 0; v < C::VR / 2; ++v) {
                const uint32_t a = vreg[2 * v][wi], b = vreg[2 * v + 1][wi];
                pk[v] = hi ? ((a >> 16) | (b & 0xffff0000u)) : ((a & 0xffffu) | (b << 16));
            }
            _Float16* dst = Vt + (8 * vdb + dd) * C::VSTR + pos;
            if constexpr (C::VR == 4)
                *reinterpret_cast<u32x2*>(dst) = u32x2{pk[0], pk[1]};
            else
                *reinterpret_cast<uint32_t*>(dst) = pk[0];
        }
    };

    float m = kNegInf;  // running max of the scaled logits, log2 units
    float l = 0.f;      // this lane's share of the running row sum
    floatx16 o[D / 32];
#pragma unroll
    for (int b = 0; b < D / 32; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[b][r] = 0.f;

    gload(0);
    lstore(0);
    __syncthreads();

    for (int j = 0; j < nT; ++j) {
        const int j0 = j * C::BN;
        if (j + 1 < nT) gload(j0 + C::BN);
        const _Float16* Ks = lds + (j & 1) * C::STAGE;
        const _Float16* Vt = Ks + C::K_HALFS;

        const bool wave_skip = CAUSAL && j0 > r_hi;  // every key is in this wave's future
        if (!wave_skip) {
            const bool need_mask = (CAUSAL && j0 + C::BN - 1 > r_lo) || (j0 + C::BN > S);
            bool blk_on[2];
            floatx16 s[2];
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                blk_on[c] = !(CAUSAL && j0 + 32 * c > r_hi);
#pragma unroll
                for (int r = 0; r < 16; ++r) s[c][r] = 0.f;
                if (blk_on[c]) {
                    const _Float16* kp = Ks + (32 * c + n) * C::KSTR + 8 * g;
#pragma unroll
                    for (int kk = 0; kk < D / 16; ++kk) {
                        const half8 a = *reinterpret_cast<const half8*>(kp + 16 * kk);
                        s[c] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, qf[kk], s[c], 0, 0, 0);
                    }
                }
            }

            // visibility of each accumulator entry (only on boundary tiles)
            auto visible = [&](int c, int r) {
                const int key = j0 + 32 * c + 8 * (r >> 2) + 4 * g + (r & 3);
                return blk_on[c] && key < S && (!CAUSAL || key <= row);
            };

            float mx = kNegInf;
#pragma unroll
            for (int c = 0; c < 2; ++c)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float x = (need_mask && !visible(c, r)) ? kNegInf : s[c][r];
                    mx = fmaxf(mx, x);
                }
            mx = fmaxf(mx, xor32(mx));
            // A row with no visible key in this tile keeps its old max; clamping
            // keeps c_scale * mx finite for c_scale = 0.
            const float m_new = fmaxf(m, c_scale * fmaxf(mx, -3.402823466e38f));
            const float alpha = __builtin_amdgcn_exp2f(m - m_new);
            m = m_new;

            float psum = 0.f;
            half8 pf[4];
#pragma unroll
            for (int c = 0; c < 2; ++c)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[c][r], c_scale, -m_new));
                    if (need_mask && !visible(c, r)) p = 0.f;
                    psum += p;
                    pf[2 * c + (r >> 3)][r & 7] = (_Float16)p;
                }
            l = l * alpha + psum;
#pragma unroll
            for (int b = 0; b < D / 32; ++b)
#pragma unroll
                for (int r = 0; r < 16; ++r) o[b][r] *= alpha;

#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                if (!blk_on[ks >> 1]) continue;
                const _Float16* vp = Vt + n * C::VSTR + 16 * ks + 8 * g;
#pragma unroll
                for (int b = 0; b < D / 32; ++b) {
                    const half8 a = *reinterpret_cast<const half8*>(vp + 32 * b * C::VSTR);
                    o[b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, pf[ks], o[b], 0, 0, 0);
                }
            }
        }

        if (j + 1 < nT) lstore((j + 1) & 1);
        __syncthreads();
    }

    // Epilogue: O = O^T / l in fp16 (round to nearest even), LSE in natural log.
    const float lt = l + xor32(l);
    const float inv = 1.0f / lt;
    if (row < S) {
        _Float16* orow = O + base + (size_t)row * D;
#pragma unroll
        for (int b = 0; b < D / 32; ++b)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                u32x2 pk;
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const _Float16 lo = (_Float16)(o[b][4 * q4 + 2 * h] * inv);
                    const _Float16 hi = (_Float16)(o[b][4 * q4 + 2 * h + 1] * inv);
                    pk[h] = (uint32_t)__builtin_bit_cast(uint16_t, lo) |
                            ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
                }
                *reinterpret_cast<u32x2*>(orow + 32 * b + 8 * q4 + 4 * g) = pk;
            }
        if (g == 0) LSE[(size_t)bh * S + row] = (m + __builtin_amdgcn_logf(lt)) * kLn2;
    }
}

template <int D, bool CAUSAL>
hipError_t launch(const FwdArgs& a) {
    using C = Cfg<D>;
    const int T = (a.S + C::BM - 1) / C::BM;
    const long long blocks = (long long)a.B * a.H * T;
    const float c_scale = fabsf(a.scale) * 1.44269504088896340736f;
    const uint32_t qsign = a.scale < 0.f ? 0x80008000u : 0u;
    hipLaunchKernelGGL((fwd_kernel<D, CAUSAL>), dim3((unsigned)blocks), dim3(C::NT), 0,
                       (hipStream_t)a.stream,
                       (const _Float16*)a.q, (const _Float16*)a.k, (const _Float16*)a.v,
                       (_Float16*)a.o, a.lse, a.B * a.H, a.S, c_scale, qsign);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fused_d64_d128(const FwdArgs& a) {
    if (a.D == 64) return a.causal ? launch<64, true>(a) : launch<64, false>(a);
    return a.causal ? launch<128, true>(a) : launch<128, false>(a);
}

}  // namespace attn
