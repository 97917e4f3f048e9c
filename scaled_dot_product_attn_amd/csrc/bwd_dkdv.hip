// dK/dV half of the attention backward (layout, helpers and the derivation are
// in bwd_common.h), and launch_bwd, which enqueues both halves.
#include "bwd_common.h"

namespace attn {
namespace {

using namespace detail;

// dK and dV for one 64-key tile.  Wave (lo, hi): keys 32lo .. +31 of the tile,
// query rows 32hi .. +31 of every query tile that sees the keys.
//   S  = Q K^T  : A = Q rows, B = this wave's K rows
//   dP = dO V^T : A = dO rows, B = this wave's V rows
//   dV^T += dO^T P, dK^T += Q^T dS : A = dO / Q columns (transposed LDS
//                 reads), B = P / dS (score registers); the accumulators hold
//                 lane = key, registers = head dims, so that rows are stored
//                 from registers
// Every operand comes from LDS (the K and V tiles stay there for the whole
// walk, one stage holds the current Q and dO tiles), so that a wave holds
// the two accumulators, the scores and a few fragments in flight: at most 256
// registers, two workgroups per CU, and one workgroup's loads and barriers
// run under the other's products.
template <int D, bool CAUSAL>
__global__ void __launch_bounds__(256, 2)
bwd_dkdv_kernel(const _Float16* __restrict__ Q, const _Float16* __restrict__ K,
                const _Float16* __restrict__ V, const _Float16* __restrict__ dO,
                const float* __restrict__ dlt, const float* __restrict__ LSE,
                _Float16* __restrict__ dK, _Float16* __restrict__ dV,
                int BH, int S, float cs, float scale)
{
    using G = GeoB<D>;
    constexpr int NB = G::NB;
    constexpr int PIECES = G::TILE * 2 / 1024 / G::NW;  // 1 KB pieces of a tile per wave
    constexpr int RPP = 1024 / (2 * D);                 // rows per piece
    // K tile, V tile, Q tile, dO tile, then LSE log2(e) [64] and Dlt [64]
    __shared__ __attribute__((aligned(1024))) _Float16 lds[4 * G::TILE + 2 * 64 * 2];
    static_assert(4 * (NB * 4) * 64 * 16 <= (4 * G::TILE + 2 * 64 * 2) * 2, "merge buffers fit");
    using LdsPtr = __attribute__((address_space(3))) void*;
    _Float16* const Ks = lds;
    _Float16* const Vs = lds + G::TILE;
    _Float16* const Qs = lds + 2 * G::TILE;
    _Float16* const Os = lds + 3 * G::TILE;
    float* const fl = reinterpret_cast<float*>(lds + 4 * G::TILE);

    const int T = (S + 63) / 64;
    const int bh = blockIdx.x % BH;
    // causal: the first half of the grid takes the key tiles that see the
    // most query tiles (0, 1, ...), the second half the others (T-1, T-2,
    // ...), so that workgroups i and i + grid/2, which share a CU when the
    // grid fills the chip once, carry T+1 query tiles between them
    const int j = blockIdx.x / BH;
    const int kt = CAUSAL ? (j < (T + 1) / 2 ? j : T - 1 - (j - (T + 1) / 2)) : j;
    const int k0 = kt * 64;

    Bwd<D> f;
    f.S = S;
    f.tid = threadIdx.x;
    f.lane = threadIdx.x & 63;
    f.g = f.lane >> 5;
    f.n = f.lane & 31;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    f.lo = w & 1;
    f.hi = w >> 1;
    f.base = (size_t)bh * S * D;
    f.row_base = (size_t)bh * S;
    const int lo = f.lo, hi = f.hi, g = f.g, n = f.n, lane = f.lane;

    // Piece u (< PIECES) of this wave's share of rows r0 .. r0+63 of t into
    // the swizzled tile dst, straight from global memory into LDS; lane L of
    // a 1 KB piece lands at byte 16 L of it, so it loads the logical chunk
    // the swizzle puts there; rows past S read as zero.  M0 = the LDS
    // address; the only waits on these loads are the explicit ones.
    auto dma_tile = [&](_Float16* dst, const _Float16* t, int r0) {
        const auto r = f.rsrc(t, r0);
#pragma unroll
        for (int u = 0; u < PIECES; ++u) {
            const int piece = w * PIECES + u;
            const int row = RPP * piece + lane / G::CPR;
            const int logical = (lane % G::CPR) ^ swz_b<D>(row);
            const uint32_t m0 = (uint32_t)(uintptr_t)(LdsPtr)(dst + piece * 512);
            asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
                         :
                         : "v"((row * D + 8 * logical) * 2), "s"(r), "{m0}"(m0)
                         : "memory");
        }
    };
    // One row fragment: row r0 + n, head dims 16kk + 8g .. +7.
    auto row1 = [&](const _Float16* tile, int r0, int kk) {
        const int row = r0 + n;
        return *reinterpret_cast<const half8*>(tile + row * D + 8 * ((2 * kk + g) ^ swz_b<D>(row)));
    };
    // One transposed fragment (head dims 32b + n of rows r0 + 16h +
    // {4g .. 4g+3, 8+4g .. 8+4g+3}), as Bwd::cols.
    auto col1 = [&](const _Float16* tile, int r0, int h, int b) {
        const int n16 = n >> 4, jj = n & 15;
        const int sub = (jj & 3) >> 1, half = jj & 1;
        half4 part[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int row = r0 + 4 * g + (jj >> 2) + 16 * h + 8 * t;
            const int chunk = (4 * b + 2 * n16 + sub) ^ swz_b<D>(row);
            part[t] = __builtin_bit_cast(half4, __builtin_amdgcn_ds_read_tr16_b64_v4f16(
                                                    (lds_half4*)(tile + row * D + 8 * chunk + 4 * half)));
        }
        return half8{part[0][0], part[0][1], part[0][2], part[0][3],
                     part[1][0], part[1][1], part[1][2], part[1][3]};
    };
    auto barrier_dma = [&]() {
        asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
    };

    floatx16 dk[NB], dv[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            dk[b][r] = 0.f;
            dv[b][r] = 0.f;
        }

    // this workgroup's K and V tiles, resident for the whole walk
    dma_tile(Ks, K, k0);
    dma_tile(Vs, V, k0);
    const int qt0 = CAUSAL ? kt : 0;
    const int key = k0 + 32 * lo + n;
    for (int qt = qt0; qt < T; ++qt) {
        // every wave is done with the previous Q and dO tiles
        barrier_dma();
        dma_tile(Qs, Q, qt * 64);
        dma_tile(Os, dO, qt * 64);
        if (f.tid < 64) {
            // rows past S: any finite value (their products are masked)
            const int row = min(qt * 64 + f.tid, S - 1);
            const float lv = LSE[f.row_base + row];
            const float dv_ = dlt[f.row_base + row];
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            fl[f.tid] = lv * kLog2e;
            fl[64 + f.tid] = dv_;
        }
        barrier_dma();
        const int q0 = qt * 64 + 32 * hi;  // first query row of this wave

        // S and dP: register r of a score block holds query
        // q0 + 8(r/4) + 4g + r%4 for key k0 + 32lo + n
        floatx16 sacc, dp;
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[r] = dp[r] = 0.f;
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) {
            sacc = __builtin_amdgcn_mfma_f32_32x32x16_f16(row1(Qs, 32 * hi, kk), row1(Ks, 32 * lo, kk),
                                                          sacc, 0, 0, 0);
            dp = __builtin_amdgcn_mfma_f32_32x32x16_f16(row1(Os, 32 * hi, kk), row1(Vs, 32 * lo, kk),
                                                        dp, 0, 0, 0);
        }
        half8 pa[2], sa[2];
        // only the diagonal tile and tiles that reach past S need the mask
        const bool edge = (CAUSAL && qt == kt) || qt * 64 + 64 > S || k0 + 64 > S;
#pragma unroll
        for (int j4 = 0; j4 < 4; ++j4) {
            const float4 l4 = *reinterpret_cast<const float4*>(fl + 32 * hi + 8 * j4 + 4 * g);
            const float4 d4 = *reinterpret_cast<const float4*>(fl + 64 + 32 * hi + 8 * j4 + 4 * g);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 4 * j4 + e;
                const float lse_r = e == 0 ? l4.x : e == 1 ? l4.y : e == 2 ? l4.z : l4.w;
                const float dlt_r = e == 0 ? d4.x : e == 1 ? d4.y : e == 2 ? d4.z : d4.w;
                float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[r], cs, -lse_r));
                if (edge) {
                    const int qrow = q0 + 8 * j4 + 4 * g + e;
                    const bool vis = qrow < S && key < S && (!CAUSAL || key <= qrow);
                    p = vis ? p : 0.f;
                }
                pa[r >> 3][r & 7] = (_Float16)p;
                sa[r >> 3][r & 7] = (_Float16)(p * (dp[r] - dlt_r));
            }
        }
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                dv[b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(col1(Os, 32 * hi, h, b), pa[h], dv[b], 0, 0, 0);
                dk[b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(col1(Qs, 32 * hi, h, b), sa[h], dk[b], 0, 0, 0);
            }
    }

    // The two query halves (hi = 0, 1) hold partial sums over disjoint rows.
    // Wave (lo, 0) finishes dK of keys 32lo .. +31 and wave (lo, 1) their dV,
    // each adding the other's partial (a + b, the same in either order), and
    // stores its rows from registers.  Register r of block b: head dim
    // 32b + 8(r/4) + 4g + r%4 of key k0 + 32lo + n.
    barrier_dma();
    {
        float4* mine = reinterpret_cast<float4*>(lds) + (2 * lo + hi) * (NB * 4) * 64;
        if (hi == 0) {
#pragma unroll
            for (int b = 0; b < NB; ++b) f.give(mine, dv[b], b);
        } else {
#pragma unroll
            for (int b = 0; b < NB; ++b) f.give(mine, dk[b], b);
        }
    }
    barrier_dma();
    {
        const float4* other = reinterpret_cast<const float4*>(lds) + (2 * lo + (hi ^ 1)) * (NB * 4) * 64;
        if (hi == 0) {
#pragma unroll
            for (int b = 0; b < NB; ++b) f.take(dk[b], other, b);
        } else {
#pragma unroll
            for (int b = 0; b < NB; ++b) f.take(dv[b], other, b);
        }
    }
    if (hi == 0) {
#pragma unroll
        for (int b = 0; b < NB; ++b) f.store_block(dK, dk[b], key, b, scale);
    } else {
#pragma unroll
        for (int b = 0; b < NB; ++b) f.store_block(dV, dv[b], key, b, 1.f);
    }
}

template <int D, bool CAUSAL>
hipError_t launch_dkdv_t(const BwdArgs& a) {
    const int BH = a.B * a.H;
    const int T = (a.S + 63) / 64;
    const dim3 grid((unsigned)((long long)BH * T));
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, CAUSAL>), grid, dim3(256), 0, (hipStream_t)a.stream,
                       (const _Float16*)a.q, (const _Float16*)a.k, (const _Float16*)a.v,
                       (const _Float16*)a.dout, (const float*)a.workspace, a.lse,
                       (_Float16*)a.dk, (_Float16*)a.dv, BH, a.S, a.scale * kLog2e, a.scale);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_dkdv(const BwdArgs& a) {
    if (a.D == 64) return a.causal ? launch_dkdv_t<64, true>(a) : launch_dkdv_t<64, false>(a);
    return a.causal ? launch_dkdv_t<128, true>(a) : launch_dkdv_t<128, false>(a);
}

hipError_t launch_bwd(const BwdArgs& a) {
    const hipError_t e = launch_bwd_dq(a);
    if (e != hipSuccess) return e;
    return launch_bwd_dkdv(a);  // reads the Dlt rows bwd_dq wrote (same stream, so after it)
}

}  // namespace attn
