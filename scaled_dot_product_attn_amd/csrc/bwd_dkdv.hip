// dK/dV half of the attention backward (layout, helpers and the derivation are
// in bwd_common.h), and launch_bwd, which enqueues both halves.
#include "bwd_common.h"

namespace attn {
namespace {

using namespace detail;

// dK and dV for one 64-key tile.  Wave (lo, hi): keys 32lo .. +31 of the tile,
// query rows 32hi .. +31 of every query tile that sees the keys.
//   S  = Q K^T  : A = Q rows (LDS), B = this wave's K rows (registers)
//   dP = dO V^T : A = dO rows (LDS), B = this wave's V rows (registers)
//   dV^T += dO^T P, dK^T += Q^T dS : A = dO / Q columns (transposed LDS
//                 reads), B = P / dS (score registers); the accumulators hold
//                 lane = key, registers = head dims, so that rows are stored
//                 from registers
template <int D, bool CAUSAL>
__global__ void __launch_bounds__(256, 1)
bwd_dkdv_kernel(const _Float16* __restrict__ Q, const _Float16* __restrict__ K,
                const _Float16* __restrict__ V, const _Float16* __restrict__ dO,
                const float* __restrict__ dlt, const float* __restrict__ LSE,
                _Float16* __restrict__ dK, _Float16* __restrict__ dV,
                int BH, int S, float c, float scale, uint32_t qsign)
{
    using G = GeoB<D>;
    constexpr int NB = G::NB;
    // two stages of (Q tile, dO tile, LSE log2(e) [64], dlt[64])
    constexpr int STAGE = 2 * G::TILE + 2 * 64 * 2;  // halfs
    __shared__ __attribute__((aligned(1024))) _Float16 lds[2 * STAGE];

    const int T = (S + 63) / 64;
    const int bh = blockIdx.x % BH;
    const int kt = blockIdx.x / BH;  // causal: kt = 0 sees the most query tiles, so runs first
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
    f.c = c;
    f.qsign = qsign;
    const int lo = f.lo, hi = f.hi, g = f.g, n = f.n, lane = f.lane;

    floatx16 dk[NB], dv[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            dk[b][r] = 0.f;
            dv[b][r] = 0.f;
        }

    const int qt0 = CAUSAL ? kt : 0;
    u32x4 xq[G::CH], xo[G::CH];
    float lv = 0.f, dv_ = 0.f;
    auto stage_of = [&](int s) { return lds + s * STAGE; };
    // The row values are loaded first and used only in put(): consumed
    // right after the tile loads, they made the wave wait for those too.
    auto fetch = [&](int qt) {
        if (f.tid < 64) {
            const int row = qt * 64 + f.tid;
            lv = row < S ? LSE[f.row_base + row] : 0.f;
            dv_ = row < S ? dlt[f.row_base + row] : 0.f;
        }
        f.load(xq, Q, qt * 64);
        f.load(xo, dO, qt * 64);
    };
    auto put = [&](int s) {
        _Float16* st = stage_of(s);
        f.store(st, xq);
        f.store(st + G::TILE, xo);
        if (f.tid < 64) {
            float* fl = reinterpret_cast<float*>(st + 2 * G::TILE);
            fl[f.tid] = lv * kLog2e;
            fl[64 + f.tid] = dv_;
        }
    };
    // All start-up loads are issued before the first wait: the first query
    // tile, then this wave's K and V rows (B operands with k = head dim, kept
    // for the whole walk).  A negative scale negates the logits through K.
    fetch(qt0);
    half8 kb[D / 16], vb[D / 16];
    f.grows(kb, K, k0 + 32 * lo, 0u);
    f.grows(vb, V, k0 + 32 * lo, 0u);
    put(0);
    f.flip(kb, qsign);
    int s = 0;
    for (int qt = qt0; qt < T; ++qt) {
        barrier();  // query tile qt is in stage s; every wave is done with qt-1
        const bool more = qt + 1 < T;
        if (more) fetch(qt + 1);
        const _Float16* Qs = stage_of(s);
        const _Float16* Os = Qs + G::TILE;
        const float* fl = reinterpret_cast<const float*>(Qs + 2 * G::TILE);
        const int q0 = qt * 64 + 32 * hi;  // first query row of this wave

        // Every LDS read of the products is issued before the first of them,
        // the row values first: with one wave per SIMD nothing else hides
        // their latency.  Register r of a score block holds query
        // q0 + 8(r/4) + 4g + r%4 for key k0 + 32lo + n.
        float4 l4[4], d4[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            l4[j] = *reinterpret_cast<const float4*>(fl + 32 * hi + 8 * j + 4 * g);
            d4[j] = *reinterpret_cast<const float4*>(fl + 64 + 32 * hi + 8 * j + 4 * g);
        }
        half8 aq[D / 16], ao[D / 16];
        f.rows(aq, Qs, 32 * hi);
        f.rows(ao, Os, 32 * hi);
        __builtin_amdgcn_sched_barrier(0);
        floatx16 sacc, dp;
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[r] = dp[r] = 0.f;
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) {
            sacc = __builtin_amdgcn_mfma_f32_32x32x16_f16(aq[kk], kb[kk], sacc, 0, 0, 0);
            dp = __builtin_amdgcn_mfma_f32_32x32x16_f16(ao[kk], vb[kk], dp, 0, 0, 0);
        }
        // the dO columns of dV += P^T dO go out while the scores are formed,
        // the Q columns of dK += dS^T Q before the dV products
        half8 bo[2][NB], bq[2][NB];
        f.cols(bo, Os, 32 * hi);
        __builtin_amdgcn_sched_barrier(0);
        const int key = k0 + 32 * lo + n;
        half8 pa[2], sa[2];
        // only the diagonal tile and tiles that reach past S need the mask
        const bool edge = (CAUSAL && qt == kt) || qt * 64 + 64 > S || k0 + 64 > S;
        if (edge) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int qrow = q0 + 8 * (r >> 2) + 4 * g + (r & 3);
                const float lse_r = l4[r >> 2][r & 3], dlt_r = d4[r >> 2][r & 3];
                const bool vis = qrow < S && key < S && (!CAUSAL || key <= qrow);
                const float p = vis ? __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[r], c, -lse_r)) : 0.f;
                pa[r >> 3][r & 7] = (_Float16)p;
                sa[r >> 3][r & 7] = (_Float16)(p * (dp[r] - dlt_r));
            }
        } else {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float lse_r = l4[r >> 2][r & 3], dlt_r = d4[r >> 2][r & 3];
                const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[r], c, -lse_r));
                pa[r >> 3][r & 7] = (_Float16)p;
                sa[r >> 3][r & 7] = (_Float16)(p * (dp[r] - dlt_r));
            }
        }
        f.cols(bq, Qs, 32 * hi);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int b = 0; b < NB; ++b)
                dv[b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(bo[h][b], pa[h], dv[b], 0, 0, 0);
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int b = 0; b < NB; ++b)
                dk[b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(bq[h][b], sa[h], dk[b], 0, 0, 0);
        if (more) put(s ^ 1);
        s ^= 1;
    }

    // The two query halves (hi = 0, 1) hold partial sums over disjoint rows.
    // Wave (lo, 0) finishes dK of keys 32lo .. +31 and wave (lo, 1) their dV,
    // each adding the other's partial (a + b, the same in either order), and
    // stores its rows from registers.  Register r of block b: head dim
    // 32b + 8(r/4) + 4g + r%4 of key k0 + 32lo + n.
    barrier();
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
    barrier();
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
    const int key = k0 + 32 * lo + n;
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
                       (_Float16*)a.dk, (_Float16*)a.dv, BH, a.S, bwd_c(a.scale), a.scale,
                       bwd_qsign(a.scale));
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
