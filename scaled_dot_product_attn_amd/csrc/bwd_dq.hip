// dQ half of the attention backward (layout, helpers and the derivation are in
// bwd_common.h).  This file is built with the MFMA accumulators in ordinary
// VGPRs (-mllvm -amdgpu-mfma-vgpr-form): by default the compiler keeps the
// loop-carried dQ blocks in VGPRs but runs the products on AGPR copies, and
// moves all 64 registers there and back in every iteration.
#include "bwd_common.h"

namespace attn {
namespace {

using namespace detail;

// dQ for one 64-row query tile.  Wave (lo, hi): query rows 32lo .. +31 of the
// tile, keys 32hi .. +31 of every key tile the rows see.
//   S^T  = K Q^T  : A = K rows (LDS), B = this wave's Q rows (registers)
//   dP^T = V dO^T : A = V rows (LDS), B = this wave's dO rows (registers)
//   dQ^T += K^T dS^T : A = K columns (transposed LDS reads), B = dS (score
//                   registers: lane = query, registers = keys); the
//                   accumulator holds lane = query, registers = head dims, so
//                   that rows are stored from registers
template <int D, bool CAUSAL>
__global__ void __launch_bounds__(256, 1)
bwd_dq_kernel(const _Float16* __restrict__ Q, const _Float16* __restrict__ K,
              const _Float16* __restrict__ V, const _Float16* __restrict__ dO,
              const _Float16* __restrict__ O, const float* __restrict__ LSE,
              float* __restrict__ dlt, _Float16* __restrict__ dQ, int BH, int S, float c,
              float scale, uint32_t qsign)
{
    using G = GeoB<D>;
    constexpr int NB = G::NB;
    constexpr int STAGE = 2 * G::TILE;  // K tile, V tile
    __shared__ __attribute__((aligned(1024))) _Float16 lds[2 * STAGE];

    const int T = (S + 63) / 64;
    const int bh = blockIdx.x % BH;
    const int qt = CAUSAL ? T - 1 - blockIdx.x / BH : blockIdx.x / BH;  // heaviest first

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

    // All start-up loads are issued before the first wait: this lane's LSE,
    // the first key tile, then this wave's Q, dO and O rows.
    const int qrow = qt * 64 + 32 * lo + n;  // the query this lane owns
    // (the row is clamped rather than the load made conditional: a select
    // right after the load would wait for it)
    const float lse_raw = LSE[f.row_base + min(qrow, S - 1)];
    u32x4 xk[G::CH], xv[G::CH];
    f.load(xk, K, 0);
    f.load(xv, V, 0);
    half8 qb[D / 16], ob[D / 16];
    f.grows(qb, Q, qt * 64 + 32 * lo, 0u);
    f.grows(ob, dO, qt * 64 + 32 * lo, 0u);
    // Dlt = dO . O of this lane's query: each half of the wave holds half of
    // the head dims (8g .. 8g+7 of every 16)
    float dlt_q;
    {
        half8 of[D / 16];
        f.grows(of, O, qt * 64 + 32 * lo, 0u);
        float acc = 0.f;
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk)
#pragma unroll
            for (int e = 0; e < 8; ++e) acc = __builtin_fmaf((float)of[kk][e], (float)ob[kk][e], acc);
        dlt_q = sum_halves(acc);
        if (hi == 0 && g == 0 && qrow < S) dlt[f.row_base + qrow] = dlt_q;
    }

    floatx16 dq[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) dq[b][r] = 0.f;

    const int nT = CAUSAL ? qt + 1 : T;
    f.flip(qb, qsign);  // a negative scale negates the logits through Q
    const float lse_q = qrow < S ? lse_raw * kLog2e : 0.f;
    f.store(lds, xk);
    f.store(lds + G::TILE, xv);
    int s = 0;
    for (int kt = 0; kt < nT; ++kt) {
        barrier();
        const bool more = kt + 1 < nT;
        if (more) {
            f.load(xk, K, (kt + 1) * 64);
            f.load(xv, V, (kt + 1) * 64);
        }
        const _Float16* Ks = lds + s * STAGE;
        const _Float16* Vs = Ks + G::TILE;
        const int k0 = kt * 64 + 32 * hi;  // first key of this wave

        // Every LDS read of the products is issued ahead of its use: with
        // one wave per SIMD nothing else hides their latency.  The K columns
        // of dQ += dS K go out while the scores are formed.
        half8 ak[D / 16], av[D / 16];
        f.rows(ak, Ks, 32 * hi);
        f.rows(av, Vs, 32 * hi);
        __builtin_amdgcn_sched_barrier(0);
        floatx16 sacc, dp;
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[r] = dp[r] = 0.f;
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) {
            sacc = __builtin_amdgcn_mfma_f32_32x32x16_f16(ak[kk], qb[kk], sacc, 0, 0, 0);
            dp = __builtin_amdgcn_mfma_f32_32x32x16_f16(av[kk], ob[kk], dp, 0, 0, 0);
        }
        half8 bf[2][NB];
        f.cols(bf, Ks, 32 * hi);
        __builtin_amdgcn_sched_barrier(0);

        // register r holds key k0 + 8(r/4) + 4g + r%4 for this lane's query;
        // only the diagonal tile and tiles that reach past S need the mask
        half8 sa[2];
        const bool edge = (CAUSAL && kt == qt) || qt * 64 + 64 > S || kt * 64 + 64 > S;
        if (edge) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = k0 + 8 * (r >> 2) + 4 * g + (r & 3);
                const bool vis = qrow < S && key < S && (!CAUSAL || key <= qrow);
                const float p = vis ? __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[r], c, -lse_q)) : 0.f;
                sa[r >> 3][r & 7] = (_Float16)(p * (dp[r] - dlt_q));
            }
        } else {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[r], c, -lse_q));
                sa[r >> 3][r & 7] = (_Float16)(p * (dp[r] - dlt_q));
            }
        }
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int b = 0; b < NB; ++b)
                dq[b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(bf[h][b], sa[h], dq[b], 0, 0, 0);
        if (more) {
            f.store(lds + (s ^ 1) * STAGE, xk);
            f.store(lds + (s ^ 1) * STAGE + G::TILE, xv);
        }
        s ^= 1;
    }

    // The two key halves (hi = 0, 1) hold partial sums over disjoint keys.
    // Wave (lo, hi) finishes head-dim blocks hi*NB/2 .. of queries 32lo .. +31,
    // adding the other's partial (a + b, the same in either order), and stores
    // those blocks of its rows from registers.  Register r of block b: head dim
    // 32b + 8(r/4) + 4g + r%4 of query qt*64 + 32lo + n.
    constexpr int HB = NB / 2;
    barrier();
    float4* mine = reinterpret_cast<float4*>(lds) + (2 * lo + hi) * (HB * 4) * 64;
    const float4* other = reinterpret_cast<const float4*>(lds) + (2 * lo + (hi ^ 1)) * (HB * 4) * 64;
    if (hi == 0) {
#pragma unroll
        for (int b = 0; b < HB; ++b) f.give(mine, dq[HB + b], b);
        barrier();
#pragma unroll
        for (int b = 0; b < HB; ++b) f.take(dq[b], other, b);
#pragma unroll
        for (int b = 0; b < HB; ++b) f.store_block(dQ, dq[b], qrow, b, scale);
    } else {
#pragma unroll
        for (int b = 0; b < HB; ++b) f.give(mine, dq[b], b);
        barrier();
#pragma unroll
        for (int b = 0; b < HB; ++b) f.take(dq[HB + b], other, b);
#pragma unroll
        for (int b = 0; b < HB; ++b) f.store_block(dQ, dq[HB + b], qrow, HB + b, scale);
    }
}

template <int D, bool CAUSAL>
hipError_t launch_dq_t(const BwdArgs& a) {
    const int BH = a.B * a.H;
    const int T = (a.S + 63) / 64;
    const dim3 grid((unsigned)((long long)BH * T));
    hipLaunchKernelGGL((bwd_dq_kernel<D, CAUSAL>), grid, dim3(256), 0, (hipStream_t)a.stream,
                       (const _Float16*)a.q, (const _Float16*)a.k, (const _Float16*)a.v,
                       (const _Float16*)a.dout, (const _Float16*)a.o, a.lse, (float*)a.workspace,
                       (_Float16*)a.dq, BH, a.S, bwd_c(a.scale), a.scale, bwd_qsign(a.scale));
    return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_dq(const BwdArgs& a) {
    if (a.D == 64) return a.causal ? launch_dq_t<64, true>(a) : launch_dq_t<64, false>(a);
    return a.causal ? launch_dq_t<128, true>(a) : launch_dq_t<128, false>(a);
}

}  // namespace attn
