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
__global__ void __launch_bounds__(256, 2)
bwd_dq_kernel(const _Float16* __restrict__ Q, const _Float16* __restrict__ K,
              const _Float16* __restrict__ V, const _Float16* __restrict__ dO,
              const _Float16* __restrict__ O, const float* __restrict__ LSE,
              float* __restrict__ dlt, _Float16* __restrict__ dQ, int BH, int S, float c,
              float scale, uint32_t qsign)
{
    using G = GeoB<D>;
    constexpr int NB = G::NB;
    constexpr int STAGE = 2 * G::TILE;  // K tile, V tile
    constexpr int PIECES = G::TILE * 2 / 1024 / G::NW;  // 1 KB pieces of a tile per wave
    constexpr int RPP = 1024 / (2 * D);                 // rows per piece
    __shared__ __attribute__((aligned(1024))) _Float16 lds[2 * STAGE];
    using LdsPtr = __attribute__((address_space(3))) void*;

    const int T = (S + 63) / 64;
    const int bh = blockIdx.x % BH;
    // Causal: the first half of the grid takes the heavy query tiles
    // (T-1, T-2, ...), the second half the light ones (0, 1, ...).  With two
    // workgroups per CU, workgroup i and i + grid/2 share a CU when the grid
    // fills the chip once, and carry T+1 key tiles between them.
    const int j = blockIdx.x / BH;
    const int qt = CAUSAL ? (j < T / 2 ? T - 1 - j : j - T / 2) : j;

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

    // Piece u (< PIECES) of this wave's share of rows r0 .. r0+63 of t into
    // the swizzled tile dst, straight from global memory into LDS (no staging
    // registers).  Lane L of a 1 KB piece lands at byte 16 L of it (row
    // RPP piece + L / CPR, physical chunk L % CPR), so it loads the logical
    // chunk the swizzle puts there; rows past S read as zero.  Inline
    // assembly with M0 = the LDS address, as the forward's tile loads, so the
    // only waits on these loads are the explicit ones before each barrier.
    auto dma_piece = [&](_Float16* dst, const _Float16* t, int r0, int u) {
        const int piece = w * PIECES + u;
        const int row = RPP * piece + lane / G::CPR;
        const int logical = (lane % G::CPR) ^ swz_b<D>(row);
        const auto r = f.rsrc(t, r0);
        const uint32_t m0 = (uint32_t)(uintptr_t)(LdsPtr)(dst + piece * 512);
        asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
                     :
                     : "v"((row * D + 8 * logical) * 2), "s"(r), "{m0}"(m0)
                     : "memory");
    };
    auto dma_tile = [&](int st, int kt) {
#pragma unroll
        for (int u = 0; u < PIECES; ++u) dma_piece(lds + st * STAGE, K, kt * 64, u);
#pragma unroll
        for (int u = 0; u < PIECES; ++u) dma_piece(lds + st * STAGE + G::TILE, V, kt * 64, u);
    };

    // All start-up loads are issued before the first wait: this lane's LSE,
    // the first key tile, then this wave's Q, dO and O rows.
    const int qrow = qt * 64 + 32 * lo + n;  // the query this lane owns
    // (the row is clamped rather than the load made conditional: a select
    // right after the load would wait for it)
    const float lse_raw = LSE[f.row_base + min(qrow, S - 1)];
    dma_tile(0, 0);
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
    int s = 0;
    for (int kt = 0; kt < nT; ++kt) {
        // key tile kt has landed (this wave's loads, then the barrier for
        // everyone's); every wave is done with tile kt-1, whose stage the
        // loads of kt+1 overwrite
        asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        if (kt + 1 < nT) dma_tile(s ^ 1, kt + 1);
        const _Float16* Ks = lds + s * STAGE;
        const _Float16* Vs = Ks + G::TILE;
        const int k0 = kt * 64 + 32 * hi;  // first key of this wave

        // Two workgroups per CU: the other one's waves hide the LDS latency,
        // so the row fragments are read one product at a time (registers).
        floatx16 sacc, dp;
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[r] = dp[r] = 0.f;
        {
            half8 af[D / 16];
            f.rows(af, Ks, 32 * hi);
#pragma unroll
            for (int kk = 0; kk < D / 16; ++kk)
                sacc = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[kk], qb[kk], sacc, 0, 0, 0);
            f.rows(af, Vs, 32 * hi);
#pragma unroll
            for (int kk = 0; kk < D / 16; ++kk)
                dp = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[kk], ob[kk], dp, 0, 0, 0);
        }
        half8 bf[2][NB];
        f.cols(bf, Ks, 32 * hi);

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
