// Attention backward for gfx950, D in {64, 128}: the gradients of
// L = sum(dO * O) for O = softmax(scale Q K^T + causal mask) V, from the
// forward's saved LSE (the probabilities are recomputed, never stored).
//
//   P[i,j]  = exp(scale q_i.k_j - LSE_i)            (0 where masked)
//   Dlt[i]  = dO_i . O_i
//   dP[i,j] = dO_i . v_j,   dS = P (dP - Dlt)
//   dV = P^T dO,   dK = scale dS^T Q,   dQ = scale dS K
//
// "Validating Memory-Optimal Transformer Kernels on Real Hardware" (abstract
// and section 4, "Paper II: Backward Pass and Fused Forward+Backward") measures
// an attention backward that never materialises the O(n^2) probabilities and
// traces its GPU cost to atomic updates of the key gradients (4.4 - 4.7).
// Here there are no atomics at all, so the result is deterministic: two
// launches,
//   bwd_dq    : one workgroup per 64-row query tile; it forms Dlt for its rows
//               (kept in the workspace for the next launch), walks the key
//               tiles the rows see and accumulates dQ;
//   bwd_dkdv  : one workgroup per 64-key tile; it walks the query tiles that
//               see it and accumulates dK and dV in registers.
// Each output row is written by exactly one workgroup.
//
// Inside both: 4 waves, wave w = (lo = w & 1, hi = w >> 1).  All products run
// on v_mfma_f32_32x32x16_f16 with fp32 accumulation; P and dS enter the MFMAs
// as fp16 (round to nearest even), dQ/dK/dV are written as fp16.
//   A[m][k]: lane holds m = n, k = 8g .. 8g+7
//   B[k][n]: lane holds n = n, k = 8g .. 8g+7
//   C[m][n]: register r holds m = 8(r/4) + 4g + r%4, n = n
// (g = lane / 32, n = lane % 32).  A score accumulator's registers 8h .. 8h+7
// are directly the next product's operand over the rows they index, with the
// k order 16h + {4g .. 4g+3, 8+4g .. 8+4g+3}; the matching operand is read
// from a row-major tile with ds_read_b64_tr_b16, as in the forward's P V.
//
// LDS tiles are read both ways (rows as an MFMA operand, and transposed), so
// their 16-byte chunks are XOR-swizzled with a pattern that keeps both the
// 16-row ds_read_b128 and the 4-row ds_read_b64_tr_b16 conflict-free.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fwd_common.h"
#include "kernels.h"

namespace attn {
namespace {

using namespace detail;

constexpr float kLog2e = 1.44269504088896340736f;

template <int D>
struct GeoB {
    static constexpr int NW = 4, NT = 256, BT = 64;  // rows (or keys) per tile
    static constexpr int CPR = D / 8;                // 16-byte chunks per row
    static constexpr int TILE = BT * D;              // halfs of one swizzled tile
    static constexpr int CH = BT * CPR / NT;         // chunks per thread per tile
    static constexpr int NB = D / 32;
    static_assert(D == 64 || D == 128, "D");
    static_assert(CH * NT == BT * CPR, "tile split");
};

// XOR applied to the 16-byte chunk index of row r.  D = 128 (16 chunks, 256 B
// per row): 4 (r & 3) | ((r >> 2) & 3) is a bijection on r mod 16, so 16
// consecutive rows at one logical chunk hit 16 distinct chunk slots, and 4
// consecutive rows (r0 = 0 mod 4) x 4 chunks 4b .. 4b+3 also map to 16
// distinct slots.  D = 64 (8 chunks, 128 B per row, two rows per bank period):
// 4 ((r >> 1) & 1) | ((r >> 2) & 3) does the same for rows of equal parity.
template <int D>
__device__ __forceinline__ int swz_b(int r) {
    return D == 128 ? (4 * (r & 3)) | ((r >> 2) & 3) : (4 * ((r >> 1) & 1)) | ((r >> 2) & 3);
}

template <int D>
struct Bwd {
    using G = GeoB<D>;
    static constexpr int NB = G::NB;

    int S, tid, lane, g, n, lo, hi;
    size_t base, row_base;  // element offset of this (batch, head); its first LSE row
    float c;                // |scale| log2(e)
    uint32_t qsign;         // 0x80008000 when the scale is negative

    // Buffer over rows r0 .. r0+63 of t, clipped at S: reads past it return zero.
    // The size goes through readfirstlane: computed as a clamp it otherwise
    // lands in a vector register, the descriptor counts as divergent and the
    // compiler wraps every load in a loop over its distinct values.
    __device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const _Float16* t, int r0) const {
        const int bytes = __builtin_amdgcn_readfirstlane(min(max(S - r0, 0), 64) * D * 2);
        return __builtin_amdgcn_make_buffer_rsrc(const_cast<_Float16*>(t + base + (size_t)r0 * D),
                                                 (short)0, bytes, 0x00020000);
    }
    // Rows r0 .. r0+63 of t (past S read as zero) -> registers x[CH].
    __device__ __forceinline__ void load(u32x4* x, const _Float16* t, int r0) const {
        const auto r = rsrc(t, r0);
#pragma unroll
        for (int u = 0; u < G::CH; ++u)
            x[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                 r, 16 * (tid + G::NT * u), 0, 0));
    }
    __device__ __forceinline__ void store(_Float16* tile, const u32x4* x) const {
#pragma unroll
        for (int u = 0; u < G::CH; ++u) {
            const int ci = tid + G::NT * u;
            const int row = ci / G::CPR, cc = ci % G::CPR;
            *reinterpret_cast<u32x4*>(tile + row * D + 8 * (cc ^ swz_b<D>(row))) = x[u];
        }
    }
    // Row fragments of rows r0 .. r0+31 (A or B operand with the head dim as k):
    // f[kk] = row (r0 + n), dims 16kk + 8g .. +7.
    __device__ __forceinline__ void rows(half8* f, const _Float16* tile, int r0) const {
        const int row = r0 + n;
        const _Float16* p = tile + row * D;
        const int sw = swz_b<D>(row);
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk)
            f[kk] = *reinterpret_cast<const half8*>(p + 8 * ((2 * kk + g) ^ sw));
    }
    // Transposed fragments of rows r0 .. r0+31 (the operand whose k runs over
    // those rows): f[h][b] holds head dims 32b + (lane % 32) for rows
    // r0 + 16h + {4g .. 4g+3, 8+4g .. 8+4g+3}.  In each 16-lane group lane
    // 4r + c addresses row r, columns 4c .. 4c+3 and receives column
    // lane % 16 of rows 0..3.
    __device__ __forceinline__ void cols(half8 (*f)[NB], const _Float16* tile, int r0) const {
        const int n16 = n >> 4, jj = n & 15;
        const int sub = (jj & 3) >> 1, half = jj & 1;
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                half4 part[2];
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    const int row = r0 + 4 * g + (jj >> 2) + 16 * h + 8 * t;
                    const int chunk = (4 * b + 2 * n16 + sub) ^ swz_b<D>(row);
                    part[t] = __builtin_bit_cast(
                        half4, __builtin_amdgcn_ds_read_tr16_b64_v4f16(
                                   (lds_half4*)(tile + row * D + 8 * chunk + 4 * half)));
                }
                f[h][b] = half8{part[0][0], part[0][1], part[0][2], part[0][3],
                                part[1][0], part[1][1], part[1][2], part[1][3]};
            }
    }
    // Output tile in LDS: 64 rows of D halfs, padded by 16 bytes per row.
    static constexpr int OP = D + 8;
    // Accumulator block acc (register r: row r0 + 8(r/4) + 4g + r%4, column
    // 32b + n) rounded to fp16 into the output tile.
    __device__ __forceinline__ void to_tile(_Float16* ot, const floatx16& acc, int r0, int b,
                                            float mul) const {
#pragma unroll
        for (int r = 0; r < 16; ++r)
            ot[(r0 + 8 * (r >> 2) + 4 * g + (r & 3)) * OP + 32 * b + n] = (_Float16)(acc[r] * mul);
    }
    // Rows r0 .. r0+63 of the output tile -> t (rows past S are not written):
    // every lane stores whole 16-byte chunks of a row.
    __device__ __forceinline__ void from_tile(_Float16* t, const _Float16* ot, int r0) const {
#pragma unroll
        for (int u = 0; u < G::CH; ++u) {
            const int ci = tid + G::NT * u;
            const int row = ci / G::CPR, cc = ci % G::CPR;
            if (r0 + row < S)
                *reinterpret_cast<u32x4*>(t + base + (size_t)(r0 + row) * D + 8 * cc) =
                    *reinterpret_cast<const u32x4*>(ot + row * OP + 8 * cc);
        }
    }
    // Partial accumulator blocks through LDS, one float4 per lane and slot.
    __device__ __forceinline__ void give(float4* buf, const floatx16& acc, int slot) const {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
            buf[(4 * slot + q4) * 64 + lane] =
                float4{acc[4 * q4], acc[4 * q4 + 1], acc[4 * q4 + 2], acc[4 * q4 + 3]};
    }
    __device__ __forceinline__ void take(floatx16& acc, const float4* buf, int slot) const {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            const float4 x = buf[(4 * slot + q4) * 64 + lane];
            acc[4 * q4] += x.x;
            acc[4 * q4 + 1] += x.y;
            acc[4 * q4 + 2] += x.z;
            acc[4 * q4 + 3] += x.w;
        }
    }
    __device__ __forceinline__ void flip(half8* f, uint32_t xsign) const {
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk)
            f[kk] = __builtin_bit_cast(half8, __builtin_bit_cast(u32x4, f[kk]) ^ xsign);
    }
    // Fragment of rows (r0 + n) straight from global memory (rows past S read
    // as zero); xsign flips fp16 signs.
    __device__ __forceinline__ void grows(half8* f, const _Float16* t, int r0, uint32_t xsign) const {
        const auto r = rsrc(t, r0);
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) {
            u32x4 x = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                    r, (n * D + 16 * kk + 8 * g) * 2, 0, 0));
            x ^= xsign;
            f[kk] = __builtin_bit_cast(half8, x);
        }
    }
};

// dK and dV for one 64-key tile.  Wave (lo, hi): keys 32lo .. +31 of the tile,
// query rows 32hi .. +31 of every query tile that sees the keys.
//   S  = Q K^T  : A = Q rows (LDS), B = this wave's K rows (registers)
//   dP = dO V^T : A = dO rows (LDS), B = this wave's V rows (registers)
//   dV += P^T dO, dK += dS^T Q : A = P^T / dS^T (score registers), B = dO / Q
//                 columns (transposed LDS reads)
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
                dv[b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(pa[h], bo[h][b], dv[b], 0, 0, 0);
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int b = 0; b < NB; ++b)
                dk[b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(sa[h], bq[h][b], dk[b], 0, 0, 0);
        if (more) put(s ^ 1);
        s ^= 1;
    }

    // The two query halves (hi = 0, 1) hold partial sums over disjoint rows.
    // Wave (lo, 0) finishes dK of keys 32lo .. +31 and wave (lo, 1) their dV,
    // each adding the other's partial (a + b, the same in either order); the
    // fp16 results go through LDS so that every global store is a 16-byte
    // chunk of a row.  Register r of block b: key k0 + 32lo + 8(r/4) + 4g + r%4,
    // head dim 32b + n.
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
    barrier();
    _Float16* ot = lds + hi * (64 * Bwd<D>::OP);  // hi = 0: dK tile, 1: dV tile
    if (hi == 0) {
#pragma unroll
        for (int b = 0; b < NB; ++b) f.to_tile(ot, dk[b], 32 * lo, b, scale);
    } else {
#pragma unroll
        for (int b = 0; b < NB; ++b) f.to_tile(ot, dv[b], 32 * lo, b, 1.f);
    }
    barrier();
    f.from_tile(dK, lds, k0);
    f.from_tile(dV, lds + 64 * Bwd<D>::OP, k0);
}

// dQ for one 64-row query tile.  Wave (lo, hi): query rows 32lo .. +31 of the
// tile, keys 32hi .. +31 of every key tile the rows see.
//   S^T  = K Q^T  : A = K rows (LDS), B = this wave's Q rows (registers)
//   dP^T = V dO^T : A = V rows (LDS), B = this wave's dO rows (registers)
//   dQ  += dS K   : A = dS (score registers: lane = query, registers = keys),
//                   B = K columns (transposed LDS reads)
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
                dq[b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(sa[h], bf[h][b], dq[b], 0, 0, 0);
        if (more) {
            f.store(lds + (s ^ 1) * STAGE, xk);
            f.store(lds + (s ^ 1) * STAGE + G::TILE, xv);
        }
        s ^= 1;
    }

    // The two key halves (hi = 0, 1) hold partial sums over disjoint keys.
    // Wave (lo, hi) finishes head-dim blocks hi*NB/2 .. of queries 32lo .. +31,
    // adding the other's partial (a + b, the same in either order); the fp16
    // results go through LDS so that every global store is a 16-byte chunk of
    // a row.  Register r of block b: query qt*64 + 32lo + 8(r/4) + 4g + r%4,
    // head dim 32b + n.
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
        barrier();
#pragma unroll
        for (int b = 0; b < HB; ++b) f.to_tile(lds, dq[b], 32 * lo, b, scale);
    } else {
#pragma unroll
        for (int b = 0; b < HB; ++b) f.give(mine, dq[b], b);
        barrier();
#pragma unroll
        for (int b = 0; b < HB; ++b) f.take(dq[HB + b], other, b);
        barrier();
#pragma unroll
        for (int b = 0; b < HB; ++b) f.to_tile(lds, dq[HB + b], 32 * lo, HB + b, scale);
    }
    barrier();
    f.from_tile(dQ, lds, qt * 64);
}

template <int D, bool CAUSAL>
hipError_t launch_bwd_t(const BwdArgs& a) {
    const int BH = a.B * a.H;
    const int T = (a.S + 63) / 64;
    float* dlt = (float*)a.workspace;
    // the sign of the scale is applied to Q/K (fp16 sign flip), its magnitude
    // in c for the logits and in the final dQ/dK scaling
    const float c = fabsf(a.scale) * kLog2e;
    const uint32_t qsign = a.scale < 0.f ? 0x80008000u : 0u;
    const dim3 grid((unsigned)((long long)BH * T));
    hipLaunchKernelGGL((bwd_dq_kernel<D, CAUSAL>), grid, dim3(256), 0, (hipStream_t)a.stream,
                       (const _Float16*)a.q, (const _Float16*)a.k, (const _Float16*)a.v,
                       (const _Float16*)a.dout, (const _Float16*)a.o, a.lse, dlt,
                       (_Float16*)a.dq, BH, a.S, c, a.scale, qsign);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // reads the Dlt rows that bwd_dq wrote (same stream, so after it)
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, CAUSAL>), grid, dim3(256), 0, (hipStream_t)a.stream,
                       (const _Float16*)a.q, (const _Float16*)a.k, (const _Float16*)a.v,
                       (const _Float16*)a.dout, dlt, a.lse, (_Float16*)a.dk, (_Float16*)a.dv,
                       BH, a.S, c, a.scale, qsign);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd(const BwdArgs& a) {
    if (a.D == 64) return a.causal ? launch_bwd_t<64, true>(a) : launch_bwd_t<64, false>(a);
    return a.causal ? launch_bwd_t<128, true>(a) : launch_bwd_t<128, false>(a);
}

}  // namespace attn
