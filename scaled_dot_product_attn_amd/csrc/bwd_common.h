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
// launches (bwd_dq.hip, bwd_dkdv.hip; this header holds what they share),
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
#pragma once

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
    // Output block b of row `row` (this lane's row: the accumulators are
    // transposed, register r holding head dim 32b + 8(r/4) + 4g + r%4), times
    // mul and rounded to fp16, stored as two 16-byte chunks: lanes n and n+32
    // swap halves (v_permlane32_swap, no LDS round trip) so that each holds 8
    // consecutive dims.  Rows past S are not written.
    __device__ __forceinline__ void store_block(_Float16* t, const floatx16& acc, int row, int b,
                                                float mul) const {
        uint32_t x[4][2];
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
#pragma unroll
            for (int e = 0; e < 2; ++e)
                x[q4][e] = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)(acc[4 * q4 + 2 * e] * mul)) |
                           ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)(acc[4 * q4 + 2 * e + 1] * mul)) << 16);
#pragma unroll
        for (int qq = 0; qq < 2; ++qq) {
            // the upper half-wave's x[2qq] trades places with the lower
            // half-wave's x[2qq+1]: afterwards lane g holds dims
            // 16qq + 8g .. +7 of the block
            const auto s0 = __builtin_amdgcn_permlane32_swap(x[2 * qq][0], x[2 * qq + 1][0], false, false);
            const auto s1 = __builtin_amdgcn_permlane32_swap(x[2 * qq][1], x[2 * qq + 1][1], false, false);
            const u32x4 v = u32x4{s0[0], s1[0], s0[1], s1[1]};
            if (row < S)
                *reinterpret_cast<u32x4*>(t + base + (size_t)row * D + 32 * b + 16 * qq + 8 * g) = v;
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

// Logit factor |scale| log2(e); the sign of the scale is applied to Q or K as
// an fp16 sign flip (qsign), its magnitude in c and in the final dQ/dK scaling.
__host__ inline float bwd_c(float scale) { return fabsf(scale) * kLog2e; }
__host__ inline uint32_t bwd_qsign(float scale) { return scale < 0.f ? 0x80008000u : 0u; }

}  // namespace

// One workgroup per 64-row query tile (grid B*H*T); writes dQ and Dlt = dO.O
// per row into the workspace.
hipError_t launch_bwd_dq(const BwdArgs& a);
// One workgroup per 64-key tile; reads the Dlt rows, so it is enqueued after
// launch_bwd_dq on the same stream.
hipError_t launch_bwd_dkdv(const BwdArgs& a);

}  // namespace attn
