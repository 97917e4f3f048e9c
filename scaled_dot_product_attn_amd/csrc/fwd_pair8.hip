// Fused scaled-dot-product attention forward for gfx950 (CDNA4), D in {64, 128}.
//
//   O = softmax(scale * Q K^T + causal mask) V,   LSE = log sum_j exp(scale q.k_j)
//
// fp16 Q/K/V/O, fp32 accumulation and fp32 LSE.  The score tile lives only in
// registers ("An Optimal Mapper Meets a Real GPU", section "Ground rules": one
// fused kernel with register-resident scores instead of a multi-kernel
// pipeline through global workspaces); the running output is rescaled when a
// later key tile raises the row maximum.
//
// Work decomposition
//   * One workgroup of 8 waves per CU, two waves per SIMD: a wave's step is a
//     dependent chain (LDS -> Q K^T on the matrix cores -> softmax on the
//     vector ALUs -> P V), so a SIMD needs a second wave to keep the matrix
//     core fed while the first runs its softmax, and one wave alone cannot
//     issue matrix instructions at the core's full rate.
//   * The workgroup owns two 64-row query tiles a and b of one (batch, head)
//     and streams 64-key tiles of K and V through LDS.  Causal: a = p and
//     b = T-1-p, so every workgroup covers T+1 tile-rows of work and the
//     causal triangle is balanced across the chip; with T odd the middle tile
//     forms a workgroup on its own (a absent).  Non-causal: a = 2p, b = 2p+1.
//   * Wave w: rg = w&1 picks query rows 32rg .. +31, kh = (w>>1)&1 picks keys
//     32kh .. +31 of a key tile, hi = w>>2 picks the role.
//     Phase 1, key tiles 0 .. na-1 that both a and b see: the hi = 0 waves
//     work on a's rows, the hi = 1 waves on b's, all on the same staged tile,
//     so each tile in LDS serves 128 query rows.
//     Phase 2, key tiles na .. nb-1 that only b sees: two tiles are staged per
//     step; the hi = 1 waves continue their b state on the even ones, the
//     hi = 0 waves (after writing a) build b state on the odd ones.
//   * Every wave processes 32 rows x 32 keys per step, so all eight do the
//     same number of steps.  Partial states over disjoint key sets (two for a,
//     up to four for b) are merged in a fixed order (deterministic); merging
//     over DISJOINT key sets is exact, unlike merging head-dim partial
//     products after the softmax.
//   * Next-step tiles are fetched with bounds-checked buffer loads (rows past
//     S read as zero) into registers at the start of a step and written to the
//     other LDS stage at its end; tiles past the causal diagonal are never
//     loaded.
//   * S^T = K Q^T on v_mfma_f32_32x32x16_f16: A = 32 keys x 16 dims from LDS,
//     B = the wave's Q^T fragment held in registers.  Each lane owns one query
//     and 16 keys, so row statistics stay in the lane and the row max needs one
//     exchange between the two 32-lane halves.
//   * O^T += V^T P^T: P^T (fp16, round-to-nearest-even) is the B operand
//     straight from the softmax registers; V^T comes from the row-major V tile
//     via ds_read_b64_tr_b16, whose key order matches the accumulator's.
//   * exp2 on v_exp_f32 with scale*log2(e) folded into one FMA; lazy rescale
//     (the reference max moves only when a row max grows by more than 2^8).
//
// MFMA lane layouts (32x32x16, wave64, g = lane / 32, n = lane % 32):
//   A[m][k]: lane holds m = n, k = 8g .. 8g+7
//   B[k][n]: lane holds n = n, k = 8g .. 8g+7
//   C[m][n]: register r holds m = 8(r/4) + 4g + r%4, n = n
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fwd_common.h"
#include "kernels.h"

namespace attn {
namespace {

using namespace detail;

template <int D>
struct Geo8 {
    static constexpr int NW = 8;                 // waves per workgroup
    static constexpr int NT = 64 * NW;           // threads
    static constexpr int BM = 64;                // query rows per tile
    static constexpr int BN = 64;                // keys per tile
    static constexpr int CPR = D / 8;            // 16-byte chunks per row
    static constexpr int KSTR = D + 8;           // K row stride in halfs (16 B pad)
    static constexpr int KTILE = BN * KSTR;      // halfs in a K tile
    static constexpr int VTILE = BN * D;         // halfs in a V tile (swizzled, no pad)
    static constexpr int TILE = KTILE + VTILE;
    static constexpr int STAGE = 2 * TILE;       // a stage holds up to two tiles
    static constexpr int LDS_HALFS = 2 * STAGE;  // two stages
    static constexpr int CH = BN * CPR / NT;     // 16-byte chunks per thread per K (or V) tile
    static constexpr int PART = 32 * D;          // floats of one wave's partial output
    static_assert(D == 64 || D == 128, "D");
    static_assert(CH >= 1 && CH * NT == BN * CPR, "tile split");
    static_assert(LDS_HALFS * 2 <= 160 * 1024, "LDS budget");
    // final merge: the eight waves' partial outputs plus their (m, l); the
    // transition merge holds four of them inside one stage
    static_assert(8 * (PART + 128) * 4 <= LDS_HALFS * 2, "merge buffer fits");
    static_assert(4 * (PART + 128) * 4 <= STAGE * 2, "transition buffer fits a stage");
};

// V tile swizzle: 16-byte chunk index XOR, so that the 32 lanes of a
// transposed read hit distinct banks.
template <int D>
__device__ __forceinline__ int swz_v8(int r) {
    return D == 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1);
}

template <int D, bool CAUSAL>
struct Fwd8 {
    using G = Geo8<D>;
    static constexpr int NB = D / 32;  // output accumulator blocks

    const _Float16* __restrict__ Q;
    const _Float16* __restrict__ K;
    const _Float16* __restrict__ V;
    _Float16* __restrict__ O;
    float* __restrict__ LSE;
    _Float16* lds;
    int S;
    size_t base;      // element offset of this (batch, head)
    size_t lse_base;  // LSE offset of this (batch, head)
    float c;          // |scale| * log2(e)
    uint32_t qsign;   // 0x80008000 when the scale is negative (Q negated)
    int tid, lane, g, n, w, rg, kh, hi;

    u32x4 kreg[2][G::CH];  // staging registers for up to two tiles
    u32x4 vreg[2][G::CH];

    // Buffer resource of rows j0 .. S-1 of this (batch, head): loads past the
    // end return zero.
    __device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const _Float16* t, int j0) const {
        return __builtin_amdgcn_make_buffer_rsrc(
            const_cast<_Float16*>(t + base + (size_t)j0 * D), (short)0,
            (S - j0) * D * 2, 0x00020000);
    }
    template <int SL>
    __device__ __forceinline__ void load_tile(int j) {
        const int j0 = j * G::BN;
        const auto rk = rows_rsrc(K, j0), rv = rows_rsrc(V, j0);
#pragma unroll
        for (int u = 0; u < G::CH; ++u) {
            const int ci = tid + G::NT * u;  // byte offset of chunk ci is 16 * ci
            kreg[SL][u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rk, 16 * ci, 0, 0));
            vreg[SL][u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rv, 16 * ci, 0, 0));
        }
    }
    template <int SL>
    __device__ __forceinline__ void store_tile(int st) {
        _Float16* Ks = lds + st * G::STAGE + SL * G::TILE;
        _Float16* Vs = Ks + G::KTILE;
#pragma unroll
        for (int u = 0; u < G::CH; ++u) {
            const int ci = tid + G::NT * u;
            const int row = ci / G::CPR, cc = ci % G::CPR;
            *reinterpret_cast<u32x4*>(Ks + row * G::KSTR + 8 * cc) = kreg[SL][u];
            *reinterpret_cast<u32x4*>(Vs + row * D + 8 * (cc ^ swz_v8<D>(row))) = vreg[SL][u];
        }
    }
    // Fetch the next step's tiles (j, j+1; cnt of them) into registers, and
    // write them to stage st at the end of the step.
    __device__ __forceinline__ void load_next(int j, int cnt) {
        if (cnt > 0) load_tile<0>(j);
        if (cnt > 1) load_tile<1>(j + 1);
    }
    __device__ __forceinline__ void store_next(int st, int cnt) {
        if (cnt > 0) store_tile<0>(st);
        if (cnt > 1) store_tile<1>(st);
    }

    // K fragments of keys 32kh .. +31 of the tile at t (A operand of S^T = K Q^T).
    __device__ __forceinline__ void read_k(half8* kf, const _Float16* t) const {
        const _Float16* kp = t + (32 * kh + n) * G::KSTR + 8 * g;
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) kf[kk] = *reinterpret_cast<const half8*>(kp + 16 * kk);
    }
    __device__ __forceinline__ floatx16 qk(const half8* kf, const half8* qf) const {
        floatx16 acc;
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk)
            acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(kf[kk], qf[kk], acc, 0, 0, 0);
        return acc;
    }
    // V^T fragments (A operand of O^T += V^T P^T) of keys 32kh .. +31 via
    // transposed LDS reads: vf[h][b] covers keys 32kh + 16h .. +15 and head
    // dims 32b .. +31.  In each 16-lane group, lane 4r + c addresses row r,
    // columns 4c .. 4c+3 and receives column (lane % 16) of rows 0..3, so two
    // reads deliver the key order 8(r/4) + 4g + r%4 of the score accumulator.
    __device__ __forceinline__ void read_v(half8 (*vf)[NB], const _Float16* t) const {
        const _Float16* Vs = t + G::KTILE;
        const int n16 = n >> 4, jj = n & 15;
        const int sub = (jj & 3) >> 1, half = (jj & 1);
        const int sw = swz_v8<D>(jj >> 2);  // row & 3 == jj >> 2 for every read below
        const _Float16* rowp = Vs + (32 * kh + 4 * g + (jj >> 2)) * D + 4 * half;
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const _Float16* pb = rowp + 8 * ((4 * b + 2 * n16 + sub) ^ sw);
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                half4 part[2];
#pragma unroll
                for (int tt = 0; tt < 2; ++tt)
                    part[tt] = __builtin_bit_cast(
                        half4, __builtin_amdgcn_ds_read_tr16_b64_v4f16(
                                   (lds_half4*)(pb + (16 * h + 8 * tt) * D)));
                vf[h][b] = half8{part[0][0], part[0][1], part[0][2], part[0][3],
                                 part[1][0], part[1][1], part[1][2], part[1][3]};
            }
        }
    }
    __device__ __forceinline__ void pv(floatx16* o, const half8 (*vf)[NB], const half8* pf) const {
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int b = 0; b < NB; ++b)
                o[b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf[h][b], pf[h], o[b], 0, 0, 0);
    }

    // First half of this wave's 32 x 32 block of key tile j at t: S = Q K^T,
    // online softmax -> P (pf), and the V^T fragments for the second half.
    template <bool MASK>
    __device__ __forceinline__ void block_qk(const _Float16* t, int j, int row, const half8* qf,
                                             float& m, float& l, floatx16* o, half8* pf,
                                             half8 (*vf)[NB]) const {
        half8 kf[D / 16];
        read_k(kf, t);
        read_v(vf, t);
        const floatx16 s = qk(kf, qf);
        // visibility: key <= min(row, S-1) (causal) or key <= S-1
        const int lim = (CAUSAL ? min(row, S - 1) : S - 1) - (j * G::BN + 32 * kh + 4 * g);
        online_softmax<MASK, NB>(s, lim, c, m, l, o, pf);
    }

    // One step: next tiles -> registers; this wave's block (if any), with the
    // next tiles written to the other stage between its softmax and its P V
    // so that the LDS writes overlap the matrix work.
    template <bool MASK>
    __device__ __forceinline__ void step(int stg, int jnext, int cnext, bool active, int slot,
                                         int j, int row, const half8* qf, float& m, float& l,
                                         floatx16* o) {
        barrier();  // this step's tiles are in LDS; every wave is done with the last step
        load_next(jnext, cnext);
        half8 pf[2];
        half8 vf[2][NB];
        if (active) block_qk<MASK>(lds + stg * G::STAGE + slot * G::TILE, j, row, qf, m, l, o, pf, vf);
        // stage stg^1 held the previous step's tiles, which every wave has
        // finished with (barrier above)
        store_next(stg ^ 1, cnext);
        if (active) pv(o, vf, pf);
    }

    __device__ __forceinline__ void load_q(half8* qf, int row) const {
        // lane holds Q[row][16kk + 8g .. +7] (rows past S read row S-1)
        const u32x4* src = reinterpret_cast<const u32x4*>(Q + base + (size_t)min(row, S - 1) * D);
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) {
            u32x4 x = src[2 * kk + g];
            x ^= qsign;
            qf[kk] = __builtin_bit_cast(half8, x);
        }
    }

    // Partial-state exchange through LDS at float offset `at`: slot q holds a
    // wave's O^T as float4 [b][q4][lane], then m and l [lane].
    // Only the blocks that other members of a merge group of GS waves combine
    // (b % GS != gidx) are written.
    template <int GS>
    __device__ __forceinline__ void publish(float* at, int q, int gidx, const floatx16* o, float m,
                                            float l) const {
        float4* mo = reinterpret_cast<float4*>(at + q * (G::PART + 128));
#pragma unroll
        for (int b = 0; b < NB; ++b)
            if (b % GS != gidx)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4)
                mo[(4 * b + q4) * 64 + lane] =
                    float4{o[b][4 * q4], o[b][4 * q4 + 1], o[b][4 * q4 + 2], o[b][4 * q4 + 3]};
        float* mm = at + q * (G::PART + 128) + G::PART;
        mm[lane] = m;
        mm[64 + lane] = l;
    }
    // Store output block b of this wave's 32 rows (already divided by l):
    // lanes n and n+32 swap halves so that each lane writes 8 consecutive
    // head dims (16 bytes).
    __device__ __forceinline__ void store_block(const floatx16& ob, int b, int row) const {
        // x[q4] packs head dims 32b + 8q4 + 4g .. +3 as two fp16 pairs
        u32x2 x[4];
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            x[q4][0] = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)ob[4 * q4]) |
                       ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)ob[4 * q4 + 1]) << 16);
            x[q4][1] = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)ob[4 * q4 + 2]) |
                       ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)ob[4 * q4 + 3]) << 16);
        }
        _Float16* orow = O + base + (size_t)row * D;
#pragma unroll
        for (int qq = 0; qq < 2; ++qq) {
            // lane (g=0) keeps q4 = 2qq and receives the partner's 2qq; lane
            // (g=1) keeps q4 = 2qq+1 and receives the partner's 2qq+1
            const u32x2 send = g ? x[2 * qq] : x[2 * qq + 1];
            const u32x2 keep = g ? x[2 * qq + 1] : x[2 * qq];
            u32x2 got;
#pragma unroll
            for (int e = 0; e < 2; ++e) got[e] = (uint32_t)__shfl_xor((int)send[e], 32, 64);
            const u32x4 v = g ? u32x4{got[0], got[1], keep[0], keep[1]}
                              : u32x4{keep[0], keep[1], got[0], got[1]};
            if (row < S) *reinterpret_cast<u32x4*>(orow + 32 * b + 16 * qq + 8 * g) = v;
        }
    }

    // Merge this wave's state with the GS-1 other partial states of the same
    // rows published in slots other[] (online-softmax merge over disjoint key
    // sets, fixed order), then write the output blocks b with b % GS == gidx
    // and, for gidx == 0, the LSE.  Every member computes the same totals.
    template <int GS>
    __device__ __forceinline__ void merge_write(const float* at, const int* other, int gidx,
                                                floatx16* o, float m, float l, int row) const {
        float mi[GS - 1], li[GS - 1], ai[GS - 1];
        float mt = m;
#pragma unroll
        for (int i = 0; i < GS - 1; ++i) {
            const float* mm = at + other[i] * (G::PART + 128) + G::PART;
            mi[i] = mm[lane];
            li[i] = mm[64 + lane];
            mt = fmaxf(mt, mi[i]);
        }
        // mt is finite: this wave's own state has seen keys
        const float a0 = __builtin_amdgcn_exp2f(m - mt);
        float lsum = l * a0;
#pragma unroll
        for (int i = 0; i < GS - 1; ++i) {
            ai[i] = __builtin_amdgcn_exp2f(mi[i] - mt);
            lsum += li[i] * ai[i];
        }
        const float lt = sum_halves(lsum);
        const float f = 1.0f / lt;
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            if (b % GS != gidx) continue;
            floatx16 ob = o[b] * (a0 * f);
#pragma unroll
            for (int i = 0; i < GS - 1; ++i) {
                const float4* mo = reinterpret_cast<const float4*>(at + other[i] * (G::PART + 128));
                const float fi = ai[i] * f;
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                    const float4 p1 = mo[(4 * b + q4) * 64 + lane];
                    ob[4 * q4] += p1.x * fi;
                    ob[4 * q4 + 1] += p1.y * fi;
                    ob[4 * q4 + 2] += p1.z * fi;
                    ob[4 * q4 + 3] += p1.w * fi;
                }
            }
            store_block(ob, b, row);
        }
        if (gidx == 0 && g == 0 && row < S) LSE[lse_base + row] = (mt + __builtin_amdgcn_logf(lt)) * kLn2;
    }

    // ta, tb: query tiles (ta < 0: absent); na: key tiles both see; nb: key
    // tiles b sees (nb >= na).
    __device__ void run(int ta, int tb, int na, int nb) {
        const int row_a = ta * G::BM + 32 * rg + n;
        const int row_b = tb * G::BM + 32 * rg + n;
        const int n2 = nb - na;
        const int ns = (n2 + 1) / 2;  // phase-2 steps
        const int par = 1 - hi;       // phase-2 tile parity of this wave
        // the last key tile needs a mask: the diagonal (causal) or a ragged end
        const bool mask_end = CAUSAL || (S % G::BN) != 0;

        // prologue: the first step's tiles and this wave's Q rows
        const int c_first = na > 0 ? 1 : min(2, nb);
        load_next(0, c_first);
        half8 qf[D / 16], qfb[D / 16];
        int row = (na > 0 && hi == 0) ? row_a : row_b;
        load_q(qf, row);
        // the b rows that the hi = 0 waves take up after phase 1
        if (hi == 0 && na > 0 && n2 > 0) load_q(qfb, row_b);
        store_next(0, c_first);

        float m = kNegInf, l = 0.f;
        floatx16 o[NB];
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) o[b][r] = 0.f;

        int stg = 0;
        // phase 1: every wave on tile i; the last tile is a's diagonal
        // (causal) or the ragged end (non-causal)
        for (int i = 0; i + 1 < na; ++i) {
            step<false>(stg, i + 1, 1, true, 0, i, row, qf, m, l, o);
            stg ^= 1;
        }
        if (na > 0) {
            if (mask_end)
                step<true>(stg, na, min(2, n2), true, 0, na - 1, row, qf, m, l, o);
            else
                step<false>(stg, na, min(2, n2), true, 0, na - 1, row, qf, m, l, o);
            stg ^= 1;
        }
        if (na > 0 && n2 > 0) {
            // a is complete over its keys: merge the two key halves of its
            // rows inside the stage just consumed (its next writer waits at
            // the next step's barrier), write a, and turn the hi = 0 waves to
            // partial state for b's rows.
            barrier();
            float* at = reinterpret_cast<float*>(lds + (stg ^ 1) * G::STAGE);
            if (hi == 0) publish<2>(at, w, kh, o, m, l);
            barrier();
            if (hi == 0) {
                const int other[1] = {w ^ 2};
                merge_write<2>(at, other, kh, o, m, l, row_a);
                row = row_b;
#pragma unroll
                for (int kk = 0; kk < D / 16; ++kk) qf[kk] = qfb[kk];
                m = kNegInf;
                l = 0.f;
#pragma unroll
                for (int b = 0; b < NB; ++b)
#pragma unroll
                    for (int r = 0; r < 16; ++r) o[b][r] = 0.f;
            }
        }
        // phase 2: tiles of this wave's parity; the last step holds b's
        // diagonal (phase 2 only exists under causal masking)
        for (int s2 = 0; s2 + 1 < ns; ++s2) {
            const int j = na + 2 * s2 + par;
            const int jn = na + 2 * s2 + 2;
            step<false>(stg, jn, min(2, nb - jn), true, par, j, row, qf, m, l, o);
            stg ^= 1;
        }
        if (ns > 0) {
            const int j = na + 2 * (ns - 1) + par;
            step<true>(stg, 0, 0, j < nb, par, j, row, qf, m, l, o);
            stg ^= 1;
        }

        // Final merge, spread over the waves that share rows: with a phase 2
        // the four partial states of b's rows (waves rg, rg+2, rg+4, rg+6),
        // each of which writes one output block; without one (non-causal)
        // the two key halves of a's rows and of b's rows.
        barrier();  // every wave is done reading the stages
        float* at = reinterpret_cast<float*>(lds);
        if (n2 > 0)
            publish<4>(at, w, w >> 1, o, m, l);
        else
            publish<2>(at, w, kh, o, m, l);
        barrier();
        if (n2 > 0) {
            const int other[3] = {w ^ 2, w ^ 4, w ^ 6};
            merge_write<4>(at, other, w >> 1, o, m, l, row);
        } else {
            const int other[1] = {w ^ 2};
            merge_write<2>(at, other, kh, o, m, l, row);
        }
    }
};

template <int D, bool CAUSAL>
__global__ void __launch_bounds__(512, 1)
fwd_pair8_kernel(const _Float16* __restrict__ Q, const _Float16* __restrict__ K,
                 const _Float16* __restrict__ V, _Float16* __restrict__ O,
                 float* __restrict__ LSE, int BH, int S, float c, uint32_t qsign)
{
    using G = Geo8<D>;
    __shared__ __attribute__((aligned(1024))) _Float16 lds[G::LDS_HALFS];

    const int bh = blockIdx.x % BH;
    const int p = blockIdx.x / BH;
    const int T = (S + G::BM - 1) / G::BM;

    Fwd8<D, CAUSAL> f;
    f.Q = Q;
    f.K = K;
    f.V = V;
    f.O = O;
    f.LSE = LSE;
    f.lds = lds;
    f.S = S;
    f.base = (size_t)bh * S * D;
    f.lse_base = (size_t)bh * S;
    f.c = c;
    f.qsign = qsign;
    f.tid = threadIdx.x;
    f.lane = threadIdx.x & 63;
    f.g = f.lane >> 5;
    f.n = f.lane & 31;
    // wave index through readfirstlane: provably uniform, so branches on it
    // stay scalar instead of becoming exec-masked
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    f.w = w;
    f.rg = w & 1;
    f.kh = (w >> 1) & 1;
    f.hi = w >> 2;

    if (CAUSAL) {
        const int tb = T - 1 - p;
        if (p < tb)
            f.run(p, tb, p + 1, T - p);  // pair: both see 0..p, b also p+1 .. T-1-p
        else
            f.run(-1, tb, 0, tb + 1);    // the middle tile of an odd T
    } else {
        // b = 2p+1 may lie past the end (T odd): its rows are never stored
        f.run(2 * p, 2 * p + 1, T, T);
    }
}

template <int D, bool CAUSAL>
hipError_t launch_pair8(const FwdArgs& a) {
    using G = Geo8<D>;
    const int T = (a.S + G::BM - 1) / G::BM;
    const long long blocks = (long long)a.B * a.H * ((T + 1) / 2);
    const float c = fabsf(a.scale) * 1.44269504088896340736f;
    const uint32_t qsign = a.scale < 0.f ? 0x80008000u : 0u;
    hipLaunchKernelGGL((fwd_pair8_kernel<D, CAUSAL>), dim3((unsigned)blocks), dim3(G::NT), 0,
                       (hipStream_t)a.stream,
                       (const _Float16*)a.q, (const _Float16*)a.k, (const _Float16*)a.v,
                       (_Float16*)a.o, a.lse, a.B * a.H, a.S, c, qsign);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fused_pair8_d64_d128(const FwdArgs& a) {
    if (a.D == 64) return a.causal ? launch_pair8<64, true>(a) : launch_pair8<64, false>(a);
    return a.causal ? launch_pair8<128, true>(a) : launch_pair8<128, false>(a);
}

}  // namespace attn
