// Fused attention forward for gfx950, D = 128, for shapes with many query
// tiles: one workgroup of four waves per 128-row query tile, two workgroups
// per CU, every wave owning 32 complete query rows.
//
//   O = softmax(scale * Q K^T + causal mask) V,   LSE = log sum_j exp(scale q.k_j)
//
// The score tile lives only in registers ("An Optimal Mapper Meets a Real
// GPU", section "Ground rules": one fused kernel instead of a pipeline of
// kernels through global workspaces).
//
// Work split.  Wave w takes query rows 32r .. 32r+31 of the tile (r = w, or
// 3 - w in the workgroups with odd u, below) and walks
// the keys in 32-key chunks; the four waves share every staged chunk, so a
// K/V byte brought into LDS feeds 128 query rows (half the global->LDS bytes
// per FLOP of a 64-row tile), and since no wave splits the keys of its rows
// with another there is no merge at the end: each wave normalises and stores
// its own rows from registers.
//
// Software pipeline, per chunk j of a wave (the D = 64/128 kernel's, with a
// 32-key chunk in place of a wave's half of a 64-key tile):
//     S(j+1) = K(j+1) Q^T        matrix cores   \  issued together, no
//     P(j)   = softmax(S(j))     vector ALUs    /  dependence between them
//     wait for this wave's loads, barrier
//     O     += V(j)^T P(j)       matrix cores, each instruction followed by a
//                                share of the loads of K(j+3) and V(j+2), one
//                                K(j+2) fragment read and one V(j+1) fragment
// K and V chunks go from global memory straight into LDS (buffer loads with
// the LDS destination bit, no staging registers) through two K and two V
// slots; the Q tile comes in the same way and stays in registers.
//
// Causal balance.  When the pairs alone still give two workgroups per CU, a
// workgroup runs two query tiles of one (batch, head), T-1-u and then u, so
// every workgroup carries T+1 tile-lengths of keys; the second tile's prologue
// loads go out right after the first tile's last barrier, ahead of its
// epilogue, and its K/V chunks are a prefix of those the first tile just read
// (same XCD L2).  Otherwise one tile per workgroup, heaviest tiles first.
//
// Causal masking.  Wave w's rows see every key of the chunks before its
// diagonal chunk cw = (q0 + 32w) / 32, part of chunk cw, and none after it.
// So the pipelined iterations never mask; chunk cw is the wave's last,
// masked, step; after it the wave only keeps issuing its share of the loads
// and meeting the barriers until the tile's other waves are done.
//
// MFMA lane layouts (v_mfma_f32_32x32x16_f16, wave64, g = lane / 32,
// n = lane % 32):
//   A[m][k]: lane holds m = n, k = 8g .. 8g+7
//   B[k][n]: lane holds n = n, k = 8g .. 8g+7
//   C[m][n]: register r holds m = 8(r/4) + 4g + r%4, n = n
// S^T = K Q^T puts one query per lane (n) and the chunk's 32 keys in 16
// registers of the two half-waves; O^T += V^T P^T takes P^T straight from
// those registers as the B operand and V^T from transposed LDS reads.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fwd_common.h"
#include "kernels.h"

namespace attn {
namespace {

using namespace detail;

struct GeoR {
    static constexpr int D = 128;
    static constexpr int NW = 4;                 // waves per workgroup
    static constexpr int NT = 64 * NW;           // threads
    static constexpr int BM = 32 * NW;           // query rows per workgroup
    static constexpr int BN = 32;                // keys per chunk
    static constexpr int NB = D / 32;            // 32-dim output blocks
    static constexpr int CPR = D / 8;            // 16-byte chunks per row
    static constexpr int TILE = BN * D;          // halfs of a K or V slot (swizzled, no pad)
    static constexpr int PIECES = TILE * 2 / 1024 / NW;  // 1 KB loads per wave per chunk
    static constexpr int QPIECES = BM * D * 2 / 1024 / NW;
    static constexpr int RPP = 1024 / (D * 2);   // rows per 1 KB piece
    static_assert(PIECES == 2 && 2 * NB == 8, "one load after each of the first four P V MFMAs");
    static_assert(PIECES * NW * 1024 == TILE * 2, "chunk split into 1 KB pieces");
    static_assert(QPIECES * NW * 1024 == BM * D * 2, "Q tile split into 1 KB pieces");
    static_assert(2 * (4 * TILE + BM * D) * 2 <= 160 * 1024, "LDS budget for two workgroups per CU");
};

// K slot and Q tile swizzle: 16-byte chunk index XOR row & 15, so that the 16
// rows one group of 16 lanes reads at a common logical chunk land on 16
// distinct bank groups.
__device__ __forceinline__ int swz_k(int r) { return r & 15; }
// V slot swizzle for the transposed reads.
__device__ __forceinline__ int swz_v(int r) { return 4 * (r & 3); }

// The LDS arrays of a workgroup: two K slots, two V slots and the Q tile,
// separate objects so that the compiler can tell a read of one from a load
// into another.
struct RowSlots {
    _Float16* k[2];
    _Float16* v[2];
    _Float16* q;
};

template <bool CAUSAL>
struct Rows {
    using G = GeoR;
    static constexpr int D = G::D;
    static constexpr int NB = G::NB;
    using LdsPtr = __attribute__((address_space(3))) void*;

    const _Float16* __restrict__ Q;
    const _Float16* __restrict__ K;
    const _Float16* __restrict__ V;
    _Float16* __restrict__ O;
    float* __restrict__ LSE;
    RowSlots sl;
    int S;
    size_t base, lse_base;
    float c;
    uint32_t qsign;
    // w: the wave (its share of every load); wr: its 32-row group of the tile
    int lane, g, n, w, wr;

    // Buffer over rows r0 .. min(r0 + rows, S) - 1 of t: reads past them
    // return zero (an empty buffer when r0 >= S).  r0 is uniform;
    // readfirstlane keeps the descriptor in scalar registers.
    __device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const _Float16* t, int r0,
                                                               int rows) const {
        r0 = __builtin_amdgcn_readfirstlane(r0);
        return __builtin_amdgcn_make_buffer_rsrc(const_cast<_Float16*>(t + base + (size_t)r0 * D),
                                                 (short)0, (S > r0 ? min(S - r0, rows) : 0) * D * 2,
                                                 0x00020000);
    }
    // One 1 KB piece (rows RPP*piece ..) of a chunk or of the Q tile from the
    // buffer r straight into LDS at dst.  Lane L lands at byte 16 L of the
    // piece, i.e. row RPP*piece + L / CPR at physical chunk L % CPR, so it
    // loads the logical chunk that the swizzle puts there.  Inline assembly
    // with M0 = the piece's LDS address: the only waits on these loads are the
    // explicit ones before the barriers.
    __device__ __forceinline__ void dma_piece(_Float16* dst, const __amdgpu_buffer_rsrc_t r,
                                              int piece, bool isk) const {
        const int row = G::RPP * piece + lane / G::CPR;
        const int phys = lane % G::CPR;
        const int logical = phys ^ (isk ? swz_k(row) : swz_v(row));
        const uint32_t m0 = (uint32_t)(uintptr_t)(LdsPtr)(dst + piece * 512);
        // s_nop: one wait state between the M0 write and its use
        asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
                     :
                     : "v"((row * D + 8 * logical) * 2), "s"(r), "{m0}"(m0)
                     : "memory");
    }
    // This wave's pieces of chunk j of K (isk) or V.
    __device__ __forceinline__ void dma(_Float16* slot, int j, bool isk) const {
        const auto r = rows_rsrc(isk ? K : V, j * G::BN, G::BN);
#pragma unroll
        for (int u = 0; u < G::PIECES; ++u) dma_piece(slot, r, w * G::PIECES + u, isk);
    }
    // K fragment kk (head dims 16kk + 8g .. +7) of the chunk's key n: the A
    // operand of S^T = K Q^T.
    __device__ __forceinline__ half8 read_k1(const _Float16* slot, int kk) const {
        return *reinterpret_cast<const half8*>(slot + n * D + 8 * ((2 * kk + g) ^ swz_k(n)));
    }
    // One V^T fragment vf[h][b] (keys 16h .. +15 of the chunk, head dims
    // 32b .. +31).  In each 16-lane group lane 4r + c addresses row r,
    // columns 4c .. 4c+3 of a transposed read and receives column lane % 16
    // of rows 0..3, so two reads give the accumulator's key order
    // 8(r/4) + 4g + r%4.
    __device__ __forceinline__ half8 read_v1(const _Float16* slot, int h, int b) const {
        const int n16 = n >> 4, jj = n & 15;
        const int sub = (jj & 3) >> 1, half = (jj & 1);
        const int sw = swz_v(jj >> 2);  // row & 3 == jj >> 2 for every read below
        const _Float16* pb = slot + (4 * g + (jj >> 2)) * D + 4 * half +
                             8 * ((4 * b + 2 * n16 + sub) ^ sw);
        half4 part[2];
#pragma unroll
        for (int t = 0; t < 2; ++t)
            part[t] = __builtin_bit_cast(
                half4, __builtin_amdgcn_ds_read_tr16_b64_v4f16((lds_half4*)(pb + (16 * h + 8 * t) * D)));
        return half8{part[0][0], part[0][1], part[0][2], part[0][3],
                     part[1][0], part[1][1], part[1][2], part[1][3]};
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
    // Barrier after this wave's loads and LDS accesses have landed.
    __device__ __forceinline__ void barrier_dma() const {
        asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
    }
    // Phase 2's loads without the products (a wave past its diagonal chunk):
    // K(j+3) over K(j+1), V(j+2) over V(j).
    template <int P>
    __device__ __forceinline__ void loads_only(int j, int nk) const {
        if (j + 3 < nk) dma(sl.k[P ^ 1], j + 3, true);
        if (j + 2 < nk) dma(sl.v[P], j + 2, false);
    }

    // Chunk j (P = j & 1) of a wave whose diagonal chunk cw is later, entered
    // with the K(j+1) and V(j) fragments in registers and the loads of K(j+2)
    // and V(j+1) in flight:
    //   S(j+1) = K(j+1) Q^T alongside the softmax of S(j) (no mask);
    //   wait for the loads, barrier;
    //   O += V(j)^T P(j), one matrix instruction at a time, the first four
    //   each followed by one 1 KB load (K(j+3) over K(j+1), then V(j+2) over
    //   V(j), both last read before this barrier), every one by one K(j+2)
    //   fragment read and the read of the V(j+1) fragment into the registers
    //   it consumed.
    // ALL: the caller knows j + 3 < nk (both loads and the K read happen; no
    // branches around them).
    template <int P, bool ALL>
    __device__ __forceinline__ void iter(int j, int nk, int lim0, const half8* qf, half8* kf,
                                         half8 (*vf)[NB], floatx16& s_cur, float& m, float& l,
                                         floatx16* o) {
        const floatx16 s_next = qk(kf, qf);
        half8 pf[2];
        softmax_block<false, NB, true>(s_cur, lim0 - j * G::BN, c, m, l, o, pf);
        barrier_dma();
        // The P V products and their loads at raised issue priority: the
        // SIMD's other wave (the CU's other workgroup) then fills the gaps
        // with its Q K^T and softmax instead of contending with this burst
        // (1-3% on the paired and unpaired shapes).
        __builtin_amdgcn_s_setprio(1);
        const bool dk = ALL || j + 3 < nk, dv = ALL || j + 2 < nk;
        const auto rk = rows_rsrc(K, (j + 3) * G::BN, G::BN);
        const auto rv = rows_rsrc(V, (j + 2) * G::BN, G::BN);
#pragma unroll
        for (int i = 0; i < 2 * NB; ++i) {
            const int h = i / NB, b = i % NB;
            o[b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf[h][b], pf[h], o[b], 0, 0, 0);
            if (i < G::PIECES) {
                if (dk) dma_piece(sl.k[P ^ 1], rk, w * G::PIECES + i, true);
            } else if (i < 2 * G::PIECES) {
                if (dv) dma_piece(sl.v[P], rv, w * G::PIECES + i - G::PIECES, false);
            }
            if (dv) kf[i] = read_k1(sl.k[P], i);
            vf[h][b] = read_v1(sl.v[P ^ 1], h, b);
            __builtin_amdgcn_sched_barrier(0);
        }
        __builtin_amdgcn_s_setprio(0);
        s_cur = s_next;
    }

    // The prologue loads of query tile qt: K(0), the Q tile, V(0) and, when
    // the tile has more than one chunk, K(1), in that order (2 + 8 + 2 + 2
    // loads of this wave).
    __device__ __forceinline__ void prologue_loads(int qt, int nk) const {
        dma(sl.k[0], 0, true);
        const auto rq = rows_rsrc(Q, qt * G::BM, G::BM);
#pragma unroll
        for (int u = 0; u < G::QPIECES; ++u) dma_piece(sl.q, rq, w * G::QPIECES + u, true);
        dma(sl.v[0], 0, false);
        if (nk > 1) dma(sl.k[1], 1, true);
    }
    static_assert(G::PIECES == 2, "the prologue waits count 2 loads per chunk");

    // Query tile qt (rows 128 qt ..), chunks 0 .. nk-1 of the workgroup.
    // issued: the prologue loads were issued already (by the previous tile of
    // this workgroup, after its last barrier).  nxt >= 0: after this tile's
    // last barrier, when no wave reads the LDS any more, issue the prologue
    // loads of tile nxt (nk_nxt chunks) ahead of this tile's epilogue.
    // STEADY: run the chunks whose loads all happen (j + 3 < nk) through a
    // copy of the step without branches around its loads (faster with one
    // workgroup per CU; with two, the branch-free copy measured slower).
    template <bool STEADY>
    __device__ void run(int qt, int nk, bool issued, int nxt, int nk_nxt) {
        const int q0 = qt * G::BM;
        const int row = q0 + 32 * wr + n;
        // last key this lane's row may see
        const int vis = CAUSAL ? min(row, S - 1) : S - 1;
        // this wave's last chunk: the one holding its rows' diagonal (or the
        // last key); every key of the earlier ones is visible to all its rows
        const int cw = CAUSAL ? min(q0 + 32 * wr, S - 1) / G::BN : nk - 1;

        // prologue: K(0), Q, V(0), K(1) into their slots; wait for K(0) and
        // Q, barrier; the Q fragments (sign-flipped for a negative scale) and
        // S(0); wait for V(0) and K(1), barrier; the K(1) and V(0)
        // fragments; a barrier (every wave is done with K(0)); then the loads
        // of K(2) and V(1).  Loads complete in order, so leaving the last
        // 2 or 4 outstanding waits for K(0) and Q; after loads issued by the
        // previous tile, its O stores came later, and the first wait takes
        // everything.
        if (!issued) {
            prologue_loads(qt, nk);
            if (nk > 1)
                asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
            else
                asm volatile("s_waitcnt vmcnt(2)" ::: "memory");
        } else {
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        }
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        half8 qf[D / 16];
        {
            const int qrow = 32 * wr + n;
            const _Float16* qp = sl.q + qrow * D;
            const int sw = swz_k(qrow);
#pragma unroll
            for (int kk = 0; kk < D / 16; ++kk) {
                u32x4 x = *reinterpret_cast<const u32x4*>(qp + 8 * ((2 * kk + g) ^ sw));
                x ^= qsign;
                qf[kk] = __builtin_bit_cast(half8, x);
            }
        }
        half8 kf[D / 16];
        half8 vf[2][NB];
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) kf[kk] = read_k1(sl.k[0], kk);
        floatx16 s_cur = qk(kf, qf);
        barrier_dma();
        if (nk > 1) {
#pragma unroll
            for (int kk = 0; kk < D / 16; ++kk) kf[kk] = read_k1(sl.k[1], kk);
        }
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int b = 0; b < NB; ++b) vf[h][b] = read_v1(sl.v[0], h, b);
        barrier_dma();
        if (nk > 2) dma(sl.k[0], 2, true);
        if (nk > 1) dma(sl.v[1], 1, false);

        float m = kNegInf, l = 0.f;
        floatx16 o[NB];
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) o[b][r] = 0.f;

        const int lim0 = vis - 4 * g;  // minus 32 j for chunk j
        // the pipelined chunks before the diagonal (one barrier each)
        int j = 0;
        for (; STEADY && j + 2 <= cw && j + 4 < nk; j += 2) {
            iter<0, true>(j, nk, lim0, qf, kf, vf, s_cur, m, l, o);
            iter<1, true>(j + 1, nk, lim0, qf, kf, vf, s_cur, m, l, o);
        }
        for (; j + 2 <= cw; j += 2) {
            iter<0, false>(j, nk, lim0, qf, kf, vf, s_cur, m, l, o);
            iter<1, false>(j + 1, nk, lim0, qf, kf, vf, s_cur, m, l, o);
        }
        if (j < cw) {
            iter<0, false>(j, nk, lim0, qf, kf, vf, s_cur, m, l, o);
            ++j;
        }
        // the diagonal chunk j = cw: masked softmax, barrier, O += V^T P with
        // the loads of this iteration
        {
            half8 pf[2];
            softmax_block<true, NB, false>(s_cur, lim0 - j * G::BN, c, m, l, o, pf);
            barrier_dma();
            if (j & 1)
                loads_only<1>(j, nk);
            else
                loads_only<0>(j, nk);
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int b = 0; b < NB; ++b)
                    o[b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf[h][b], pf[h], o[b], 0, 0, 0);
            ++j;
        }
        // the chunks after the diagonal: this wave's share of the loads and
        // the barriers only
        for (; j < nk; ++j) {
            barrier_dma();
            if (j & 1)
                loads_only<1>(j, nk);
            else
                loads_only<0>(j, nk);
        }
        // every load of this tile was waited for before the last barrier
        if (nxt >= 0) prologue_loads(nxt, nk_nxt);

        // O = O / l, fp16, and LSE.  Register r of block b holds head dim
        // 32b + 8(r/4) + 4g + r%4; lanes n and n+32 swap halves
        // (v_permlane32_swap, no LDS round trip) so that each lane stores 8
        // consecutive dims (16 bytes).
        const float lt = sum_halves(l);
        const float inv = 1.0f / lt;
        _Float16* orow = O + base + (size_t)min(row, S - 1) * D;
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            u32x2 x[4];
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const float x0 = o[b][4 * q4] * inv, x1 = o[b][4 * q4 + 1] * inv;
                const float x2 = o[b][4 * q4 + 2] * inv, x3 = o[b][4 * q4 + 3] * inv;
                x[q4][0] = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)x0) |
                           ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)x1) << 16);
                x[q4][1] = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)x2) |
                           ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)x3) << 16);
            }
#pragma unroll
            for (int qq = 0; qq < 2; ++qq) {
                const auto s0 = __builtin_amdgcn_permlane32_swap(x[2 * qq][0], x[2 * qq + 1][0],
                                                                 false, false);
                const auto s1 = __builtin_amdgcn_permlane32_swap(x[2 * qq][1], x[2 * qq + 1][1],
                                                                 false, false);
                const u32x4 v = u32x4{s0[0], s1[0], s0[1], s1[1]};
                if (row < S) *reinterpret_cast<u32x4*>(orow + 32 * b + 16 * qq + 8 * g) = v;
            }
        }
        if (row < S && g == 0) LSE[lse_base + row] = (m + __builtin_amdgcn_logf(lt)) * kLn2;
    }
};

template <bool CAUSAL, bool PAIRED>
__global__ void __launch_bounds__(256, 2)
fwd_rows_kernel(const _Float16* __restrict__ Q, const _Float16* __restrict__ K,
                const _Float16* __restrict__ V, _Float16* __restrict__ O, float* __restrict__ LSE,
                int BH, int S, float c, uint32_t qsign)
{
    using G = GeoR;
    __shared__ __attribute__((aligned(1024))) _Float16 k0[G::TILE];
    __shared__ __attribute__((aligned(1024))) _Float16 k1[G::TILE];
    __shared__ __attribute__((aligned(1024))) _Float16 v0[G::TILE];
    __shared__ __attribute__((aligned(1024))) _Float16 v1[G::TILE];
    __shared__ __attribute__((aligned(1024))) _Float16 qs[G::BM * G::D];
    const int T = (S + G::BM - 1) / G::BM;
    const int bh = blockIdx.x % BH;
    const int u = blockIdx.x / BH;
    // causal: the heaviest query tiles first, so that the dispatcher, handing
    // out workgroups in order as CU slots free up, fills in the light ones
    // last.  Paired (causal, many tiles): workgroup u runs tile T-1-u and then
    // tile u of its (batch, head), T+1 tile-lengths of work for every
    // workgroup.
    const int qt0 = CAUSAL ? T - 1 - u : u;

    Rows<CAUSAL> f;
    f.Q = Q;
    f.K = K;
    f.V = V;
    f.O = O;
    f.LSE = LSE;
    f.sl.k[0] = k0;
    f.sl.k[1] = k1;
    f.sl.v[0] = v0;
    f.sl.v[1] = v1;
    f.sl.q = qs;
    f.S = S;
    f.base = (size_t)bh * S * G::D;
    f.lse_base = (size_t)bh * S;
    f.c = c;
    f.qsign = qsign;
    f.lane = threadIdx.x & 63;
    f.g = f.lane >> 5;
    f.n = f.lane & 31;
    f.w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    // odd u: row groups in reverse order.  Under causal masking the wave with
    // row group r idles after its diagonal chunk for 3 - r chunks; the
    // dispatcher gives every CU one workgroup of the grid's first half and
    // one of its second, i.e. u and u+1 of a head when the grid fills the
    // chip once, with wave w of each on SIMD w: reversed, each SIMD gets one
    // early- and one late-finishing wave
    f.wr = (u & 1) ? 3 - f.w : f.w;
    const int nk0 = ((CAUSAL ? min(S, (qt0 + 1) * G::BM) : S) + G::BN - 1) / G::BN;
    const bool two = PAIRED && u != qt0;
    const int nk1 = (min(S, (u + 1) * G::BM) + G::BN - 1) / G::BN;
    // one copy of the tile code for both tiles of a pair
    int qt = qt0, nk = nk0;
#pragma unroll 1
    for (int it = 0; it < (two ? 2 : 1); ++it) {
        // opaque lane indices: the second tile recomputes its per-lane
        // offsets instead of keeping the first tile's alive across it
        asm volatile("" : "+v"(f.lane), "+v"(f.g), "+v"(f.n));
        f.template run<!PAIRED>(qt, nk, it > 0, (it == 0 && two) ? u : -1, nk1);
        qt = u;
        nk = nk1;
    }
}

}  // namespace

hipError_t launch_fused_rows_d128(const FwdArgs& a) {
    using G = GeoR;
    const int BH = a.B * a.H;
    const int T = (a.S + G::BM - 1) / G::BM;
    const float c = fabsf(a.scale) * 1.44269504088896340736f;
    const uint32_t qsign = a.scale < 0.f ? 0x80008000u : 0u;
    // causal tiles in pairs (T-1-u, u) when the pairs alone still give two
    // workgroups per CU (256 CUs)
    const int pairs = (T + 1) / 2;
    const int paired = a.causal && (long long)BH * pairs >= 512;
    const dim3 grid((unsigned)((long long)BH * (paired ? pairs : T)));
#define ROWS_LAUNCH(C, P)                                                                   \
    hipLaunchKernelGGL((fwd_rows_kernel<C, P>), grid, dim3(G::NT), 0, (hipStream_t)a.stream, \
                       (const _Float16*)a.q, (const _Float16*)a.k, (const _Float16*)a.v,     \
                       (_Float16*)a.o, a.lse, BH, a.S, c, qsign)
    if (paired)
        ROWS_LAUNCH(true, true);
    else if (a.causal)
        ROWS_LAUNCH(true, false);
    else
        ROWS_LAUNCH(false, false);
#undef ROWS_LAUNCH
    return hipGetLastError();
}

}  // namespace attn
