// Fused attention forward for gfx950, D in {64, 128}: one workgroup of four
// waves per 64-row query tile, two workgroups per CU, with the next key
// tile's Q K^T on the matrix cores while the vector ALUs run the current
// tile's softmax.
//
//   O = softmax(scale * Q K^T + causal mask) V,   LSE = log sum_j exp(scale q.k_j)
//
// The score tile lives only in registers ("An Optimal Mapper Meets a Real
// GPU", section "Ground rules": one fused kernel instead of a pipeline of
// kernels through global workspaces).
//
// Wave w takes query rows 32(w&1) .. +31 of the tile against keys
// 32(w>>1) .. +31 of every 64-key tile; the two key halves are merged in LDS
// at the end (an online-softmax merge over disjoint key sets, exact up to
// rounding, fixed order).
//
// Software pipeline, per key tile j of a wave:
//     S(j+1) = K(j+1) Q^T        matrix cores   \  issued together, no
//     P(j)   = softmax(S(j))     vector ALUs    /  dependence between them
//     O     += V(j)^T P(j)       matrix cores
// so K runs one tile ahead of V.  K and V tiles go from global memory
// straight into LDS (buffer loads with the LDS destination bit: no
// registers, no LDS write instructions), into two K slots and two V slots,
// each a separate LDS array.  Iteration j starts with the K(j+1) and V(j)
// fragments in registers and the loads of K(j+2) and V(j+1) in flight;
// after S(j+1) and the softmax of S(j) every wave waits for its loads and
// meets the barrier, then runs O += V(j)^T P(j) one matrix instruction at a
// time, each followed by one 1 KB load (K(j+3) over K(j+1), then V(j+2)
// over V(j), both read before the barrier), one K(j+2) fragment read and
// the V(j+1) fragment that replaces the one the instruction consumed.  No
// LDS latency sits between the barrier and the next matrix instruction.
//
// The Q tile comes in the same way (through the second V slot, before V(1)
// needs it) and then stays in registers as the B operand of Q K^T.
//
// The K slots are XOR-swizzled by row (no padding, so that a 1 KB load
// lands as whole rows), the V slots as for the transposed reads.
//
// MFMA lane layouts (v_mfma_f32_32x32x16_f16, wave64, g = lane / 32,
// n = lane % 32):
//   A[m][k]: lane holds m = n, k = 8g .. 8g+7
//   B[k][n]: lane holds n = n, k = 8g .. 8g+7
//   C[m][n]: register r holds m = 8(r/4) + 4g + r%4, n = n
// S^T = K Q^T puts one query per lane (n) and 16 of the wave's 32 keys in
// its registers; O^T += V^T P^T takes P^T straight from those registers as
// the B operand and V^T from transposed LDS reads (ds_read_b64_tr_b16).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fwd_common.h"
#include "kernels.h"

namespace attn {
namespace {

using namespace detail;

template <int D>
struct GeoP {
    static constexpr int NW = 4;                 // waves per workgroup
    static constexpr int NT = 64 * NW;           // threads
    static constexpr int BM = 64;                // query rows per tile
    static constexpr int BN = 64;                // keys per tile
    static constexpr int CPR = D / 8;            // 16-byte chunks per row
    static constexpr int TILE = BN * D;          // halfs of a K or V slot (swizzled, no pad)
    static constexpr int PIECES = TILE * 2 / 1024 / NW;  // 1 KB DMA pieces per wave per tile
    static constexpr int ROWS_PER_PIECE = 1024 / (D * 2);
    static constexpr int SLOT = 16 * D + 128;    // floats of one wave's merge slot
    static_assert(D == 64 || D == 128, "D");
    static_assert(PIECES * NW * 1024 == TILE * 2, "tile split into 1 KB pieces");
    static_assert(4 * TILE * 2 * 2 <= 160 * 1024, "LDS budget for two workgroups per CU");
    static_assert(SLOT * 4 <= TILE * 2, "a merge slot fits one tile array");
};

// K slot swizzle (16-byte chunk index XOR): the 16 rows that one group of 16
// lanes reads at a common logical chunk land on 16 distinct bank groups.
template <int D>
__device__ __forceinline__ int swz_k(int r) {
    return D == 128 ? (r & 15) : ((r >> 1) & 7);
}

// V slot swizzle: 16-byte chunk index XOR, so that the lanes of a transposed
// read hit distinct banks.
template <int D>
__device__ __forceinline__ int swz_vp(int r) {
    return D == 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1);
}

// The four LDS tile arrays of a workgroup: two K slots and two V slots.
// They are separate objects so that the compiler can tell a DMA into one
// from a read of another and never waits for the former before the latter.
template <int D>
struct Slots {
    _Float16* k[2];
    _Float16* v[2];
};

template <int D, bool CAUSAL>
struct Pipe {
    using G = GeoP<D>;
    static constexpr int NB = D / 32;
    using LdsPtr = __attribute__((address_space(3))) void*;

    const _Float16* __restrict__ Q;
    const _Float16* __restrict__ K;
    const _Float16* __restrict__ V;
    _Float16* __restrict__ O;
    float* __restrict__ LSE;
    Slots<D> sl;
    int S;
    size_t base, lse_base;
    float c;
    uint32_t qsign;
    int tid, lane, g, n, w, rg, kh;

    // Buffer over rows j0 .. min(j0 + 64, S) - 1 of t: reads past them return zero.
    __device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const _Float16* t, int j0) const {
        return __builtin_amdgcn_make_buffer_rsrc(const_cast<_Float16*>(t + base + (size_t)j0 * D),
                                                 (short)0, min(S - j0, G::BN) * D * 2, 0x00020000);
    }
    // One 1 KB piece (u < PIECES) of this wave's share of a tile, from the
    // buffer r straight into an LDS slot (global -> LDS, no registers).  Lane
    // L of a piece lands at byte 16 L of it, i.e. row ROWS_PER_PIECE * piece
    // + L / CPR at physical chunk L % CPR, so it loads the logical chunk that
    // the swizzle puts there.
    //
    // The load is written as inline assembly (M0 = LDS address of the piece)
    // rather than the compiler builtin: for the builtin the compiler cannot
    // tell that a later transposed LDS read of another slot does not alias the
    // load's destination, and waits for every load in flight before that
    // read, i.e. for the tiles just issued.  Here the only waits are the
    // explicit ones in barrier_dma(), which every reader of a slot passes
    // after the load into that slot.
    __device__ __forceinline__ void dma_piece(_Float16* slot, const __amdgpu_buffer_rsrc_t r,
                                              int u, bool isk) const {
        const int piece = w * G::PIECES + u;
        const int row = G::ROWS_PER_PIECE * piece + lane / G::CPR;
        const int phys = lane % G::CPR;
        const int logical = phys ^ (isk ? swz_k<D>(row) : swz_vp<D>(row));
        const uint32_t m0 = (uint32_t)(uintptr_t)(LdsPtr)(slot + piece * 512);
        // s_nop: one wait state between the M0 write and its use
        asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
                     :
                     : "v"((row * D + 8 * logical) * 2), "s"(r), "{m0}"(m0)
                     : "memory");
    }
    // Tile j of t, this wave's pieces.
    __device__ __forceinline__ void dma(_Float16* slot, const _Float16* t, int j, bool isk) const {
        const auto r = tile_rsrc(t, j * G::BN);
#pragma unroll
        for (int u = 0; u < G::PIECES; ++u) dma_piece(slot, r, u, isk);
    }
    // K fragments of keys 32kh .. +31 (A operand of S^T = K Q^T)
    __device__ __forceinline__ void read_k(half8* kf, const _Float16* slot) const {
        const int row = 32 * kh + n;
        const _Float16* kp = slot + row * D;
        const int sw = swz_k<D>(row);
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk)
            kf[kk] = *reinterpret_cast<const half8*>(kp + 8 * ((2 * kk + g) ^ sw));
    }
    // V^T fragments of keys 32kh .. +31: vf[h][b] covers keys 32kh + 16h .. +15
    // and head dims 32b .. +31.  In each 16-lane group lane 4r + c addresses
    // row r, columns 4c .. 4c+3 of a transposed read and receives column
    // lane % 16 of rows 0..3, so two reads give the accumulator's key order
    // 8(r/4) + 4g + r%4.
    __device__ __forceinline__ void read_v(half8 (*vf)[NB], const _Float16* slot) const {
        const int n16 = n >> 4, jj = n & 15;
        const int sub = (jj & 3) >> 1, half = (jj & 1);
        const int sw = swz_vp<D>(jj >> 2);  // row & 3 == jj >> 2 for every read below
        const _Float16* rowp = slot + (32 * kh + 4 * g + (jj >> 2)) * D + 4 * half;
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const _Float16* pb = rowp + 8 * ((4 * b + 2 * n16 + sub) ^ sw);
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                half4 part[2];
#pragma unroll
                for (int t = 0; t < 2; ++t)
                    part[t] = __builtin_bit_cast(
                        half4, __builtin_amdgcn_ds_read_tr16_b64_v4f16(
                                   (lds_half4*)(pb + (16 * h + 8 * t) * D)));
                vf[h][b] = half8{part[0][0], part[0][1], part[0][2], part[0][3],
                                 part[1][0], part[1][1], part[1][2], part[1][3]};
            }
        }
    }
    // One V^T fragment vf[h][b] (keys 32kh + 16h .. +15, head dims 32b .. +31).
    __device__ __forceinline__ half8 read_v1(const _Float16* slot, int h, int b) const {
        const int n16 = n >> 4, jj = n & 15;
        const int sub = (jj & 3) >> 1, half = (jj & 1);
        const int sw = swz_vp<D>(jj >> 2);
        const _Float16* pb = slot + (32 * kh + 4 * g + (jj >> 2)) * D + 4 * half +
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
    __device__ __forceinline__ void pv(floatx16* o, const half8 (*vf)[NB], const half8* pf) const {
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int b = 0; b < NB; ++b)
                o[b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf[h][b], pf[h], o[b], 0, 0, 0);
    }
    // Barrier after this wave's DMA writes and LDS accesses have landed.
    __device__ __forceinline__ void barrier_dma() const {
        asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
    }

    // Iteration j (P = j & 1), entered with K(j+1) and V(j) fragments in
    // registers and the DMA of K(j+2) and V(j+1) in flight:
    //   S(j+1) = K(j+1) Q^T alongside the softmax of S(j);
    //   wait for the DMA, barrier;
    //   O += V(j)^T P(j), each matrix instruction followed by one 1 KB load
    //   (K(j+3) over K(j+1), then V(j+2) over V(j), both slots last read
    //   before this barrier), one K(j+2) fragment read and the read of the
    //   V(j+1) fragment into the registers that instruction consumed: a wave
    //   stalls on issuing a load while the texture unit drains the other
    //   waves' loads, and this way the matrix core works through those
    //   stalls and the LDS reads issue under them.
    template <int P>
    __device__ __forceinline__ void iter(int j, int nk, int lim0, const half8* qf, half8* kf,
                                         half8 (*vf)[NB], floatx16& s_cur, float& m, float& l,
                                         floatx16* o) {
        const floatx16 s_next = qk(kf, qf);
        half8 pf[2];
        softmax_block<false, NB, true>(s_cur, lim0 - j * G::BN, c, m, l, o, pf);
        barrier_dma();
        // O += V(j)^T P(j), one matrix instruction at a time, each followed
        // by one 1 KB tile load (K(j+3), then V(j+2)), one K(j+2) fragment
        // read and one V(j+1) fragment, so that the loads queue at the
        // texture unit while the matrix core runs
        {
            const bool dk = j + 3 < nk, dv = j + 2 < nk;
            const auto rk = tile_rsrc(K, (j + 3) * G::BN);
            const auto rv = tile_rsrc(V, (j + 2) * G::BN);
            const int krow = 32 * kh + n;
            const _Float16* kp = sl.k[P] + krow * D;
            const int ksw = swz_k<D>(krow);
            static_assert(2 * NB == 2 * G::PIECES && 2 * NB == D / 16, "one load and one read per MFMA");
#pragma unroll
            for (int i = 0; i < 2 * NB; ++i) {
                const int h = i / NB, b = i % NB;
                o[b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf[h][b], pf[h], o[b], 0, 0, 0);
                if (i < G::PIECES) {
                    if (dk) dma_piece(sl.k[P ^ 1], rk, i, true);
                } else {
                    if (dv) dma_piece(sl.v[P], rv, i - G::PIECES, false);
                }
                if (dv) kf[i] = *reinterpret_cast<const half8*>(kp + 8 * ((2 * i + g) ^ ksw));
                // the fragment this MFMA consumed, now of V(j+1)
                vf[h][b] = read_v1(sl.v[P ^ 1], h, b);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        s_cur = s_next;
    }

    // Query tile qt over key tiles 0 .. nk-1.
    __device__ void run(int qt, int nk) {
        const int row = qt * G::BM + 32 * rg + n;
        // last key this lane's row may see
        const int vis = CAUSAL ? min(row, S - 1) : S - 1;
        // the last key tile needs a mask: the diagonal (causal) or a ragged end
        const bool mask_end = CAUSAL || (S % G::BN) != 0;

        // prologue: K(0), Q, V(0), K(1) into their slots (Q through v[1],
        // free until V(1) is loaded, laid out like a K tile: sixteen 1 KB
        // loads instead of each lane gathering its row 16 bytes at a time);
        // wait for K(0) and Q only (the last 2 or 1 tiles' loads may still
        // be in flight), S(0); then wait for the rest, K(1) and V(0)
        // fragments, and the DMA of K(2) and V(1)
        dma(sl.k[0], K, 0, true);
        dma(sl.v[1], Q, qt, true);
        dma(sl.v[0], V, 0, false);
        if (nk > 1) dma(sl.k[1], K, 1, true);
        half8 qf[D / 16];
        if (nk > 1) {
            asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" :: "n"(2 * G::PIECES) : "memory");
        } else {
            asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" :: "n"(G::PIECES) : "memory");
        }
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        {
            const int qrow = 32 * rg + n;
            const _Float16* qp = sl.v[1] + qrow * D;
            const int sw = swz_k<D>(qrow);
#pragma unroll
            for (int kk = 0; kk < D / 16; ++kk) {
                u32x4 x = *reinterpret_cast<const u32x4*>(qp + 8 * ((2 * kk + g) ^ sw));
                x ^= qsign;
                qf[kk] = __builtin_bit_cast(half8, x);
            }
        }
        half8 kf[D / 16];
        half8 vf[2][NB];
        read_k(kf, sl.k[0]);
        floatx16 s_cur = qk(kf, qf);
        // V(0) and K(1) landed everywhere; every wave is done with K(0) and Q
        // before K(2) and V(1) go over them
        barrier_dma();
        if (nk > 1) read_k(kf, sl.k[1]);
        read_v(vf, sl.v[0]);
        if (nk > 2) dma(sl.k[0], K, 2, true);
        if (nk > 1) dma(sl.v[1], V, 1, false);

        float m = kNegInf, l = 0.f;
        floatx16 o[NB];
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) o[b][r] = 0.f;

        const int lim0 = vis - (32 * kh + 4 * g);  // add -64 j for tile j
        for (int j = 0; j + 1 < nk; j += 2) {
            iter<0>(j, nk, lim0, qf, kf, vf, s_cur, m, l, o);
            if (j + 2 < nk) iter<1>(j + 1, nk, lim0, qf, kf, vf, s_cur, m, l, o);
        }
        {
            const int j = nk - 1;
            half8 pf[2];
            if (mask_end)
                softmax_block<true, NB, false>(s_cur, lim0 - j * G::BN, c, m, l, o, pf);
            else
                softmax_block<false, NB, false>(s_cur, lim0 - j * G::BN, c, m, l, o, pf);
            pv(o, vf, pf);
        }

        // merge the two key halves: each wave publishes the output blocks the
        // other one writes (b % 2 != kh) and its (m, l) into its own tile
        // array, then combines and writes its own blocks
        barrier_dma();
        // wave (rg, kh) owns tile array 2 rg + kh (selected, not indexed, so
        // that no pointer table goes to scratch memory)
        auto arr = [&](int i) -> _Float16* {
            return i == 0 ? sl.k[0] : i == 1 ? sl.k[1] : i == 2 ? sl.v[0] : sl.v[1];
        };
        float* mine = reinterpret_cast<float*>(arr(2 * rg + kh));
        const float* theirs = reinterpret_cast<const float*>(arr(2 * rg + (kh ^ 1)));
#pragma unroll
        for (int b = 0; b < NB; ++b)
            if ((b & 1) != kh)
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4)
                    reinterpret_cast<float4*>(mine)[((b >> 1) * 4 + q4) * 64 + lane] =
                        float4{o[b][4 * q4], o[b][4 * q4 + 1], o[b][4 * q4 + 2], o[b][4 * q4 + 3]};
        mine[16 * D + lane] = m;
        mine[16 * D + 64 + lane] = l;
        barrier_dma();
        const float m1 = theirs[16 * D + lane], l1 = theirs[16 * D + 64 + lane];
        const float mt = fmaxf(m, m1);  // finite: every row sees key 0 in the kh = 0 half
        const float a0 = m == kNegInf ? 0.f : __builtin_amdgcn_exp2f(m - mt);
        const float a1 = m1 == kNegInf ? 0.f : __builtin_amdgcn_exp2f(m1 - mt);
        const float lt = sum_halves(l * a0 + l1 * a1);
        const float inv = 1.0f / lt;
        // register r of block b holds head dim 32b + 8(r/4) + 4g + r%4; lanes
        // n and n+32 swap halves (v_permlane32_swap, no LDS round trip) so
        // that each lane stores 8 consecutive dims (16 bytes): lane g = 0
        // keeps dim group q4 = 2qq, g = 1 keeps 2qq+1
        _Float16* orow = O + base + (size_t)min(row, S - 1) * D;
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            if ((b & 1) != kh) continue;
            u32x2 x[4];
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const float4 p1 = reinterpret_cast<const float4*>(theirs)[((b >> 1) * 4 + q4) * 64 + lane];
                const float x0 = (o[b][4 * q4] * a0 + p1.x * a1) * inv;
                const float x1 = (o[b][4 * q4 + 1] * a0 + p1.y * a1) * inv;
                const float x2 = (o[b][4 * q4 + 2] * a0 + p1.z * a1) * inv;
                const float x3 = (o[b][4 * q4 + 3] * a0 + p1.w * a1) * inv;
                x[q4][0] = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)x0) |
                           ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)x1) << 16);
                x[q4][1] = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)x2) |
                           ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)x3) << 16);
            }
#pragma unroll
            for (int qq = 0; qq < 2; ++qq) {
                // swap the upper half-wave's x[2qq] with the lower half-wave's
                // x[2qq+1]: afterwards the first result holds dims 8g .. 8g+3
                // and the second dims 8g+4 .. 8g+7 of this lane's 16-byte
                // group, in both halves
                const auto s0 = __builtin_amdgcn_permlane32_swap(x[2 * qq][0], x[2 * qq + 1][0],
                                                                 false, false);
                const auto s1 = __builtin_amdgcn_permlane32_swap(x[2 * qq][1], x[2 * qq + 1][1],
                                                                 false, false);
                const u32x4 v = u32x4{s0[0], s1[0], s0[1], s1[1]};
                if (row < S) *reinterpret_cast<u32x4*>(orow + 32 * b + 16 * qq + 8 * g) = v;
            }
        }
        if (row < S) {
            if (kh == 0 && g == 0) LSE[lse_base + row] = (mt + __builtin_amdgcn_logf(lt)) * kLn2;
        }
    }
};

template <int D, bool CAUSAL>
__global__ void __launch_bounds__(256, 2)
fwd_pipe_kernel(const _Float16* __restrict__ Q, const _Float16* __restrict__ K,
                const _Float16* __restrict__ V, _Float16* __restrict__ O, float* __restrict__ LSE,
                int BH, int S, float c, uint32_t qsign)
{
    using G = GeoP<D>;
    __shared__ __attribute__((aligned(1024))) _Float16 k0[G::TILE];
    __shared__ __attribute__((aligned(1024))) _Float16 k1[G::TILE];
    __shared__ __attribute__((aligned(1024))) _Float16 v0[G::TILE];
    __shared__ __attribute__((aligned(1024))) _Float16 v1[G::TILE];
    const int T = (S + G::BM - 1) / G::BM;
    const int bh = blockIdx.x % BH;
    const int u = blockIdx.x / BH;
    // causal: the first half of the grid runs the heavy tiles (last first),
    // the second half the light ones (first first), so that workgroups
    // launched half a grid apart carry complementary work
    int qt = u;
    if (CAUSAL) {
        const int half = (T + 1) / 2;
        qt = u < half ? T - 1 - u : u - half;
    }
    const int nk = CAUSAL ? qt + 1 : T;

    Pipe<D, CAUSAL> f;
    f.Q = Q;
    f.K = K;
    f.V = V;
    f.O = O;
    f.LSE = LSE;
    f.sl.k[0] = k0;
    f.sl.k[1] = k1;
    f.sl.v[0] = v0;
    f.sl.v[1] = v1;
    f.S = S;
    f.base = (size_t)bh * S * D;
    f.lse_base = (size_t)bh * S;
    f.c = c;
    f.qsign = qsign;
    f.tid = threadIdx.x;
    f.lane = threadIdx.x & 63;
    f.g = f.lane >> 5;
    f.n = f.lane & 31;
    f.w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    f.rg = f.w & 1;
    f.kh = f.w >> 1;
    f.run(qt, nk);
}

}  // namespace

hipError_t launch_fused_pipe_d64_d128(const FwdArgs& a) {
    const int BH = a.B * a.H;
    const int T = (a.S + 63) / 64;
    const float c = fabsf(a.scale) * 1.44269504088896340736f;
    const uint32_t qsign = a.scale < 0.f ? 0x80008000u : 0u;
    const dim3 grid((unsigned)((long long)BH * T));
#define LAUNCH(DD, CC)                                                                          \
    hipLaunchKernelGGL((fwd_pipe_kernel<DD, CC>), grid, dim3(256), 0, (hipStream_t)a.stream,   \
                       (const _Float16*)a.q, (const _Float16*)a.k, (const _Float16*)a.v,        \
                       (_Float16*)a.o, a.lse, BH, a.S, c, qsign)
    if (a.D == 64) {
        if (a.causal) LAUNCH(64, true); else LAUNCH(64, false);
    } else {
        if (a.causal) LAUNCH(128, true); else LAUNCH(128, false);
    }
#undef LAUNCH
    return hipGetLastError();
}

}  // namespace attn
