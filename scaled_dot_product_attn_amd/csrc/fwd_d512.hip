// Fused scaled-dot-product attention forward for head dimension 512 (gfx950).
//
// Same operation as the D = 64 / 128 kernel: O = softmax(scale Q K^T + causal
// mask) V with fp16 in / fp32 accumulate / fp16 O and fp32 LSE, scores kept on
// chip.  What changes at D = 512 is how Q K^T is split.  Following the notes on
// the head-dim-512 kernel (STAGE_D.md, sections "2. External k_sub Merge is
// Mathematically Impossible" and "6. The k_tile Parameter"), the head
// dimension is cut into two 256-wide sub-tiles and their partial logits are
// ADDED in logit space, S = S_0 + S_1, before any max or exp: softmax is
// nonlinear, so merging softmax(S_0)V and softmax(S_1)V afterwards would be
// wrong.  Here the two sub-tiles live in two different waves:
//
//   * A workgroup of NW waves owns 32 NW/2 query rows: 64 rows with four
//     waves (split-KV units, fused calls with many tiles), 32 rows with two
//     (fused calls with few tiles).  Wave w handles row group
//     rg = w % (NW/2) (32 rows) and head-dim half dh = w / (NW/2) (256 dims).
//   * Per 32-key tile, wave (rg, dh) computes the partial S^T over its 256
//     dims (16 v_mfma_f32_32x32x16_f16), publishes it in LDS, and after the
//     next barrier adds its partner's (rg, 1-dh) partial: both waves then
//     hold the same S = S_0 + S_1 (fp32 addition is commutative, so they
//     agree bit for bit) and run the same online softmax.
//   * Each wave accumulates O^T for its own 256 output dims (16 MFMAs),
//     reading V^T with ds_read_b64_tr_b16, like the smaller-D kernel.
//     Splitting P V along the output dims is what the notes call the
//     pv_n_tile knob; it keeps a wave's output accumulator at 128 registers.
//   * K and V rows (XOR-swizzled in 16-byte chunks) stream through two LDS
//     stages each, loaded straight from global memory into LDS
//     (bounds-checked buffer loads with the LDS destination bit, one 1 KB row
//     per instruction, no staging registers), issued between the matrix
//     instructions of a two-phase software pipeline (run(), below).
//
// Split-KV.  Eight heads of 1024 rows give only 128 workgroups for 256 CUs, and
// under causal masking the last query tile does 32 key tiles while the first
// does 2.  The split variant cuts every query tile's key range into chunks of
// at most C 32-key tiles; each chunk is one workgroup that leaves its partial
// state (its own normalised O in fp16, row max m and row sum l) in a workspace, and
// a second kernel merges the chunks of a row in chunk order.  The merge is
// exact because the chunks hold DISJOINT key sets (STAGE_D.md notes, section
// "2. External k_sub Merge is Mathematically Impossible": outputs over
// different token sets combine through their weights, unlike head-dim
// sub-tiles); the partial write, re-read and reduction are the split-k costs
// that "An Optimal Mapper Meets a Real GPU" (section "Experiment one: ten
// mappings, forty handwritten kernels", cost term (1)) says must be paid and
// measured.  Query tiles with a single chunk write O and LSE directly.  The
// fused entry point is the same kernel with C = every key tile (one chunk per
// query tile, heaviest first).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fwd_common.h"
#include "kernels.h"

namespace attn {
namespace {

using namespace detail;

// NW waves: NW/2 row groups of 32 query rows, each split over two head-dim
// halves.  NW = 4: 64-row tiles (the split-KV units and large grids);
// NW = 2: 32-row tiles (fused calls with few tiles: twice the workgroups,
// and per key tile half the fragment reads and exchange traffic through the
// CU's LDS, the tile fills being the same).
template <int NW_>
struct G512T {
    static constexpr int D = 512;
    static constexpr int DH = 256;               // head dims per sub-tile
    static constexpr int NW = NW_;
    static constexpr int RG = NW / 2;            // 32-row groups per workgroup
    static constexpr int NT = 64 * NW;
    static constexpr int BM = 32 * RG;           // query rows per workgroup
    static constexpr int BN = 32;                // keys per tile
    static constexpr int NB = DH / 32;           // 32-dim output blocks of a wave
    static constexpr int TILE = BN * D;          // halfs of a K or V stage (swizzled rows, no pad)
    static constexpr int ROWS = BN / NW;         // 1 KB rows a wave loads per K (or V) tile
    static constexpr int XCH = NW * 16 * 64;     // floats of the S^T exchange buffer
    // two K stages, two V stages and the exchange buffer
    static constexpr int LDS_BYTES = 4 * TILE * 2 + XCH * 4;
    static_assert(NW == 2 || NW == 4, "row groups");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
};
using G512 = G512T<4>;

// K row swizzle: 16-byte chunk index XOR (row & 15).  Every 1 KB row starts on
// the same bank, so without it the 16 rows that a group of 16 lanes reads at
// one logical chunk would all hit the same four banks.
__device__ __forceinline__ int swz_k512(int r) { return r & 15; }
// V row swizzle: XOR chunk bits 2-3 with the row's low two bits, so that the
// four rows of a transposed read hit different banks.
__device__ __forceinline__ int swz_v512(int r) { return 4 * (r & 3); }

// A chunk's slot: its normalised partial output O_c / l_c as fp16
// [64][512] (kSlotOFloats floats' worth of bytes), then m [64] (log2 units)
// and l [64] in fp32.
constexpr size_t kSlotOFloats = (size_t)G512::BM * G512::D / 2;
constexpr size_t kSlotFloats = kSlotOFloats + 2 * G512::BM;

template <int NW>
struct Fwd512 {
    using G = G512T<NW>;
    static constexpr int NB = G::NB;
    const _Float16* __restrict__ Q;
    const _Float16* __restrict__ K;
    const _Float16* __restrict__ V;
    _Float16* __restrict__ O;
    float* __restrict__ LSE;
    _Float16* lds;  // the workgroup's LDS: K stages, V stages, exchange buffers
    int S;
    bool causal;
    size_t base, lse_base;
    float c;
    uint32_t qsign;
    int w, lane, g, n, rg, dh;
    using LdsPtr = __attribute__((address_space(3))) void*;

    // x, opaque to the optimiser: lane-dependent LDS and global offsets
    // derived from it are recomputed where they are used (a few VALU
    // instructions) instead of being hoisted out of the key loop, where the
    // dozens of distinct swizzled offsets would each hold a register.
    __device__ __forceinline__ static int fresh(int x) {
        asm volatile("" : "+v"(x));
        return x;
    }

    // Stage addresses by arithmetic on the LDS base (no pointer arrays: a
    // runtime index into one would leave the address space unknown).
    __device__ __forceinline__ _Float16* ks(int st) const { return lds + st * G::TILE; }
    __device__ __forceinline__ _Float16* vs(int st) const { return lds + (2 + st) * G::TILE; }
    __device__ __forceinline__ float* xch() const {
        return reinterpret_cast<float*>(lds + 4 * G::TILE);
    }

    // Buffer over key rows j0 .. min(j0 + BN, S) - 1 of t (reads past them
    // return zero).  j0 is uniform; readfirstlane keeps the descriptor in
    // scalar registers.
    __device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const _Float16* t, int j0) const {
        j0 = __builtin_amdgcn_readfirstlane(j0);
        return __builtin_amdgcn_make_buffer_rsrc(
            const_cast<_Float16*>(t + base + (size_t)j0 * G::D), (short)0,
            (S > j0 ? min(S - j0, G::BN) : 0) * G::D * 2, 0x00020000);
    }
    // This wave's ROWS rows of key tile j of t (K when isk, else V) into the
    // LDS stage dst, straight from global memory: one 1 KB load instruction
    // per row, lane L landing at byte 16 L of the row and so loading the
    // logical chunk that the row's swizzle puts there.  Inline assembly with
    // M0 = the row's LDS address; the only waits on these loads are the
    // explicit ones before the barriers.
    __device__ __forceinline__ void dma_row(const __amdgpu_buffer_rsrc_t r, _Float16* dst, int u,
                                            bool isk, int ln) const {
        const int row = G::ROWS * w + u;
        const int logical = ln ^ (isk ? swz_k512(row) : swz_v512(row));
        const uint32_t m0 = (uint32_t)(uintptr_t)(LdsPtr)(dst + row * G::D);
        asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
                     :
                     : "v"((row * G::D + 8 * logical) * 2), "s"(r), "{m0}"(m0)
                     : "memory");
    }
    __device__ __forceinline__ void dma(const _Float16* t, _Float16* dst, int j, bool isk) const {
        const auto r = tile_rsrc(t, j * G::BN);
        const int ln = fresh(lane);
#pragma unroll
        for (int u = 0; u < G::ROWS; ++u) dma_row(r, dst, u, isk, ln);
    }
    // This wave's loads and LDS accesses have landed, then the workgroup barrier.
    __device__ __forceinline__ void barrier_dma() const {
        asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
    }
    // The same, with this wave's last ROWS (8 or 16) tile-row loads still in
    // flight (loads complete in issue order).
    __device__ __forceinline__ void barrier_dma_but8() const {
        if constexpr (G::ROWS == 8)
            asm volatile("s_waitcnt vmcnt(8) lgkmcnt(0)" ::: "memory");
        else
            asm volatile("s_waitcnt vmcnt(16) lgkmcnt(0)" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
    }

    // Partial S^T over this wave's 256 head dims (32 keys x 32 queries) from
    // K stage st: 16 matrix instructions in two independent accumulation
    // chains (even and odd 16-dim steps, added at the end), the K fragments
    // (key n, head dims 256 dh + 16 kk + 8g ..) read a group of four ahead.
    // With DMA, this wave's 8 rows of key tile jn of K go to K stage dn, one
    // after every second product, so that the CU's load path is fed evenly
    // while the matrix cores run.
    template <bool DMA>
    __device__ __forceinline__ floatx16 qk_half(const half8* qf, int st, int jn = 0,
                                                int dn = 0) const {
        const _Float16* kp = ks(st) + n * G::D;
        // chunk 32 dh + 2 kk + g = (32 dh + g) | 2 kk (disjoint bits), so the
        // swizzled chunk is x ^ 2 kk with x = (32 dh + g) ^ swizzle
        const int x = fresh((32 * dh + g) ^ swz_k512(n));
        __amdgpu_buffer_rsrc_t r;
        int ln = 0;
        if (DMA) {
            r = tile_rsrc(K, jn * G::BN);
            ln = fresh(lane);
        }
        floatx16 acc[2];
#pragma unroll
        for (int r2 = 0; r2 < 16; ++r2) acc[0][r2] = acc[1][r2] = 0.f;
        half8 kf[2][4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
            kf[0][e] = *reinterpret_cast<const half8*>(kp + 8 * (x ^ (2 * e)));
#pragma unroll
        for (int k4 = 0; k4 < 4; ++k4) {
            if (k4 + 1 < 4) {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    kf[(k4 + 1) & 1][e] = *reinterpret_cast<const half8*>(
                        kp + 8 * (x ^ (2 * (4 * (k4 + 1) + e))));
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                acc[e & 1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(kf[k4 & 1][e], qf[4 * k4 + e],
                                                                    acc[e & 1], 0, 0, 0);
                if constexpr (G::ROWS == 8) {
                    if (DMA && (e & 1)) dma_row(r, ks(dn), 2 * k4 + (e >> 1), true, ln);
                } else {
                    if (DMA) dma_row(r, ks(dn), 4 * k4 + e, true, ln);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        return acc[0] + acc[1];
    }
    // Publish this wave's partial S^T in exchange buffer x; add the partner's
    // (same row group, other head-dim half).  Both waves then hold
    // S_0 + S_1 = S_1 + S_0 bit for bit (fp32 addition commutes).
    __device__ __forceinline__ void publish(float* x, const floatx16& s) const {
        float* mine = x + w * 16 * 64;
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
            *reinterpret_cast<float4*>(mine + (4 * q4) * 64 + 4 * lane) =
                float4{s[4 * q4], s[4 * q4 + 1], s[4 * q4 + 2], s[4 * q4 + 3]};
    }
    __device__ __forceinline__ void add_partner(const float* x, floatx16& s) const {
        const float* other = x + (w ^ G::RG) * 16 * 64;  // (rg, 1 - dh)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            const float4 p = *reinterpret_cast<const float4*>(other + (4 * q4) * 64 + 4 * lane);
            s[4 * q4] += p.x;
            s[4 * q4 + 1] += p.y;
            s[4 * q4 + 2] += p.z;
            s[4 * q4 + 3] += p.w;
        }
    }

    // O^T (this wave's 256 dims) += V^T P^T for the 32-key tile in V stage st.
    template <bool SCHED>
    __device__ __forceinline__ void pv_half(floatx16* o, const half8* pf, int st) const {
        const _Float16* Vs = vs(st);
        const int n16 = n >> 4, jj = n & 15;
        const int sub = (jj & 3) >> 1, half = jj & 1;
        const int sw = swz_v512(jj >> 2);  // (row & 3) == jj >> 2 for every row read
        const _Float16* rowp = Vs + (4 * g + (jj >> 2)) * G::D + 4 * half;
        // chunk 32 dh + 4 b + 2 n16 + sub = (32 dh + 2 n16 + sub) | 4 b
        // (disjoint bits): swizzled, x ^ 4 b
        const int x = fresh((32 * dh + 2 * n16 + sub) ^ sw);
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const _Float16* pb = rowp + 8 * (x ^ (4 * b));
            half8 a[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                half4 part[2];
#pragma unroll
                for (int t = 0; t < 2; ++t)
                    part[t] = __builtin_bit_cast(
                        half4, __builtin_amdgcn_ds_read_tr16_b64_v4f16(
                                   (lds_half4*)(pb + (16 * h + 8 * t) * G::D)));
                a[h] = half8{part[0][0], part[0][1], part[0][2], part[0][3],
                             part[1][0], part[1][1], part[1][2], part[1][3]};
            }
#pragma unroll
            for (int h = 0; h < 2; ++h)
                o[b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[h], pf[h], o[b], 0, 0, 0);
        }
        if (SCHED) {
            // the transposed reads of block b+1 ahead of block b's two products
            __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);  // DS read
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                if (b + 1 < NB) __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
                __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);  // MFMA
            }
        }
    }

    // One V^T fragment pair (keys 0-15 and 16-31 of the tile, head dims
    // 256 dh + 32 b ..) from V stage Vs, for the lane offsets of pv_half.
    __device__ __forceinline__ void read_v(half8* a, const _Float16* rowp, int x, int b) const {
        const _Float16* pb = rowp + 8 * (x ^ (4 * b));
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            half4 part[2];
#pragma unroll
            for (int t = 0; t < 2; ++t)
                part[t] = __builtin_bit_cast(
                    half4, __builtin_amdgcn_ds_read_tr16_b64_v4f16(
                               (lds_half4*)(pb + (16 * h + 8 * t) * G::D)));
            a[h] = half8{part[0][0], part[0][1], part[0][2], part[0][3],
                         part[1][0], part[1][1], part[1][2], part[1][3]};
        }
    }

    // O^T += V^T P_prev^T for the tile in V stage st, interleaved by hand
    // with the online softmax of the next score tile s (the lazy-rescale
    // softmax of softmax_block, same steps and results): block b's two
    // products go out with the transposed reads of block b+2 and the
    // weights of registers 2b and 2b+1, so the vector ALUs work while the
    // matrix cores do.  P of s goes to pn.
    __device__ __forceinline__ void pv_softmax(floatx16* o, const half8* pf, int st, floatx16 s,
                                               int lim, float& m, float& l, half8* pn, int jv,
                                               int dv) const {
        const _Float16* Vs = vs(st);
        const int n16 = n >> 4, jj = n & 15;
        const int sub = (jj & 3) >> 1, half = jj & 1;
        const int sw = swz_v512(jj >> 2);
        const _Float16* rowp = Vs + (4 * g + (jj >> 2)) * G::D + 4 * half;
        const int x = fresh((32 * dh + 2 * n16 + sub) ^ sw);
        const auto rv = tile_rsrc(V, jv * G::BN);
        const int ln = fresh(lane);
        half8 a[3][2];
        read_v(a[0], rowp, x, 0);
        read_v(a[1], rowp, x, 1);
        float q[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            if (b + 2 < NB) read_v(a[(b + 2) % 3], rowp, x, b + 2);
#pragma unroll
            for (int h = 0; h < 2; ++h)
                o[b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[b % 3][h], pf[h], o[b], 0, 0, 0);
            // rows of this wave's share of V tile jv into V stage dv
#pragma unroll
            for (int u = b * G::ROWS / NB; u < (b + 1) * G::ROWS / NB; ++u)
                dma_row(rv, vs(dv), u, false, ln);
#pragma unroll
            for (int r = 2 * b; r < 2 * b + 2; ++r) {
                float t = __builtin_fmaf(s[r], c, -m);
                if ((8 * (r >> 2) + (r & 3)) > lim) t = kNegInf;
                const float e = __builtin_amdgcn_exp2f(t);
                q[r & 3] += e;
                pn[r >> 3][r & 7] = (_Float16)e;
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        float psum = (q[0] + q[1]) + (q[2] + q[3]);
        // every weight is at most the lane's sum; NaN (m = -inf meeting a
        // masked key) takes the branch too
        if (__builtin_amdgcn_ballot_w64(!(psum <= kLazyBound)) != 0) {
#pragma unroll
            for (int r = 0; r < 16; ++r)
                if ((8 * (r >> 2) + (r & 3)) > lim) s[r] = kNegInf;
            const float mx = fmaxf(fmaxf(fmaxf(fmaxf(s[0], s[1]), s[2]), fmaxf(fmaxf(s[3], s[4]), s[5])),
                                   fmaxf(fmaxf(fmaxf(s[6], s[7]), s[8]),
                                         fmaxf(fmaxf(fmaxf(s[9], s[10]), s[11]),
                                               fmaxf(fmaxf(fmaxf(s[12], s[13]), s[14]), s[15]))));
            const float cand = fmaxf(c * max_halves(mx), -kFltMax);
            const float m_new = fmaxf(m, cand);
            const float alpha = __builtin_amdgcn_exp2f(m - m_new);
            m = m_new;
            l *= alpha;
#pragma unroll
            for (int b = 0; b < NB; ++b)
#pragma unroll
                for (int r = 0; r < 16; ++r) o[b][r] *= alpha;
            float q2[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float t = __builtin_fmaf(s[r], c, -m);
                if ((8 * (r >> 2) + (r & 3)) > lim) t = kNegInf;
                const float e = __builtin_amdgcn_exp2f(t);
                q2[r & 3] += e;
                pn[r >> 3][r & 7] = (_Float16)e;
            }
            psum = (q2[0] + q2[1]) + (q2[2] + q2[3]);
        }
        l += psum;
    }

    // Query tile qt over key tiles [kt0, kt1).  part == nullptr: write O and
    // LSE; otherwise leave the partial state in the chunk's workspace slot:
    // O / l as fp16 [64][512], then m[64] (log2 units) and l[64] in fp32.
    //
    // Software pipeline, per key tile i, in two phases with a barrier each:
    //   P: wait for V(i-1) (K(i+1) may still be in flight), barrier;
    //      S(i) = own partial + the partner's;
    //      O += V(i-1)^T P(i-1) on the matrix cores while the vector ALUs
    //      form P(i) = softmax(S(i)), the loads of V(i) (into V(i-2)'s
    //      stage) issued between the products
    //   Q: wait for K(i+1) (V(i) may still be in flight), barrier;
    //      partial S(i+1) = K(i+1) Q^T, the loads of K(i+2) (into K(i)'s
    //      stage) issued between the products; publish the partial
    // and O += V(last)^T P(last) after the loop.  Every tile load has a
    // phase pair to land; the scores of one tile are live at a time.  The
    // exchange buffer is written after barrier Q and read after the next
    // barrier P, always before the writer's next barrier Q: one buffer.
    __device__ void run(int qt, int kt0, int kt1, float* part) {
        const int q0 = qt * G::BM;
        const int row = q0 + 32 * rg + n;
        const int vis = causal ? min(row, S - 1) : S - 1;  // last key this lane's row sees

        // The tile's 64 query rows go through the two V stages (free until
        // the first V tile) as whole 1 KB rows, swizzled like K rows, and
        // this wave's Q^T fragments are read from there.  Loading the
        // fragments straight from global memory (16 bytes per lane across 32
        // rows, four instructions per 128-byte line, 64 KB per workgroup in
        // flight at once) thrashed the vector L1 cache.  Rows past S read
        // zero (their outputs are not stored).
#pragma unroll
        for (int h = 0; h < G::RG; ++h) dma(Q, vs(h), G::RG * qt + h, true);

        float m = kNegInf, l = 0.f;
        floatx16 o[NB];
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) o[b][r] = 0.f;

        const int nt = kt1 - kt0;
        // Tiles whose keys are all in the future of this wave's rows (at most
        // the last one, for the upper row group of a causal tile) go through
        // the same steps: every key masked, P = 0, nothing changes.

        // prologue: K(kt0), K(kt0+1); the partial S(kt0) as soon as Q and
        // K(kt0) are in (K(kt0+1) is waited for at the next barrier)
        dma(K, ks(0), kt0, true);
        if (nt > 1) {
            dma(K, ks(1), kt0 + 1, true);
            barrier_dma_but8();
        } else {
            barrier_dma();
        }
        // Q^T fragment of this wave's rows and head-dim half (rows 32 rg + n
        // of the two stages), the sign of a negative scale applied
        half8 qf[G::DH / 16];
        {
            const _Float16* qp = vs(0) + (32 * rg + n) * G::D;
            const int x = (32 * dh + g) ^ swz_k512(n);
#pragma unroll
            for (int kk = 0; kk < G::DH / 16; ++kk) {
                u32x4 v = *reinterpret_cast<const u32x4*>(qp + 8 * (x ^ (2 * kk)));
                v ^= qsign;
                qf[kk] = __builtin_bit_cast(half8, v);
                // held in accumulation registers, which the matrix
                // instructions read their B operand from directly: the
                // ordinary registers go to O, the scores and the fragments
                asm volatile("" : "+a"(qf[kk]));
            }
        }
        floatx16 s_cur = qk_half<false>(qf, 0);
        publish(xch(), s_cur);

        // tile kt0: no P V yet
        half8 pf[2];
        barrier_dma();
        add_partner(xch(), s_cur);
        dma(V, vs(0), kt0, false);
        softmax_block<true, NB, false>(s_cur, vis - (kt0 * G::BN + 4 * g), c, m, l, o, pf);
        if (nt > 1) {
            barrier_dma_but8();
            s_cur = nt > 2 ? qk_half<true>(qf, 1, kt0 + 2, 0) : qk_half<false>(qf, 1);
            publish(xch(), s_cur);
        }
        for (int li = 1; li < nt; ++li) {
            const int i = kt0 + li;
            const int st = li & 1;
            // phase P
            if (li + 1 < nt)
                barrier_dma_but8();
            else
                barrier_dma();
            add_partner(xch(), s_cur);
            half8 pn[2];
            pv_softmax(o, pf, st ^ 1, s_cur, vis - (i * G::BN + 4 * g), m, l, pn, i, st);
            pf[0] = pn[0];
            pf[1] = pn[1];
            // phase Q
            if (li + 1 < nt) {
                barrier_dma_but8();
                s_cur = li + 2 < nt ? qk_half<true>(qf, st ^ 1, i + 2, st)
                                    : qk_half<false>(qf, st ^ 1);
                publish(xch(), s_cur);
            }
        }
        // the last tile's P V
        barrier_dma();
        pv_half<true>(o, pf, (nt - 1) & 1);

        // Epilogue: both waves of a row group hold the same m and l; each
        // writes its 256 output dims.
        const float lt = sum_halves(l);
        // (partial states: 64-row split-KV units only)
        if (NW == 4 && part) {
            // the chunk's own normalised output O / l in fp16 (|O / l| <=
            // max |V|; 0 where the chunk saw no key of the row), then m, l
            const float pinv = lt > 0.f ? 1.0f / lt : 0.f;
            _Float16* po = reinterpret_cast<_Float16*>(part) + (size_t)(32 * rg + n) * G::D +
                           G::DH * dh;
#pragma unroll
            for (int b = 0; b < NB; ++b)
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                    u32x2 pk;
#pragma unroll
                    for (int h = 0; h < 2; ++h)
                        pk[h] = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)(o[b][4 * q4 + 2 * h] * pinv)) |
                                ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)(o[b][4 * q4 + 2 * h + 1] * pinv)) << 16);
                    *reinterpret_cast<u32x2*>(po + 32 * b + 8 * q4 + 4 * g) = pk;
                }
            float* pml = part + kSlotOFloats;
            if (dh == 0 && g == 0) {
                pml[32 * rg + n] = m;
                pml[G::BM + 32 * rg + n] = lt;
            }
            return;
        }
        const float inv = 1.0f / lt;
        if (row < S) {
            _Float16* orow = O + base + (size_t)row * G::D + G::DH * dh;
#pragma unroll
            for (int b = 0; b < NB; ++b)
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
            if (dh == 0 && g == 0) LSE[lse_base + row] = (m + __builtin_amdgcn_logf(lt)) * kLn2;
        }
    }
};

// Chunking of the key range.  Query tile qt sees nkt(qt) 32-key tiles and is
// cut into nchunks(qt) chunks of at most C tiles.  Work units enumerate
// (query tile, chunk) heaviest tile first; a unit's partial-state slot is
// (bh * U + unit).
struct Chunking {
    int S, T, C, causal;
    __host__ __device__ int nkt(int qt) const {
        const int kv_end = causal ? min(S, (qt + 1) * G512::BM) : S;
        return (kv_end + G512::BN - 1) / G512::BN;
    }
    __host__ __device__ int nchunks(int qt) const { return (nkt(qt) + C - 1) / C; }
    __host__ __device__ long long units() const {
        long long u = 0;
        for (int qt = 0; qt < T; ++qt) u += nchunks(qt);
        return u;
    }
    // unit u -> (query tile, chunk)
    __host__ __device__ void decode(int u, int& qt, int& chunk) const {
        for (qt = T - 1; qt > 0; --qt) {
            const int c = nchunks(qt);
            if (u < c) break;
            u -= c;
        }
        chunk = u;
    }
    __host__ __device__ int first_unit(int qt) const {
        int u = 0;
        for (int q = T - 1; q > qt; --q) u += nchunks(q);
        return u;
    }
};



// NW = 4: one workgroup per (batch, head, 64-row tile, key chunk) of ch.
// NW = 2: one per (batch, head, 32-row tile), all of its keys, heaviest
// tiles first under causal masking (ch, U and ws unused).
template <int NW>
__global__ void __launch_bounds__(64 * NW, 1)
fwd512_kernel(const _Float16* __restrict__ Q, const _Float16* __restrict__ K,
              const _Float16* __restrict__ V, _Float16* __restrict__ O,
              float* __restrict__ LSE, int BH, int S, int causal, float c, uint32_t qsign,
              Chunking ch, int U, float* __restrict__ ws)
{
    using G = G512T<NW>;
    __shared__ __attribute__((aligned(1024))) _Float16 lds[G::LDS_BYTES / 2];

    const int bh = blockIdx.x % BH;
    const int unit = blockIdx.x / BH;
    int qt, kt0 = 0, kt1;
    float* part = nullptr;
    if constexpr (NW == 4) {
        int chunk;
        ch.decode(unit, qt, chunk);
        const int n = ch.nkt(qt);
        kt0 = chunk * ch.C;
        kt1 = min(n, kt0 + ch.C);
        if (ch.nchunks(qt) > 1) part = ws + ((size_t)bh * U + unit) * kSlotFloats;
    } else {
        const int T = (S + G::BM - 1) / G::BM;
        qt = causal ? T - 1 - unit : unit;
        kt1 = ((causal ? min(S, (qt + 1) * G::BM) : S) + G::BN - 1) / G::BN;
    }

    Fwd512<NW> f;
    f.Q = Q;
    f.K = K;
    f.V = V;
    f.O = O;
    f.LSE = LSE;
    f.lds = lds;
    f.S = S;
    f.causal = causal != 0;
    f.base = (size_t)bh * S * G::D;
    f.lse_base = (size_t)bh * S;
    f.c = c;
    f.qsign = qsign;
    f.w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    f.lane = threadIdx.x & 63;
    f.g = f.lane >> 5;
    f.n = f.lane & 31;
    f.rg = f.w % G::RG;
    f.dh = f.w / G::RG;
    f.run(qt, kt0, kt1, part);
}

// Merge the chunks of one query tile's rows in chunk order: with
// m* = max_c m_c and w_c = 2^(m_c - m*), O = sum_c w_c O_c / sum_c w_c l_c and
// LSE = (m* + log2 sum_c w_c l_c) ln 2.  A workgroup takes 8 rows of one query
// tile; 32 threads share a row, each owning 16 consecutive head dims, so the
// partial outputs are read as contiguous 2 KB rows.
constexpr int kMergeRows = 8;

__global__ void __launch_bounds__(256)
merge512_kernel(const float* __restrict__ ws, _Float16* __restrict__ O, float* __restrict__ LSE,
                int BH, int S, Chunking ch, int U, int qt_first)
{
    using G = G512;
    const int per_tile = G::BM / kMergeRows;
    const int bh = blockIdx.x % BH;
    const int rest = blockIdx.x / BH;
    const int qt = qt_first + rest / per_tile, rb = rest % per_tile;
    const int nch = ch.nchunks(qt);
    if (nch <= 1) return;  // written directly by the first kernel
    const float* slot0 = ws + ((size_t)bh * U + ch.first_unit(qt)) * kSlotFloats;
    const int r = rb * kMergeRows + (threadIdx.x >> 5);  // row within the query tile
    const int d0 = 16 * (threadIdx.x & 31);
    const int row = qt * G::BM + r;
    // Chunks in groups of four, every load of a group issued before any is
    // used (the chunk order of the sums unchanged).
    float mt = kNegInf;
    for (int c0 = 0; c0 < nch; c0 += 4) {
        float mv[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
            mv[j] = c0 + j < nch ? slot0[(c0 + j) * kSlotFloats + kSlotOFloats + r] : kNegInf;
#pragma unroll
        for (int j = 0; j < 4; ++j) mt = fmaxf(mt, mv[j]);
    }
    // O = sum_c w_c l_c (O_c / l_c) / sum_c w_c l_c with w_c = 2^(m_c - m*);
    // a chunk that saw no key of this row has l = 0 (and a zero O_c / l_c)
    float lsum = 0.f;
    float4 acc[4] = {};
    for (int c0 = 0; c0 < nch; c0 += 4) {
        float mv[4], lv[4];
        u32x4 xv[4][2];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            // chunks past the last re-read it (unused)
            const float* sl = slot0 + min(c0 + j, nch - 1) * kSlotFloats;
            mv[j] = sl[kSlotOFloats + r];
            lv[j] = sl[kSlotOFloats + G::BM + r];
            const u32x4* x = reinterpret_cast<const u32x4*>(
                reinterpret_cast<const _Float16*>(sl) + (size_t)r * G::D + d0);
            xv[j][0] = x[0];
            xv[j][1] = x[1];
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (c0 + j >= nch) break;
            const float wl = __builtin_amdgcn_exp2f(mv[j] - mt) * lv[j];
            lsum += wl;
#pragma unroll
            for (int e2 = 0; e2 < 2; ++e2) {
                const half8 y = __builtin_bit_cast(half8, xv[j][e2]);
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    float4& a = acc[2 * e2 + e];
                    a.x += wl * (float)y[4 * e];
                    a.y += wl * (float)y[4 * e + 1];
                    a.z += wl * (float)y[4 * e + 2];
                    a.w += wl * (float)y[4 * e + 3];
                }
            }
        }
    }
    if (row >= S) return;
    const float inv = 1.0f / lsum;
    u32x4 pk[2];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        pk[e >> 1][2 * (e & 1)] =
            (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)(acc[e].x * inv)) |
            ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)(acc[e].y * inv)) << 16);
        pk[e >> 1][2 * (e & 1) + 1] =
            (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)(acc[e].z * inv)) |
            ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)(acc[e].w * inv)) << 16);
    }
    u32x4* dst = reinterpret_cast<u32x4*>(O + ((size_t)bh * S + row) * G::D + d0);
    dst[0] = pk[0];
    dst[1] = pk[1];
    if (d0 == 0) LSE[(size_t)bh * S + row] = (mt + __builtin_amdgcn_logf(lsum)) * kLn2;
}

// Fused calls with fewer 64-row tiles than this run on 32-row tiles.
constexpr long long kFew512 = 256;

Chunking make_chunking(int S, int causal, int splits) {
    Chunking ch;
    ch.S = S;
    ch.T = (S + G512::BM - 1) / G512::BM;
    ch.causal = causal;
    const int nmax = (S + G512::BN - 1) / G512::BN;  // key tiles of the longest row
    ch.C = splits <= 0 ? nmax : (nmax + splits - 1) / splits;
    return ch;
}

hipError_t launch(const FwdArgs& a, int splits, float* ws) {
    using G = G512;
    const Chunking ch = make_chunking(a.S, a.causal, splits);
    const int U = (int)ch.units();  // checked to fit by the caller
    const int BH = a.B * a.H;
    const float c = fabsf(a.scale) * 1.44269504088896340736f;
    const uint32_t qsign = a.scale < 0.f ? 0x80008000u : 0u;
    if (splits <= 0 && (long long)BH * ch.T < kFew512) {
        // few 64-row tiles: 32-row tiles of two waves, twice the workgroups
        using G2 = G512T<2>;
        const long long T2 = (a.S + G2::BM - 1) / G2::BM;
        hipLaunchKernelGGL(fwd512_kernel<2>, dim3((unsigned)(T2 * BH)), dim3(G2::NT), 0,
                           (hipStream_t)a.stream,
                           (const _Float16*)a.q, (const _Float16*)a.k, (const _Float16*)a.v,
                           (_Float16*)a.o, a.lse, BH, a.S, a.causal, c, qsign, ch, U, ws);
        return hipGetLastError();
    }
    hipLaunchKernelGGL(fwd512_kernel<4>, dim3((unsigned)((long long)U * BH)), dim3(G::NT), 0,
                       (hipStream_t)a.stream,
                       (const _Float16*)a.q, (const _Float16*)a.k, (const _Float16*)a.v,
                       (_Float16*)a.o, a.lse, BH, a.S, a.causal, c, qsign, ch, U, ws);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || U == ch.T) return e;  // no query tile was split
    // the split tiles are qt_first .. T-1 (a tile's key count grows with qt)
    int qt_first = 0;
    while (ch.nchunks(qt_first) <= 1) ++qt_first;
    const long long merge_blocks = (long long)(ch.T - qt_first) * (G::BM / kMergeRows) * BH;
    hipLaunchKernelGGL(merge512_kernel, dim3((unsigned)merge_blocks), dim3(256), 0,
                       (hipStream_t)a.stream, ws, (_Float16*)a.o, a.lse, BH, a.S, ch, U, qt_first);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fused_d512(const FwdArgs& a) { return launch(a, 0, nullptr); }

size_t splitkv_d512_workspace_floats(int B, int H, int S, int causal, int splits) {
    const Chunking ch = make_chunking(S, causal, splits);
    return (size_t)B * H * ch.units() * kSlotFloats;
}

long long splitkv_d512_units(int S, int causal, int splits) {
    return make_chunking(S, causal, splits).units();
}

hipError_t launch_splitkv_d512(const FwdArgs& a, int splits, void* workspace) {
    return launch(a, splits, (float*)workspace);
}

}  // namespace attn
