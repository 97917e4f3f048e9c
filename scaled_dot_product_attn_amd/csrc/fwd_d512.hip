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
//   * A workgroup (4 waves) owns 64 query rows.  Wave w handles row group
//     rg = w & 1 (32 rows) and head-dim half dh = w >> 1 (256 dims).
//   * Per 32-key tile, wave (rg, dh) computes the partial S^T over its 256
//     dims (16 v_mfma_f32_32x32x16_f16), publishes it in LDS, and adds its
//     partner's (rg, 1-dh) partial: both waves then hold the same
//     S = S_0 + S_1 (fp32 addition is commutative, so they agree bit for bit)
//     and run the same online softmax.
//   * Each wave then accumulates O^T for its own 256 output dims
//     (16 MFMAs), reading V^T with ds_read_b64_tr_b16, like the smaller-D
//     kernel.  Splitting P V along the output dims is what the notes call the
//     pv_n_tile knob; it keeps a wave's output accumulator at 128 registers.
//   * K (padded rows) and V (XOR-swizzled rows) stream through two LDS stages,
//     loaded straight from global memory into LDS (bounds-checked buffer loads
//     with the LDS destination bit, one 1 KB row per instruction, no staging
//     registers).
//
// Split-KV.  Eight heads of 1024 rows give only 128 workgroups for 256 CUs, and
// under causal masking the last query tile does 32 key tiles while the first
// does 2.  The split variant cuts every query tile's key range into chunks of
// at most C 32-key tiles; each chunk is one workgroup that leaves its partial
// state (unnormalised O in fp32, row max m and row sum l) in a workspace, and
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

struct G512 {
    static constexpr int D = 512;
    static constexpr int DH = 256;               // head dims per sub-tile
    static constexpr int NW = 4;
    static constexpr int NT = 64 * NW;
    static constexpr int BM = 64;                // query rows per workgroup
    static constexpr int BN = 32;                // keys per tile
    static constexpr int NS = 2;                 // LDS stages
    static constexpr int CPR = D / 8;            // 16-byte chunks per row
    static constexpr int KSTR = D + 8;           // padded K row (halfs)
    static constexpr int KTILE = BN * KSTR;
    static constexpr int VTILE = BN * D;
    static constexpr int STAGE = KTILE + VTILE;
    static constexpr int XCH = NW * 16 * 64;     // floats of the S^T exchange buffer
    static constexpr int LDS_BYTES = NS * STAGE * 2 + XCH * 4;
    static constexpr int CH = BN * CPR / NT;     // chunks per thread per K (or V) tile
    static_assert(CH * NT == BN * CPR, "tile split");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
};

// V row swizzle: XOR chunk bits 2-3 with the row's low two bits, so that the
// four rows of a transposed read hit different banks.
__device__ __forceinline__ int swz_v512(int r) { return 4 * (r & 3); }

struct Fwd512 {
    using G = G512;
    const _Float16* __restrict__ Q;
    const _Float16* __restrict__ K;
    const _Float16* __restrict__ V;
    _Float16* __restrict__ O;
    float* __restrict__ LSE;
    _Float16* lds;
    float* xch;
    int S;
    bool causal;
    size_t base, lse_base;
    float c;
    uint32_t qsign;
    int tid, w, lane, g, n, rg, dh;
    using LdsPtr = __attribute__((address_space(3))) void*;

    __device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const _Float16* t, int j0) const {
        return __builtin_amdgcn_make_buffer_rsrc(
            const_cast<_Float16*>(t + base + (size_t)j0 * G::D), (short)0,
            min(S - j0, G::BN) * G::D * 2, 0x00020000);
    }
    // Key tile j into LDS stage st, straight from global memory (no staging
    // registers): one 1 KB load instruction per row (a D = 512 row is 1 KB),
    // rows 8w .. 8w+7 of K and of V from this wave.  Lane L lands at byte 16 L
    // of the row: K rows keep their 16-byte pad (M0 = the padded row's
    // address), V rows are swizzled, so lane L loads the logical chunk the
    // swizzle puts at physical chunk L.  Rows past S read as zero.  Inline
    // assembly with M0 = the LDS address, as in the D <= 128 kernel, so the
    // only waits on these loads are the explicit ones before the barriers.
    template <bool DO_K = true, bool DO_V = true>
    __device__ __forceinline__ void dma_tile(int j, int st) const {
        // uniform by construction; readfirstlane keeps it (and so the buffer
        // descriptors) in scalar registers where the loop counter lives in a
        // vector register
        const int j0 = __builtin_amdgcn_readfirstlane(j * G::BN);
        const auto rk = tile_rsrc(K, j0), rv = tile_rsrc(V, j0);
        _Float16* Ks = lds + st * G::STAGE;
        _Float16* Vs = Ks + G::KTILE;
#pragma unroll
        for (int u = 0; u < G::BN / G::NW; ++u) {
            const int row = (G::BN / G::NW) * w + u;
            const uint32_t mk = (uint32_t)(uintptr_t)(LdsPtr)(Ks + row * G::KSTR);
            if (DO_K) asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
                         :
                         : "v"((row * G::D + 8 * lane) * 2), "s"(rk), "{m0}"(mk)
                         : "memory");
            const uint32_t mv = (uint32_t)(uintptr_t)(LdsPtr)(Vs + row * G::D);
            if (DO_V) asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
                         :
                         : "v"((row * G::D + 8 * (lane ^ swz_v512(row))) * 2), "s"(rv), "{m0}"(mv)
                         : "memory");
        }
    }
    // This wave's tile loads have landed, then the workgroup barrier.
    __device__ __forceinline__ void barrier_dma() const {
        asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
    }

    // Partial S^T over this wave's 256 head dims: 32 keys x 32 queries.
    __device__ __forceinline__ floatx16 qk_half(const half8* qf, int st) const {
        const _Float16* kp = lds + st * G::STAGE + n * G::KSTR + G::DH * dh + 8 * g;
        floatx16 acc;
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
        for (int k4 = 0; k4 < 4; ++k4) {
            half8 kf[4];
#pragma unroll
            for (int e = 0; e < 4; ++e)
                kf[e] = *reinterpret_cast<const half8*>(kp + 16 * (4 * k4 + e));
#pragma unroll
            for (int e = 0; e < 4; ++e)
                acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(kf[e], qf[4 * k4 + e], acc, 0, 0, 0);
        }
        return acc;
    }

    // O^T (this wave's 256 dims) += V^T P^T for the 32-key tile in stage st.
    __device__ __forceinline__ void pv_half(floatx16* o, const half8* pf, int st) const {
        const _Float16* Vs = lds + st * G::STAGE + G::KTILE;
        const int n16 = n >> 4, jj = n & 15;
        const int sub = (jj & 3) >> 1, half = jj & 1;
        const int sw = swz_v512(jj >> 2);  // (row & 3) == jj >> 2 for every row read
        const _Float16* rowp = Vs + (4 * g + (jj >> 2)) * G::D + 4 * half;
#pragma unroll
        for (int b = 0; b < G::DH / 32; ++b) {
            const _Float16* pb = rowp + 8 * ((32 * dh + 4 * b + 2 * n16 + sub) ^ sw);
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
    }

    // Query tile qt over key tiles [kt0, kt1).  part == nullptr: write O and
    // LSE; otherwise leave the partial state in the chunk's workspace slot:
    // unnormalised O as fp32 [64][512], then m[64] (log2 units) and l[64].
    __device__ void run(int qt, int kt0, int kt1, float* part) {
        const int q0 = qt * G::BM;
        const int row = q0 + 32 * rg + n;
        const int r_lo = q0 + 32 * rg, r_hi = r_lo + 31;

        // Q^T fragment of this wave's rows and head-dim half.
        half8 qf[G::DH / 16];
        {
            const u32x4* src = reinterpret_cast<const u32x4*>(
                Q + base + (size_t)min(row, S - 1) * G::D + G::DH * dh);
#pragma unroll
            for (int kk = 0; kk < G::DH / 16; ++kk) {
                u32x4 x = src[2 * kk + g];
                x ^= qsign;
                qf[kk] = __builtin_bit_cast(half8, x);
            }
        }

        float m = kNegInf, l = 0.f;
        floatx16 o[G::DH / 32];
#pragma unroll
        for (int b = 0; b < G::DH / 32; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) o[b][r] = 0.f;

        dma_tile(kt0, 0);
        barrier_dma();
        float* mine = xch + w * 16 * 64;
        const float* other = xch + (w ^ 2) * 16 * 64;  // same row group, other half
        for (int i = kt0; i < kt1; ++i) {
            const int li = i - kt0;  // LDS stage of tile i: li & 1
            const int j0 = i * G::BN;
            // the next tile goes into the stage of tile i-1, which every wave
            // finished before the last barrier
            if (i + 1 < kt1) dma_tile<true, false>(i + 1, (li + 1) & 1);
            const bool skip = causal && j0 > r_hi;  // every key is in this wave's future
            floatx16 s;
            if (!skip) {
                s = qk_half(qf, li & 1);
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4)
                    *reinterpret_cast<float4*>(mine + (4 * q4) * 64 + 4 * lane) =
                        float4{s[4 * q4], s[4 * q4 + 1], s[4 * q4 + 2], s[4 * q4 + 3]};
            }
            barrier();  // both sub-tile partials are published
            if (i + 1 < kt1) dma_tile<false, true>(i + 1, (li + 1) & 1);
            if (!skip) {
                // S = S_0 + S_1 in logit space (the same sum in both waves)
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                    const float4 p = *reinterpret_cast<const float4*>(other + (4 * q4) * 64 + 4 * lane);
                    s[4 * q4] += p.x;
                    s[4 * q4 + 1] += p.y;
                    s[4 * q4 + 2] += p.z;
                    s[4 * q4 + 3] += p.w;
                }
                half8 pf[2];
                const int lim = (causal ? min(row, S - 1) : S - 1) - (j0 + 4 * g);
                const bool need_mask = (causal && j0 + G::BN - 1 > r_lo) || (j0 + G::BN > S);
                if (need_mask)
                    online_softmax<true, G::DH / 32>(s, lim, c, m, l, o, pf);
                else
                    online_softmax<false, G::DH / 32>(s, lim, c, m, l, o, pf);
                pv_half(o, pf, li & 1);
            }
            barrier_dma();  // next tile in LDS; exchange buffer free again
        }

        // Epilogue: both waves of a row group hold the same m and l; each
        // writes its 256 output dims.
        const float lt = sum_halves(l);
        if (part) {
            float* po = part + (size_t)(32 * rg + n) * G::D + G::DH * dh;
#pragma unroll
            for (int b = 0; b < G::DH / 32; ++b)
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4)
                    *reinterpret_cast<float4*>(po + 32 * b + 8 * q4 + 4 * g) =
                        float4{o[b][4 * q4], o[b][4 * q4 + 1], o[b][4 * q4 + 2], o[b][4 * q4 + 3]};
            if (dh == 0 && g == 0) {
                part[G::BM * G::D + 32 * rg + n] = m;
                part[G::BM * G::D + G::BM + 32 * rg + n] = lt;
            }
            return;
        }
        const float inv = 1.0f / lt;
        if (row < S) {
            _Float16* orow = O + base + (size_t)row * G::D + G::DH * dh;
#pragma unroll
            for (int b = 0; b < G::DH / 32; ++b)
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

constexpr size_t kSlotFloats = (size_t)G512::BM * G512::D + 2 * G512::BM;

__global__ void __launch_bounds__(256, 1)
fwd512_kernel(const _Float16* __restrict__ Q, const _Float16* __restrict__ K,
              const _Float16* __restrict__ V, _Float16* __restrict__ O,
              float* __restrict__ LSE, int BH, int S, int causal, float c, uint32_t qsign,
              Chunking ch, int U, float* __restrict__ ws)
{
    using G = G512;
    __shared__ __attribute__((aligned(1024))) _Float16 lds[G::NS * G::STAGE + 2 * G::XCH];

    const int bh = blockIdx.x % BH;
    const int unit = blockIdx.x / BH;
    int qt, chunk;
    ch.decode(unit, qt, chunk);
    const int n = ch.nkt(qt);
    const int kt0 = chunk * ch.C, kt1 = min(n, kt0 + ch.C);
    float* part = ch.nchunks(qt) > 1 ? ws + ((size_t)bh * U + unit) * kSlotFloats : nullptr;

    Fwd512 f;
    f.Q = Q;
    f.K = K;
    f.V = V;
    f.O = O;
    f.LSE = LSE;
    f.lds = lds;
    f.xch = reinterpret_cast<float*>(lds + G::NS * G::STAGE);
    f.S = S;
    f.causal = causal != 0;
    f.base = (size_t)bh * S * G::D;
    f.lse_base = (size_t)bh * S;
    f.c = c;
    f.qsign = qsign;
    f.tid = threadIdx.x;
    f.w = threadIdx.x >> 6;
    f.lane = threadIdx.x & 63;
    f.g = f.lane >> 5;
    f.n = f.lane & 31;
    f.rg = f.w & 1;
    f.dh = f.w >> 1;
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
                int BH, int S, Chunking ch, int U)
{
    using G = G512;
    const int per_tile = G::BM / kMergeRows;
    const int bh = blockIdx.x % BH;
    const int rest = blockIdx.x / BH;
    const int qt = rest / per_tile, rb = rest % per_tile;
    const int nch = ch.nchunks(qt);
    if (nch <= 1) return;  // written directly by the first kernel
    const float* slot0 = ws + ((size_t)bh * U + ch.first_unit(qt)) * kSlotFloats;
    const int r = rb * kMergeRows + (threadIdx.x >> 5);  // row within the query tile
    const int d0 = 16 * (threadIdx.x & 31);
    const int row = qt * G::BM + r;
    float mt = kNegInf;
    for (int cc = 0; cc < nch; ++cc) mt = fmaxf(mt, slot0[cc * kSlotFloats + G::BM * G::D + r]);
    float lsum = 0.f;
    float4 acc[4] = {};
    for (int cc = 0; cc < nch; ++cc) {
        const float* sl = slot0 + cc * kSlotFloats;
        // a chunk that saw no key of this row has l = 0 and zero O
        const float wgt = __builtin_amdgcn_exp2f(sl[G::BM * G::D + r] - mt);
        lsum += wgt * sl[G::BM * G::D + G::BM + r];
        const float4* x = reinterpret_cast<const float4*>(sl + (size_t)r * G::D + d0);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float4 y = x[e];
            acc[e].x += wgt * y.x;
            acc[e].y += wgt * y.y;
            acc[e].z += wgt * y.z;
            acc[e].w += wgt * y.w;
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
    hipLaunchKernelGGL(fwd512_kernel, dim3((unsigned)((long long)U * BH)), dim3(G::NT), 0,
                       (hipStream_t)a.stream,
                       (const _Float16*)a.q, (const _Float16*)a.k, (const _Float16*)a.v,
                       (_Float16*)a.o, a.lse, BH, a.S, a.causal, c, qsign, ch, U, ws);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || U == ch.T) return e;  // no query tile was split
    const long long merge_blocks = (long long)ch.T * (G::BM / kMergeRows) * BH;
    hipLaunchKernelGGL(merge512_kernel, dim3((unsigned)merge_blocks), dim3(256), 0,
                       (hipStream_t)a.stream, ws, (_Float16*)a.o, a.lse, BH, a.S, ch, U);
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
