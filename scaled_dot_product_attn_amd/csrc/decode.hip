// Attention forward with Sq query rows against Sk keys (decode: a few queries
// against a long key/value cache), D in {64, 128}, for gfx950.
//
//   O = softmax(scale * Q K^T + mask) V,   LSE = log sum_j exp(scale q.k_j)
//
// q, o: fp16 [B, H, Sq, D]; k, v: fp16 [B, H, Sk, D]; lse: fp32 [B, H, Sq].
// Causal masking is aligned bottom-right: query i sits at position
// i + Sk - Sq of the sequence, so key j is visible iff j <= i + Sk - Sq (the
// pages' decode kernel, "Validating Memory-Optimal Transformer Kernels on
// Real Hardware", section 5, fixes no alignment; this is the one a cache of
// past keys implies).
//
// With Sq small the work lies along the keys, so the key range of every
// 64-row query tile is cut into chunks of at most C 64-key tiles, one
// workgroup per (batch, head, query tile, chunk).  A chunk leaves its partial
// state (unnormalised O in fp32, row max m and row sum l) in a workspace and a
// second kernel merges the chunks of each row in chunk order; the merge over
// DISJOINT key sets is exact up to rounding (STAGE_D.md notes, section
// "2. External k_sub Merge is Mathematically Impossible": outputs over
// different token sets combine through their weights).  A query tile with a
// single chunk is written directly.
//
// Inside a workgroup (4 waves, two workgroups per CU): wave w takes query rows
// 32(w&1) .. +31 of the tile against keys 32(w>>1) .. +31 of every 64-key
// tile, and the two key halves are merged in LDS at the end, as in the square
// kernel.  S^T = K Q^T and O^T += V^T P^T on v_mfma_f32_32x32x16_f16 with the
// same lane layouts:
//   A[m][k]: lane holds m = n, k = 8g .. 8g+7
//   B[k][n]: lane holds n = n, k = 8g .. 8g+7
//   C[m][n]: register r holds m = 8(r/4) + 4g + r%4, n = n
// (g = lane / 32, n = lane % 32).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "attn.h"

#include "fwd_common.h"
#include "kernels.h"

namespace attn {
namespace {

using namespace detail;

template <int D>
struct GeoD {
    static constexpr int NW = 4;                 // waves per workgroup
    static constexpr int NT = 64 * NW;           // threads
    static constexpr int BM = 64;                // query rows per tile
    static constexpr int BN = 64;                // keys per tile
    static constexpr int CPR = D / 8;            // 16-byte chunks per row
    static constexpr int KSTR = D + 8;           // K row stride in halfs (16 B pad)
    static constexpr int KTILE = BN * KSTR;
    static constexpr int VTILE = BN * D;         // swizzled, no pad
    static constexpr int STAGE = KTILE + VTILE;
    static constexpr int LDS_HALFS = 2 * STAGE;  // two stages
    static constexpr int CH = BN * CPR / NT;     // 16-byte chunks per thread per K (or V) tile
    static constexpr size_t SLOT = (size_t)BM * D + 2 * BM;  // floats of a partial state
    static_assert(D == 64 || D == 128, "D");
    static_assert(CH * NT == BN * CPR, "tile split");
    static_assert(LDS_HALFS * 2 * 2 <= 160 * 1024, "LDS budget for two workgroups per CU");
    static_assert((D * 64 + 256) * 4 <= LDS_HALFS * 2, "merge buffer fits");
};

template <int D>
__device__ __forceinline__ int swz_vd(int r) {
    return D == 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1);
}

// Query tiles, their key ranges and the chunking of those ranges.  Work
// units enumerate (query tile, chunk) heaviest tile first; a unit's
// partial-state slot is bh * U + unit.
struct KvChunking {
    int Sq, Sk, Tq, C, causal;
    // keys visible to some row of query tile qt: [0, kv_end)
    __host__ __device__ int kv_end(int qt) const {
        if (!causal) return Sk;
        const int last_row = min(Sq, (qt + 1) * 64) - 1;
        return min(Sk, last_row + (Sk - Sq) + 1);
    }
    __host__ __device__ int nkt(int qt) const { return (kv_end(qt) + 63) / 64; }
    __host__ __device__ int nchunks(int qt) const { return (nkt(qt) + C - 1) / C; }
    __host__ __device__ long long units() const {
        long long u = 0;
        for (int qt = 0; qt < Tq; ++qt) u += nchunks(qt);
        return u;
    }
    __host__ __device__ void decode(int u, int& qt, int& chunk) const {
        for (qt = Tq - 1; qt > 0; --qt) {
            const int c = nchunks(qt);
            if (u < c) break;
            u -= c;
        }
        chunk = u;
    }
    __host__ __device__ int first_unit(int qt) const {
        int u = 0;
        for (int q = Tq - 1; q > qt; --q) u += nchunks(q);
        return u;
    }
};

template <int D, bool CAUSAL>
struct Dec {
    using G = GeoD<D>;
    static constexpr int NB = D / 32;

    const _Float16* __restrict__ Q;
    const _Float16* __restrict__ K;
    const _Float16* __restrict__ V;
    _Float16* __restrict__ O;
    float* __restrict__ LSE;
    _Float16* lds;
    int Sq, Sk;
    size_t qbase, kbase, lse_base;
    float c;
    uint32_t qsign;
    int tid, lane, g, n, rg, kh;

    u32x4 kreg[G::CH];
    u32x4 vreg[G::CH];

    __device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const _Float16* t, int j0) const {
        return __builtin_amdgcn_make_buffer_rsrc(
            const_cast<_Float16*>(t + kbase + (size_t)j0 * D), (short)0,
            min(Sk - j0, G::BN) * D * 2, 0x00020000);
    }
    __device__ __forceinline__ void load_tile(int j) {
        const int j0 = j * G::BN;
        const auto rk = rows_rsrc(K, j0), rv = rows_rsrc(V, j0);
#pragma unroll
        for (int u = 0; u < G::CH; ++u) {
            const int ci = tid + G::NT * u;
            kreg[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rk, 16 * ci, 0, 0));
            vreg[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rv, 16 * ci, 0, 0));
        }
    }
    __device__ __forceinline__ void store_tile(int st) {
        _Float16* Ks = lds + st * G::STAGE;
        _Float16* Vs = Ks + G::KTILE;
#pragma unroll
        for (int u = 0; u < G::CH; ++u) {
            const int ci = tid + G::NT * u;
            const int row = ci / G::CPR, cc = ci % G::CPR;
            *reinterpret_cast<u32x4*>(Ks + row * G::KSTR + 8 * cc) = kreg[u];
            *reinterpret_cast<u32x4*>(Vs + row * D + 8 * (cc ^ swz_vd<D>(row))) = vreg[u];
        }
    }

    // One 64-key tile j in stage st: this wave's S^T over keys 32kh .. +31,
    // online softmax, O^T += V^T P^T.  row: the query this lane owns; vis:
    // the last key it may see.
    template <bool MASK>
    __device__ __forceinline__ void tile(int st, int j, int vis, const half8* qf, float& m,
                                         float& l, floatx16* o) const {
        const _Float16* Ks = lds + st * G::STAGE;
        const _Float16* Vs = Ks + G::KTILE;
        half8 kf[D / 16];
        const _Float16* kp = Ks + (32 * kh + n) * G::KSTR + 8 * g;
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) kf[kk] = *reinterpret_cast<const half8*>(kp + 16 * kk);
        // V^T fragments: vf[h][b] covers keys 32kh + 16h .. +15, head dims
        // 32b .. +31; in each 16-lane group lane 4r + c addresses row r,
        // columns 4c .. 4c+3 of a transposed read, so two reads deliver the
        // accumulator's key order 8(r/4) + 4g + r%4.
        half8 vf[2][NB];
        {
            const int n16 = n >> 4, jj = n & 15;
            const int sub = (jj & 3) >> 1, half = (jj & 1);
            const int sw = swz_vd<D>(jj >> 2);
            const _Float16* rowp = Vs + (32 * kh + 4 * g + (jj >> 2)) * D + 4 * half;
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
        floatx16 s;
#pragma unroll
        for (int r = 0; r < 16; ++r) s[r] = 0.f;
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk)
            s = __builtin_amdgcn_mfma_f32_32x32x16_f16(kf[kk], qf[kk], s, 0, 0, 0);
        half8 pf[2];
        const int lim = vis - (j * G::BN + 32 * kh + 4 * g);
        online_softmax<MASK, NB>(s, lim, c, m, l, o, pf);
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int b = 0; b < NB; ++b)
                o[b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf[h][b], pf[h], o[b], 0, 0, 0);
    }

    template <bool MASK>
    __device__ __forceinline__ void step(int& st, int i, int kt1, int vis, const half8* qf,
                                         float& m, float& l, floatx16* o) {
        barrier();  // tile i is in LDS; every wave is done with tile i-1
        const bool more = i + 1 < kt1;
        if (more) load_tile(i + 1);
        tile<MASK>(st, i, vis, qf, m, l, o);
        if (more) store_tile(st ^ 1);
        st ^= 1;
    }

    // Query tile qt over key tiles [kt0, kt1).  part == nullptr: write O and
    // LSE; otherwise the partial state: unnormalised O fp32 [64][D], then
    // m [64] (log2 units) and l [64].
    __device__ void run(int qt, int kt0, int kt1, float* part) {
        const int q0 = qt * G::BM;
        const int row = q0 + 32 * rg + n;
        const int off = Sk - Sq;
        // last visible key of this lane's row, and of the wave's first row
        const int vis = CAUSAL ? min(min(row, Sq - 1) + off, Sk - 1) : Sk - 1;
        const int vis_lo = CAUSAL ? min(q0 + 32 * rg + off, Sk - 1) : Sk - 1;

        load_tile(kt0);
        half8 qf[D / 16];
        {
            const u32x4* src = reinterpret_cast<const u32x4*>(Q + qbase + (size_t)min(row, Sq - 1) * D);
#pragma unroll
            for (int kk = 0; kk < D / 16; ++kk) {
                u32x4 x = src[2 * kk + g];
                x ^= qsign;
                qf[kk] = __builtin_bit_cast(half8, x);
            }
        }
        store_tile(0);

        float m = kNegInf, l = 0.f;
        floatx16 o[NB];
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) o[b][r] = 0.f;

        // tiles whose every key is visible to every row of this wave run
        // unmasked; the rest (the causal band and the ragged end) masked
        int st = 0, i = kt0;
        for (; i < kt1 && (i + 1) * G::BN - 1 <= vis_lo; ++i) step<false>(st, i, kt1, vis, qf, m, l, o);
        for (; i < kt1; ++i) step<true>(st, i, kt1, vis, qf, m, l, o);

        // merge the two key halves: kh = 1 publishes, kh = 0 combines
        barrier();
        float4* mo = reinterpret_cast<float4*>(lds) + rg * (D / 8) * 64;
        float* mm = reinterpret_cast<float*>(lds) + 2 * (D / 2) * 64 + rg * 128;
        if (kh == 1) {
#pragma unroll
            for (int b = 0; b < NB; ++b)
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4)
                    mo[(4 * b + q4) * 64 + lane] =
                        float4{o[b][4 * q4], o[b][4 * q4 + 1], o[b][4 * q4 + 2], o[b][4 * q4 + 3]};
            mm[lane] = m;
            mm[64 + lane] = l;
        }
        barrier();
        if (kh != 0) return;
        const float m1 = mm[lane], l1 = mm[64 + lane];
        const float mt = fmaxf(m, m1);
        // both halves may have seen no key of this row inside a chunk
        const float a0 = mt == kNegInf ? 0.f : __builtin_amdgcn_exp2f(m - mt);
        const float a1 = mt == kNegInf ? 0.f : __builtin_amdgcn_exp2f(m1 - mt);
        const float lt = sum_halves(l * a0 + l1 * a1);
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const float4 p1 = mo[(4 * b + q4) * 64 + lane];
                o[b][4 * q4] = o[b][4 * q4] * a0 + p1.x * a1;
                o[b][4 * q4 + 1] = o[b][4 * q4 + 1] * a0 + p1.y * a1;
                o[b][4 * q4 + 2] = o[b][4 * q4 + 2] * a0 + p1.z * a1;
                o[b][4 * q4 + 3] = o[b][4 * q4 + 3] * a0 + p1.w * a1;
            }
        if (part) {
            float* po = part + (size_t)(32 * rg + n) * D;
#pragma unroll
            for (int b = 0; b < NB; ++b)
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4)
                    *reinterpret_cast<float4*>(po + 32 * b + 8 * q4 + 4 * g) =
                        float4{o[b][4 * q4], o[b][4 * q4 + 1], o[b][4 * q4 + 2], o[b][4 * q4 + 3]};
            if (g == 0) {
                part[G::BM * D + 32 * rg + n] = mt;
                part[G::BM * D + G::BM + 32 * rg + n] = lt;
            }
            return;
        }
        if (row >= Sq) return;
        const float inv = 1.0f / lt;
        _Float16* orow = O + qbase + (size_t)row * D;
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                u32x2 pk;
                pk[0] = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)(o[b][4 * q4] * inv)) |
                        ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)(o[b][4 * q4 + 1] * inv)) << 16);
                pk[1] = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)(o[b][4 * q4 + 2] * inv)) |
                        ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)(o[b][4 * q4 + 3] * inv)) << 16);
                *reinterpret_cast<u32x2*>(orow + 32 * b + 8 * q4 + 4 * g) = pk;
            }
        if (g == 0) LSE[lse_base + row] = (mt + __builtin_amdgcn_logf(lt)) * kLn2;
    }
};

template <int D, bool CAUSAL>
__global__ void __launch_bounds__(256, 2)
dec_kernel(const _Float16* __restrict__ Q, const _Float16* __restrict__ K,
           const _Float16* __restrict__ V, _Float16* __restrict__ O, float* __restrict__ LSE,
           int BH, float c, uint32_t qsign, KvChunking ch, int U, float* __restrict__ ws)
{
    using G = GeoD<D>;
    __shared__ __attribute__((aligned(1024))) _Float16 lds[G::LDS_HALFS];
    const int bh = blockIdx.x % BH;
    const int unit = blockIdx.x / BH;
    int qt, chunk;
    ch.decode(unit, qt, chunk);
    const int kt0 = chunk * ch.C, kt1 = min(ch.nkt(qt), kt0 + ch.C);
    float* part = ch.nchunks(qt) > 1 ? ws + ((size_t)bh * U + unit) * G::SLOT : nullptr;

    Dec<D, CAUSAL> f;
    f.Q = Q;
    f.K = K;
    f.V = V;
    f.O = O;
    f.LSE = LSE;
    f.lds = lds;
    f.Sq = ch.Sq;
    f.Sk = ch.Sk;
    f.qbase = (size_t)bh * ch.Sq * D;
    f.kbase = (size_t)bh * ch.Sk * D;
    f.lse_base = (size_t)bh * ch.Sq;
    f.c = c;
    f.qsign = qsign;
    f.tid = threadIdx.x;
    f.lane = threadIdx.x & 63;
    f.g = f.lane >> 5;
    f.n = f.lane & 31;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    f.rg = w & 1;
    f.kh = w >> 1;
    f.run(qt, kt0, kt1, part);
}

// Merge the chunks of a query tile's rows in chunk order: with m* = max_c m_c
// and w_c = 2^(m_c - m*), O = sum_c w_c O_c / sum_c w_c l_c and
// LSE = (m* + log2 sum_c w_c l_c) ln 2.  A workgroup takes 8 rows; 32 threads
// share a row, each owning D/32 consecutive head dims.
template <int D>
__global__ void __launch_bounds__(256)
dec_merge_kernel(const float* __restrict__ ws, _Float16* __restrict__ O, float* __restrict__ LSE,
                 int BH, KvChunking ch, int U)
{
    using G = GeoD<D>;
    constexpr int DPT = D / 32;  // dims per thread: 4 or 2
    const int per_tile = G::BM / 8;
    const int bh = blockIdx.x % BH;
    const int rest = blockIdx.x / BH;
    const int qt = rest / per_tile, rb = rest % per_tile;
    const int nch = ch.nchunks(qt);
    if (nch <= 1) return;
    const int r = rb * 8 + (threadIdx.x >> 5);
    const int d0 = DPT * (threadIdx.x & 31);
    const int row = qt * G::BM + r;
    // rows past Sq have no output (with a few query rows most of a tile)
    if (row >= ch.Sq) return;
    const float* slot0 = ws + ((size_t)bh * U + ch.first_unit(qt)) * G::SLOT;
    // the chunks' loads are independent: batch them so that their latencies
    // overlap instead of adding up
    float mt = kNegInf;
#pragma unroll 8
    for (int cc = 0; cc < nch; ++cc) mt = fmaxf(mt, slot0[cc * G::SLOT + G::BM * D + r]);
    float lsum = 0.f;
    float acc[DPT] = {};
#pragma unroll 4
    for (int cc = 0; cc < nch; ++cc) {
        const float* sl = slot0 + cc * G::SLOT;
        const float mc = sl[G::BM * D + r];
        // a chunk that saw no key of this row carries m = -inf and l = 0
        const float wgt = mc == kNegInf ? 0.f : __builtin_amdgcn_exp2f(mc - mt);
        lsum += wgt * sl[G::BM * D + G::BM + r];
#pragma unroll
        for (int e = 0; e < DPT; ++e) acc[e] += wgt * sl[(size_t)r * D + d0 + e];
    }
    const float inv = 1.0f / lsum;
    _Float16* orow = O + ((size_t)bh * ch.Sq + row) * D + d0;
#pragma unroll
    for (int e = 0; e < DPT; ++e) orow[e] = (_Float16)(acc[e] * inv);
    if (d0 == 0) LSE[(size_t)bh * ch.Sq + row] = (mt + __builtin_amdgcn_logf(lsum)) * kLn2;
}

KvChunking make_kv_chunking(int Sq, int Sk, int causal, int splits) {
    KvChunking ch;
    ch.Sq = Sq;
    ch.Sk = Sk;
    ch.Tq = (Sq + 63) / 64;
    ch.causal = causal;
    const int nmax = (Sk + 63) / 64;
    ch.C = (nmax + splits - 1) / splits;
    return ch;
}

template <int D, bool CAUSAL>
hipError_t launch_dec(const DecArgs& a) {
    using G = GeoD<D>;
    const KvChunking ch = make_kv_chunking(a.Sq, a.Sk, a.causal, a.splits);
    const int U = (int)ch.units();  // checked to fit by the caller
    const int BH = a.B * a.H;
    const float c = fabsf(a.scale) * 1.44269504088896340736f;
    const uint32_t qsign = a.scale < 0.f ? 0x80008000u : 0u;
    hipLaunchKernelGGL((dec_kernel<D, CAUSAL>), dim3((unsigned)((long long)U * BH)), dim3(G::NT), 0,
                       (hipStream_t)a.stream, (const _Float16*)a.q, (const _Float16*)a.k,
                       (const _Float16*)a.v, (_Float16*)a.o, a.lse, BH, c, qsign, ch, U,
                       (float*)a.workspace);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || U == ch.Tq) return e;
    hipLaunchKernelGGL((dec_merge_kernel<D>), dim3((unsigned)((long long)ch.Tq * 8 * BH)), dim3(256),
                       0, (hipStream_t)a.stream, (const float*)a.workspace, (_Float16*)a.o, a.lse,
                       BH, ch, U);
    return hipGetLastError();
}

}  // namespace

long long decode_units(int Sq, int Sk, int causal, int splits) {
    return make_kv_chunking(Sq, Sk, causal, splits).units();
}

size_t decode_workspace_floats(int B, int H, int Sq, int Sk, int D, int causal, int splits) {
    const KvChunking ch = make_kv_chunking(Sq, Sk, causal, splits);
    if (ch.units() == ch.Tq) return 0;  // no query tile is split
    return (size_t)B * H * ch.units() * ((size_t)64 * D + 128);
}

// The workspace of attn_fwd_decode_noalloc: a static device array, so that a
// caller that cannot allocate (code under HIP graph capture, a tight serving
// loop) still gets the split-key path.  Each GPU the library runs on holds its
// own copy until the process ends.  Every call on a GPU shares it and every
// call writes each slot it later reads, so nothing needs clearing; calls that
// overlap on one GPU (different streams, no ordering) race on it.
static __device__ __align__(256) float scratch[ATTN_DECODE_NOALLOC_SCRATCH_BYTES / sizeof(float)];

hipError_t decode_scratch(void** ptr) {
    // In host code `scratch` names a host-side stand-in, not device memory:
    // the address kernels may use comes from hipGetSymbolAddress, once per
    // device with that device current, kept per device.
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void* addr[kMaxDevices] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        addr[dev] = p;
    }
    *ptr = addr[dev];
    return hipSuccess;
}

hipError_t launch_decode(const DecArgs& a) {
    if (a.D == 64) return a.causal ? launch_dec<64, true>(a) : launch_dec<64, false>(a);
    return a.causal ? launch_dec<128, true>(a) : launch_dec<128, false>(a);
}

}  // namespace attn
