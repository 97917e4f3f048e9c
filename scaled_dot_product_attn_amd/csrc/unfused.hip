// Unfused three-kernel attention forward, kept as an ablation of the fused
// kernels: the same result, but with the n x n intermediates written to and
// read back from global memory.  It is the three-branch pipeline
// QK -> softmax -> AV with globally addressed workspaces that "An Optimal
// Mapper Meets a Real GPU" contrasts with a single fused kernel holding the
// scores in registers (sections "Ground rules" and "The uncomfortable
// audit"); for D = 512 the Q K^T kernel runs once per 256-wide head-dim half,
// the second pass adding into S (option 2 of the STAGE_D.md notes).
//
// One decision apart from the fused path: the same MFMA tiles and the same
// transposed LDS reads of V, only the place where S and P live differs.
//
//   qk_kernel      S[b,h,i,j] = scale * q_i . k_j           (fp32, row stride Sp)
//   softmax_reg_kernel (rows up to 4096 entries; softmax_kernel beyond)
//                  P[b,h,i,j] = exp(S - max) / sum  (fp16),  LSE = max + log(sum)
//   pv_stream_kernel (D = 64, 128; pv_kernel at D = 512)
//                  O = P V                                  (fp16 out)
//
// Workspace: S (fp32) then P (fp16), both [B, H, S, Sp] with Sp = S rounded up
// to 64, so every row starts 128-byte aligned.  Under causal masking only the
// entries a later kernel reads are produced: S for j <= i, P up to the next
// multiple of 128 keys (zeros past the diagonal).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fwd_common.h"
#include "kernels.h"

namespace attn {
namespace {

using namespace detail;

constexpr float kLog2e = 1.44269504088896340736f;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}

// ---------------------------------------------------------------- Q K^T

// One workgroup per (batch, head, 64-row query tile, chunk of up to kQkChunk
// 64-key tiles), the heaviest query tiles first under causal masking, walking
// the key tiles of its chunk that the tile's rows see.  Wave
// (wq, wk): query rows 32wq .. +31 against keys 32wk .. +31 of every key
// tile.  The query rows and then each key tile come in as whole rows (each
// thread a run of contiguous 16-byte chunks, bounds-checked), go through an
// XOR-swizzled LDS tile and are read back as MFMA fragments: loading the
// fragments straight from global memory, 16 bytes per lane across 32 rows,
// requested every 128-byte line four times and ran ~15% slower.  The Q
// fragments stay in registers; the next two key tiles' loads are in flight
// while the current tile's products and stores run.
// DC head dims starting at d0 are reduced (D = 512: all of them in one pass;
// two passes over the halves, the second adding into S, took ~20% longer per
// ablation or backward call).  Under causal masking only the blocks holding some j <= i are
// stored (the softmax reads no other entry).
// Key tiles per workgroup: 8, or at D = 512 the longest of 8, 4 that still
// makes at least 256 workgroups (one per CU), else 2.  B1 H8 S1024 keeps 8
// (4: +3.5%); B2 H4 S700 takes 4 (backward 100.0 -> 82.6 us), B2 H3 S449
// takes 2 (ablation 34.3 -> 22.1 us).
int qk_chunk(int D, int BH, int TQ) {
    if (D != 512) return 8;
    for (int c : {8, 4})
        if ((long long)BH * TQ * ((TQ + c - 1) / c) >= 256) return c;
    return 2;
}

template <int DC>
__global__ void __launch_bounds__(256)
qk_kernel(const _Float16* __restrict__ Q, const _Float16* __restrict__ K,
          float* __restrict__ Sm, int BH, int S, int Sp, int D, int d0, int causal, float scale,
          int kQkChunk)
{
    constexpr int NK = DC / 16;
    const int TQ = (S + 63) / 64;
    const int NC = (TQ + kQkChunk - 1) / kQkChunk;  // chunks of the longest row
    const int bh = blockIdx.x % BH;
    const int u = blockIdx.x / BH;
    const int qt = causal ? TQ - 1 - u / NC : u / NC;
    const int kc = u % NC;
    const int kend = causal ? qt + 1 : TQ;        // key tiles the rows see
    const int kt0 = kc * kQkChunk;
    if (kt0 >= kend) return;                      // a chunk past the diagonal
    const int nkt = min(kend - kt0, kQkChunk);
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int g = lane >> 5, n = lane & 31;
    const int wq = w & 1, wk = w >> 1;
    const size_t base = (size_t)bh * S * D;
    half8 qf[NK];
    // key tile t: its 64 rows (DC head dims from d0) loaded as contiguous
    // 16-byte chunks per thread, bounds-checked (zeros past S), staged in
    // registers, then written to the LDS tile with the chunk index XOR-ed by
    // the row's swizzle; the B operand fragments are read from there
    constexpr int CPR = DC / 8;               // 16-byte chunks per K row
    constexpr int CH = 64 * CPR / 256;        // chunks per thread per tile
    __shared__ __attribute__((aligned(1024))) _Float16 kt[64 * DC];
    auto swz = [](int r) { return CPR == 16 ? (r & 15) : CPR == 8 ? ((r >> 1) & 7) : (r & 31); };
    auto load_k = [&](int t, u32x4* st) {
        const int j0 = t * 64;
        const auto r = rsrc(K + base + (size_t)j0 * D, (uint32_t)max(0, min(S - j0, 64)) * D * 2);
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const int ci = threadIdx.x + 256 * c, row = ci / CPR, cc = ci % CPR;
            st[c] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                r, (row * D + d0 + 8 * cc) * 2, 0, 0));
        }
    };
    auto put_k = [&](const u32x4* st) {
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const int ci = threadIdx.x + 256 * c, row = ci / CPR, cc = ci % CPR;
            *reinterpret_cast<u32x4*>(kt + row * DC + 8 * (cc ^ swz(row))) = st[c];
        }
    };
    auto frag_k = [&](half8* kf) {
        const int kr = 32 * wk + n;
#pragma unroll
        for (int kk = 0; kk < NK; ++kk)
            kf[kk] = *reinterpret_cast<const half8*>(kt + kr * DC + 8 * ((2 * kk + g) ^ swz(kr)));
    };
    const int i0 = qt * 64 + 32 * wq;  // first query row of the wave
    // the wave's 32 x 32 fp32 block goes out through LDS, so that every
    // store writes whole 128-byte row pieces: 16-byte lanes, 8 rows per
    // instruction
    __shared__ __attribute__((aligned(16))) float tb[4][32 * 32];
    float* mine = tb[w];
    auto block = [&](int t, const half8* kf) {
        floatx16 acc;
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
        for (int kk = 0; kk < NK; ++kk)
            acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(qf[kk], kf[kk], acc, 0, 0, 0);
        const int k0 = t * 64 + 32 * wk;
        if (causal && k0 > i0 + 31) return;  // every key past every row (uniform)
        // C[m = query][n = key]: register r holds query 8(r/4) + 4g + r%4, key n
#pragma unroll
        for (int r = 0; r < 16; ++r) mine[(8 * (r >> 2) + 4 * g + (r & 3)) * 32 + n] = scale * acc[r];
        __builtin_amdgcn_wave_barrier();
        wait_lgkm0();
        // lane L: row L / 8 + 8 s of the block, columns 4 (L % 8) .. +3
        const int c4 = 4 * (lane & 7);
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4) {
            const int rr = (lane >> 3) + 8 * s4;
            float4 v = *reinterpret_cast<const float4*>(mine + rr * 32 + c4);
            const int i = i0 + rr, j = k0 + c4;
            // Sp is a multiple of 64 and j of 4: the 4 columns lie in the row
            // (past S they are padding that no kernel reads)
            if (i < S && j < Sp) {
                *reinterpret_cast<float4*>(Sm + ((size_t)bh * S + i) * Sp + j) = v;
            }
        }
        // the block's LDS reads are done before the next block's writes
        wait_lgkm0();
        __builtin_amdgcn_wave_barrier();
    };
    // one LDS tile: put (after the previous step's reads, barrier), read the
    // fragments (barrier), products and stores; the next tiles' loads in
    // flight meanwhile (issued unconditionally, past the chunk re-reading its
    // last tile, so that the wait counts are exact)
    auto step = [&](int t, const u32x4* st) {
        put_k(st);
        barrier();
        half8 kf[NK];
        frag_k(kf);
        barrier();
        block(t, kf);
    };
    u32x4 sa[CH], sb[CH], sc[CH];
    const int last = kt0 + nkt - 1;
    {
        // the query tile's rows through the same LDS tile, as the A operand
        const int j0 = qt * 64;
        const auto r = rsrc(Q + base + (size_t)j0 * D, (uint32_t)max(0, min(S - j0, 64)) * D * 2);
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const int ci = threadIdx.x + 256 * c, row = ci / CPR, cc = ci % CPR;
            sa[c] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                r, (row * D + d0 + 8 * cc) * 2, 0, 0));
        }
        put_k(sa);
        barrier();
        const int qr = 32 * wq + n;
#pragma unroll
        for (int kk = 0; kk < NK; ++kk)
            qf[kk] = *reinterpret_cast<const half8*>(kt + qr * DC + 8 * ((2 * kk + g) ^ swz(qr)));
        barrier();
    }
    load_k(kt0, sa);
    load_k(min(kt0 + 1, last), sb);
    for (int t = kt0; t <= last; t += 3) {
        load_k(min(t + 2, last), sc);
        step(t, sa);
        if (t + 1 > last) break;
        load_k(min(t + 3, last), sa);
        step(t + 1, sb);
        if (t + 2 > last) break;
        load_k(min(t + 4, last), sb);
        step(t + 2, sc);
    }
}

// ---------------------------------------------------------------- softmax

// One wave per row, 4 rows per workgroup: 16-byte loads (a row of S is
// 256-byte aligned, Sp being a multiple of 64), a pass for the row max and
// sum, a second for P (the row is then in L2), 8-byte P stores.
__global__ void __launch_bounds__(256)
softmax_kernel(const float* __restrict__ Sm, _Float16* __restrict__ P, float* __restrict__ LSE,
               int BHS, int S, int Sp, int causal)
{
    const int rowid = blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (rowid >= BHS) return;
    const int lane = threadIdx.x & 63;
    const int i = rowid % S;
    const int L = causal ? i + 1 : S;                                  // visible keys
    // P columns written: the P V kernel reads whole 64-key tiles up to the end
    // of its query block (at most 128 rows), so past the diagonal write zeros
    // up to the next multiple of 128.
    const int Lp = causal ? min(Sp, ((i + 128) / 128) * 128) : Sp;
    const float4* srow = reinterpret_cast<const float4*>(Sm + (size_t)rowid * Sp);
    _Float16* prow = P + (size_t)rowid * Sp;
    // per-lane running max and sum (base-2) over 4-column groups, then a
    // wave reduction
    float m = kNegInf, l = 0.f;
#pragma unroll 4
    for (int j4 = lane; 4 * j4 < L; j4 += 64) {
        const float4 x4 = srow[j4];
        float x[4] = {x4.x, x4.y, x4.z, x4.w};
        float mx = kNegInf;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            x[e] = 4 * j4 + e < L ? x[e] * kLog2e : kNegInf;
            mx = fmaxf(mx, x[e]);
        }
        const float mn = fmaxf(m, mx);
        float add = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) add += __builtin_amdgcn_exp2f(x[e] - mn);
        l = l * __builtin_amdgcn_exp2f(m - mn) + add;
        m = mn;
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        const float mo = __shfl_xor(m, off, 64), lo = __shfl_xor(l, off, 64);
        const float mn = fmaxf(m, mo);
        l = (mn == kNegInf) ? 0.f
                            : l * __builtin_amdgcn_exp2f(m - mn) + lo * __builtin_amdgcn_exp2f(mo - mn);
        m = mn;
    }
    const float inv = 1.0f / l;
#pragma unroll 4
    for (int j4 = lane; 4 * j4 < Lp; j4 += 64) {
        float x[4] = {0.f, 0.f, 0.f, 0.f};
        if (4 * j4 < L) {
            const float4 x4 = srow[j4];
            x[0] = x4.x, x[1] = x4.y, x[2] = x4.z, x[3] = x4.w;
        }
        u32x2 pk;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int j = 4 * j4 + 2 * h;
            const float p0 = j < L ? __builtin_amdgcn_exp2f(x[2 * h] * kLog2e - m) * inv : 0.f;
            const float p1 = j + 1 < L ? __builtin_amdgcn_exp2f(x[2 * h + 1] * kLog2e - m) * inv : 0.f;
            pk[h] = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)p0) |
                    ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)p1) << 16);
        }
        *reinterpret_cast<u32x2*>(prow + 4 * j4) = pk;
    }
    if (lane == 0) LSE[rowid] = (m + __builtin_amdgcn_logf(l)) * kLn2;
}

// One wave per row with the whole row in registers, for rows of up to 512 NG
// entries: lane L holds entries 8(L + 64t) .. +7 for t < NG.  S is read once
// (two 16-byte loads per group, all in flight together), the row max and sum
// are wave reductions, and P goes out in 16-byte stores.
template <int NG>
__global__ void __launch_bounds__(256)
softmax_reg_kernel(const float* __restrict__ Sm, _Float16* __restrict__ P, float* __restrict__ LSE,
                   int BHS, int S, int Sp, int causal)
{
    const int rowid = blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (rowid >= BHS) return;
    const int lane = threadIdx.x & 63;
    const int i = rowid % S;
    const int L = causal ? i + 1 : S;  // visible keys
    // P columns written, as softmax_kernel: zeros past the diagonal up to the
    // next multiple of 128 (the P V kernel reads whole tiles)
    const int Lp = causal ? min(Sp, ((i + 128) / 128) * 128) : Sp;
    const float* srow = Sm + (size_t)rowid * Sp;
    _Float16* prow = P + (size_t)rowid * Sp;
    float x[NG][8];
#pragma unroll
    for (int t = 0; t < NG; ++t) {
        const int j = 8 * (lane + 64 * t);
        float4 a = {kNegInf, kNegInf, kNegInf, kNegInf}, b = a;
        if (j < L) {
            a = *reinterpret_cast<const float4*>(srow + j);
            b = *reinterpret_cast<const float4*>(srow + j + 4);
        }
        x[t][0] = a.x, x[t][1] = a.y, x[t][2] = a.z, x[t][3] = a.w;
        x[t][4] = b.x, x[t][5] = b.y, x[t][6] = b.z, x[t][7] = b.w;
    }
    // base-2 logits, -inf past the visible keys; the row max
    float m = kNegInf;
#pragma unroll
    for (int t = 0; t < NG; ++t)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            x[t][e] = 8 * (lane + 64 * t) + e < L ? x[t][e] * kLog2e : kNegInf;
            m = fmaxf(m, x[t][e]);
        }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
    // every row sees key 0, so m is finite
    float l = 0.f;
#pragma unroll
    for (int t = 0; t < NG; ++t)
#pragma unroll
        for (int e = 0; e < 8; ++e) l += __builtin_amdgcn_exp2f(x[t][e] - m);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) l += __shfl_xor(l, off, 64);
    const float inv = 1.0f / l;
#pragma unroll
    for (int t = 0; t < NG; ++t) {
        const int j = 8 * (lane + 64 * t);
        if (j < Lp) {
            u32x4 pk;
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                const float p0 = __builtin_amdgcn_exp2f(x[t][2 * h] - m) * inv;
                const float p1 = __builtin_amdgcn_exp2f(x[t][2 * h + 1] - m) * inv;
                pk[h] = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)p0) |
                        ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)p1) << 16);
            }
            *reinterpret_cast<u32x4*>(prow + j) = pk;
        }
    }
    if (lane == 0) LSE[rowid] = (m + __builtin_amdgcn_logf(l)) * kLn2;
}

// ---------------------------------------------------------------- P V

template <int D, int DWX = (D < 128 ? D : 128)>
struct PvGeo {
    static constexpr int DW = DWX;                 // output dims per wave
    static constexpr int DQ = D / DW;              // waves sharing a query group
    static constexpr int QG = 4 / DQ;              // 32-query groups per workgroup
    static constexpr int BM = 32 * QG;             // queries per workgroup
    static constexpr int BN = 64;                  // keys per tile
    static constexpr int CPR = D / 8;
    static constexpr int CH = BN * CPR / 256;      // V chunks per thread per tile
    static_assert(DQ * QG == 4, "4 waves");
};

template <int D>
__device__ __forceinline__ int swz_pv(int r) {
    return D == 64 ? 4 * ((r >> 1) & 1) : 4 * (r & 3);
}

// P V with D output columns per workgroup out of rows of LD (D = LD: whole
// rows; D < LD: LD / D workgroups per query tile, each owning a column slice
// of V and O), DWX of them per wave.
template <int D, int DWX = (D < 128 ? D : 128), int LD = D>
__global__ void __launch_bounds__(256, LD == D ? 1 : 2)
pv_kernel(const _Float16* __restrict__ P, const _Float16* __restrict__ V, _Float16* __restrict__ O,
          int S, int Sp, int causal)
{
    using G = PvGeo<D, DWX>;
    constexpr int NC = LD / D;  // column slices
    static_assert(NC * D == LD, "whole slices");
    __shared__ __attribute__((aligned(1024))) _Float16 vs[G::BN * D];
    __shared__ __attribute__((aligned(1024))) _Float16 ps[G::BM * G::BN];
    constexpr int PCH = G::BM * G::BN / 8 / 256;  // 16-byte P chunks per thread per tile
    static_assert(PCH >= 1, "whole P tile per pass");
    const int TQ = (S + G::BM - 1) / G::BM;
    const int cs = blockIdx.x % NC, item = blockIdx.x / NC;
    const int bh = item / TQ, qt = item % TQ;
    const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int g = lane >> 5, n = lane & 31;
    const int qg = w / G::DQ, dq = w % G::DQ;
    const int q0 = qt * G::BM;
    const int qrow = q0 + 32 * qg + n;
    const int c0 = cs * D;  // first column of this workgroup's slice
    const size_t vbase = (size_t)bh * S * LD + c0;
    // the P rows q0 .. q0 + BM - 1 of the workgroup (rows past S read zero)
    const auto prs = rsrc(P + ((size_t)bh * S + q0) * Sp, (uint32_t)min(S - q0, G::BM) * Sp * 2);
    auto swzp = [](int r) { return (r >> 1) & 7; };
    // causal = 1: rows see keys up to their own (lower triangle); causal = 2:
    // rows see keys from their own on (upper triangle: P^T and dS^T of a
    // causal call, zero below the diagonal), so the walk starts at the
    // diagonal tile
    const int kend = causal == 1 ? min(S, q0 + G::BM) : S;
    const int nT = (kend + G::BN - 1) / G::BN;
    const int t0 = causal == 2 ? q0 / G::BN : 0;

    floatx16 o[G::DW / 32];
#pragma unroll
    for (int b = 0; b < G::DW / 32; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[b][r] = 0.f;

    // V rows and the BM x BN block of P of key tile t, as contiguous 16-byte
    // chunks per thread (P once per workgroup, through an XOR-swizzled LDS
    // tile: every wave of a query group reads the same P fragments)
    u32x4 st[G::CH], pc[PCH];
    auto load = [&](int t) {
        const int j0 = t * G::BN;
        // rows j0 .. of the slice: the last valid row ends inside the range,
        // the next one starts past it (zeros)
        const auto r = rsrc(V + vbase + (size_t)j0 * LD,
                            (uint32_t)(min(S - j0, G::BN) * LD - c0) * 2);
#pragma unroll
        for (int u = 0; u < G::CH; ++u) {
            const int ci = tid + 256 * u;
            st[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                  r, ((ci / G::CPR) * LD + 8 * (ci % G::CPR)) * 2, 0, 0));
        }
#pragma unroll
        for (int c = 0; c < PCH; ++c) {
            const int ci = tid + 256 * c, row = ci >> 3, cc = ci & 7;
            pc[c] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                prs, (row * Sp + j0 + 8 * cc) * 2, 0, 0));
        }
    };
    auto store = [&]() {
#pragma unroll
        for (int u = 0; u < G::CH; ++u) {
            const int ci = tid + 256 * u, row = ci / G::CPR, cc = ci % G::CPR;
            *reinterpret_cast<u32x4*>(vs + row * D + 8 * (cc ^ swz_pv<D>(row))) = st[u];
        }
#pragma unroll
        for (int c = 0; c < PCH; ++c) {
            const int ci = tid + 256 * c, row = ci >> 3, cc = ci & 7;
            *reinterpret_cast<u32x4*>(ps + row * G::BN + 8 * (cc ^ swzp(row))) = pc[c];
        }
    };

    const int n16 = n >> 4, jj = n & 15;
    const int sub = (jj & 3) >> 1, half = jj & 1;
    const int sw = swz_pv<D>(jj >> 2);  // (row & 3) == jj >> 2 for every row read
    // the next tile's loads go out after this tile's stores to LDS,
    // unconditionally (past the last tile re-reading it) so that the wait
    // counts stay exact
    load(t0);
    for (int t = t0; t < nT; ++t) {
        store();
        barrier();
        load(min(t + 1, nT - 1));
        // P^T operands: this lane's query, keys 16ks + 8g .. +7 of the tile
        half8 pcur[G::BN / 16];
        {
            const int pr = 32 * qg + n;
#pragma unroll
            for (int ks = 0; ks < G::BN / 16; ++ks)
                pcur[ks] = *reinterpret_cast<const half8*>(ps + pr * G::BN +
                                                           8 * ((2 * ks + g) ^ swzp(pr)));
        }
        // transposed reads deliver keys 16ks + 8g + 4tt + 0..3: the lane's 8 keys
        // are contiguous, matching a 16-byte load of its P row
        const _Float16* rowp = vs + (8 * g + (jj >> 2)) * D + 4 * half;
#pragma unroll
        for (int ks = 0; ks < G::BN / 16; ++ks) {
            const half8 pf = pcur[ks];
#pragma unroll
            for (int b = 0; b < G::DW / 32; ++b) {
                const int logical = (G::DW * dq) / 8 + 4 * b + 2 * n16 + sub;
                const _Float16* pb = rowp + 8 * (logical ^ sw) + 16 * ks * D;
                half4 part[2];
#pragma unroll
                for (int tt = 0; tt < 2; ++tt)
                    part[tt] = __builtin_bit_cast(
                        half4, __builtin_amdgcn_ds_read_tr16_b64_v4f16((lds_half4*)(pb + 4 * tt * D)));
                const half8 a = {part[0][0], part[0][1], part[0][2], part[0][3],
                                 part[1][0], part[1][1], part[1][2], part[1][3]};
                o[b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, pf, o[b], 0, 0, 0);
            }
        }
        barrier();
    }
    if (qrow < S) {
        _Float16* orow = O + vbase + (size_t)qrow * LD + G::DW * dq;
#pragma unroll
        for (int b = 0; b < G::DW / 32; ++b)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                u32x2 pk;
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const _Float16 lo = (_Float16)o[b][4 * q4 + 2 * h];
                    const _Float16 hi = (_Float16)o[b][4 * q4 + 2 * h + 1];
                    pk[h] = (uint32_t)__builtin_bit_cast(uint16_t, lo) |
                            ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
                }
                *reinterpret_cast<u32x2*>(orow + 32 * b + 8 * q4 + 4 * g) = pk;
            }
    }
}

// P V for D = 64, 128 with DW output dims per wave (DW = D: four 32-row
// groups, 128 queries per workgroup; DW = D/2: two 32-row groups of two
// waves each, 64 queries), streaming: the V rows and P fragments of key tiles t+1 and t+2
// are in flight while tile t's products run (three register sets, the loop
// unrolled by three so that each set has a fixed name).  Workgroup order:
// (batch, head) fastest, so that a head's query tiles land on one XCD (heads
// are dealt round-robin to the XCDs when B*H is a multiple of 8) and share
// its V in that XCD's L2; under causal masking the heaviest query tiles
// first across all heads (keeping a head's tiles back to back on its XCD
// instead cut the re-reads but cost more in balance than it saved).
template <int D, int DW>
__global__ void __launch_bounds__(256, (D == 64 || DW < D) ? 2 : 1)
pv_stream_kernel(const _Float16* __restrict__ P, const _Float16* __restrict__ V,
                 _Float16* __restrict__ O, int BH, int S, int Sp, int causal)
{
    using G = PvGeo<D, DW>;
    constexpr int PCH = G::BM * G::BN / 8 / 256;  // 16-byte P chunks per thread per tile
    __shared__ __attribute__((aligned(1024))) _Float16 vs[G::BN * D];
    __shared__ __attribute__((aligned(1024))) _Float16 ps[G::BM * G::BN];
    const int TQ = (S + G::BM - 1) / G::BM;
    const int bh = blockIdx.x % BH, u = blockIdx.x / BH;
    // causal, 128-row tiles (one workgroup per CU): heaviest first.  64-row
    // tiles (two per CU): the heavy half of the tiles in the first half of
    // the grid and the light half in the second, so that the two workgroups
    // a CU receives carry about T+1 tiles of work between them.
    const int qt = !causal ? u : G::BM == 128 ? TQ - 1 - u
                                              : (u < TQ / 2 ? TQ - 1 - u : u - TQ / 2);
    const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int g = lane >> 5, n = lane & 31;
    const int qg = w / G::DQ, dq = w % G::DQ;
    const int q0 = qt * G::BM;
    const int qrow = q0 + 32 * qg + n;
    const size_t vbase = (size_t)bh * S * D;
    const int kend = causal ? min(S, q0 + G::BM) : S;
    const int nT = (kend + G::BN - 1) / G::BN;

    floatx16 o[G::DW / 32];
#pragma unroll
    for (int b = 0; b < G::DW / 32; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[b][r] = 0.f;

    // V rows of key tile t (bounds-checked: zeros past S) and the tile's
    // 128 x 64 block of P (written up to the workgroup's last tile end), both
    // as contiguous 16-byte chunks per thread; P goes through an XOR-swizzled
    // LDS tile (16-byte fragment reads across 32 rows straight from global
    // memory requested every line four times)
    // P rows q0 .. q0 + 127 of the tile (rows past S read zero)
    const auto prs = rsrc(P + ((size_t)bh * S + q0) * Sp, (uint32_t)min(S - q0, G::BM) * Sp * 2);
    auto swzp = [](int r) { return (r >> 1) & 7; };
    auto load = [&](int t, u32x4* st, u32x4* pc) {
        const int j0 = t * G::BN;
        const auto r = rsrc(V + vbase + (size_t)j0 * D, (uint32_t)min(S - j0, G::BN) * D * 2);
#pragma unroll
        for (int c = 0; c < G::CH; ++c)
            st[c] = __builtin_bit_cast(
                u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, 16 * (tid + 256 * c), 0, 0));
#pragma unroll
        for (int c = 0; c < PCH; ++c) {
            const int ci = tid + 256 * c, row = ci >> 3, cc = ci & 7;
            pc[c] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                prs, (row * Sp + j0 + 8 * cc) * 2, 0, 0));
        }
    };
    const int n16 = n >> 4, jj = n & 15;
    const int sub = (jj & 3) >> 1, half = jj & 1;
    const int sw = swz_pv<D>(jj >> 2);  // (row & 3) == jj >> 2 for every row read
    auto step = [&](const u32x4* st, const u32x4* pc) {
#pragma unroll
        for (int c = 0; c < G::CH; ++c) {
            const int ci = tid + 256 * c, row = ci / G::CPR, cc = ci % G::CPR;
            *reinterpret_cast<u32x4*>(vs + row * D + 8 * (cc ^ swz_pv<D>(row))) = st[c];
        }
#pragma unroll
        for (int c = 0; c < PCH; ++c) {
            const int ci = tid + 256 * c, row = ci >> 3, cc = ci & 7;
            *reinterpret_cast<u32x4*>(ps + row * G::BN + 8 * (cc ^ swzp(row))) = pc[c];
        }
        barrier();
        half8 pf[G::BN / 16];
        {
            const int pr = 32 * qg + n;
#pragma unroll
            for (int ks = 0; ks < G::BN / 16; ++ks)
                pf[ks] = *reinterpret_cast<const half8*>(ps + pr * G::BN + 8 * ((2 * ks + g) ^ swzp(pr)));
        }
        // transposed reads deliver keys 16ks + 8g + 4tt + 0..3, the lane's P keys
        const _Float16* rowp = vs + (8 * g + (jj >> 2)) * D + 4 * half;
#pragma unroll
        for (int ks = 0; ks < G::BN / 16; ++ks)
#pragma unroll
            for (int b = 0; b < G::DW / 32; ++b) {
                const int logical = (G::DW * dq) / 8 + 4 * b + 2 * n16 + sub;
                const _Float16* pb = rowp + 8 * (logical ^ sw) + 16 * ks * D;
                half4 part[2];
#pragma unroll
                for (int tt = 0; tt < 2; ++tt)
                    part[tt] = __builtin_bit_cast(
                        half4, __builtin_amdgcn_ds_read_tr16_b64_v4f16((lds_half4*)(pb + 4 * tt * D)));
                const half8 a = {part[0][0], part[0][1], part[0][2], part[0][3],
                                 part[1][0], part[1][1], part[1][2], part[1][3]};
                o[b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, pf[ks], o[b], 0, 0, 0);
            }
        barrier();
    };
    // Loads past the last tile re-read the last tile (unused): issuing every
    // load unconditionally keeps the wait counts exact, so the products of
    // tile t wait for tile t's loads only.
    u32x4 s0[G::CH], s1[G::CH], s2[G::CH];
    u32x4 f0[PCH], f1[PCH], f2[PCH];
    const int last = nT - 1;
    load(0, s0, f0);
    load(min(1, last), s1, f1);
    for (int t = 0; t < nT; t += 3) {
        load(min(t + 2, last), s2, f2);
        step(s0, f0);
        if (t + 1 >= nT) break;
        load(min(t + 3, last), s0, f0);
        step(s1, f1);
        if (t + 2 >= nT) break;
        load(min(t + 4, last), s1, f1);
        step(s2, f2);
    }
    if (qrow < S) {
        _Float16* orow = O + vbase + (size_t)qrow * D + G::DW * dq;
#pragma unroll
        for (int b = 0; b < G::DW / 32; ++b)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                u32x2 pk;
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const _Float16 lo = (_Float16)o[b][4 * q4 + 2 * h];
                    const _Float16 hi = (_Float16)o[b][4 * q4 + 2 * h + 1];
                    pk[h] = (uint32_t)__builtin_bit_cast(uint16_t, lo) |
                            ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
                }
                *reinterpret_cast<u32x2*>(orow + 32 * b + 8 * q4 + 4 * g) = pk;
            }
    }
}

// O = P V at D = 512 (P: [BH, S, Sp] fp16, V and O: [BH, S, 512]): four
// workgroups per 64-row query tile, each owning 128 output columns (two waves
// of 64 per 32-row group).  At B1 H8 S1024 (causal) that is 512 workgroups,
// two per CU; one workgroup per 32-row tile and all 512 columns gave 256,
// one per CU, and took 16-22% longer per call in the ablation and the
// backward.
void pv512(hipStream_t st, const _Float16* P, const _Float16* V, _Float16* O, int BH, int S,
           int Sp, int causal) {
    constexpr int DV = 128, DW = 64;
    using G = PvGeo<DV, DW>;
    const int TQ = (S + G::BM - 1) / G::BM;
    hipLaunchKernelGGL((pv_kernel<DV, DW, 512>), dim3((unsigned)(BH * TQ * (512 / DV))), dim3(256),
                       0, st, P, V, O, S, Sp, causal);
}

// ---------------------------------------------------------------- backward, D = 512
//
// The D <= 128 backward (bwd_dq.hip, bwd_dkdv.hip) keeps a key tile's K and V
// rows and its dK, dV accumulators in registers; at D = 512 those alone are
// four times the register file of a wave.  The D = 512 backward instead
// materialises the n x n intermediates, with the ablation's kernels:
//   S  = scale Q K^T, dP = dO V^T      qk_kernel, two 256-wide passes each (fp32)
//   Dlt = rowsum(dO * O)               bwd512_delta_kernel
//   P = exp(S - LSE), dS = scale P (dP - Dlt)   bwd512_ds_kernel: dS, and P^T,
//                                      dS^T transposed through LDS (fp16)
//   dV = P^T dO, dK = dS^T Q, dQ = dS K         pv_kernel
// the storing-and-re-reading trade that "Validating Memory-Optimal Transformer
// Kernels on Real Hardware" (section 4) measures against atomics: no atomics,
// deterministic, and the n x n traffic paid in HBM.

// Dlt[row] = dO_row . O_row (fp32), one wave per row, 8 dims per lane.
__global__ void __launch_bounds__(256)
bwd512_delta_kernel(const _Float16* __restrict__ dO, const _Float16* __restrict__ O,
                    float* __restrict__ dlt, int BHS)
{
    const int row = blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (row >= BHS) return;
    const int lane = threadIdx.x & 63;
    const half8 a = *reinterpret_cast<const half8*>(dO + (size_t)row * 512 + 8 * lane);
    const half8 b = *reinterpret_cast<const half8*>(O + (size_t)row * 512 + 8 * lane);
    float x = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) x = __builtin_fmaf((float)a[e], (float)b[e], x);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
    if (lane == 0) dlt[row] = x;
}

// One workgroup per 64 x 64 tile (query block bi, key block bj) of a (batch,
// head), every tile of the S x Sp matrices (tiles past the causal diagonal
// and columns past S write zeros): P = exp(S - LSE) where key j is visible
// to query i, else 0; dS = scale P (dP - Dlt).  Thread t takes row t/4 of
// the tile, 16 columns; dS goes out row-major, P and dS also into LDS and out
// transposed (P^T, dS^T: row = key, column = query).
__global__ void __launch_bounds__(256)
bwd512_ds_kernel(const float* __restrict__ Sm, const float* __restrict__ dPm,
                 const float* __restrict__ LSE, const float* __restrict__ dlt,
                 _Float16* __restrict__ dS, _Float16* __restrict__ PT, _Float16* __restrict__ dST,
                 int S, int Sp, int T, int causal, float scale)
{
    constexpr int LD = 64 + 8;  // padded LDS row (halfs)
    __shared__ _Float16 tp[64 * LD];
    __shared__ _Float16 td[64 * LD];
    const int tiles = T * T;
    const int bh = blockIdx.x / tiles, rem = blockIdx.x % tiles;
    const int bi = rem / T, bj = rem % T;
    const int tid = threadIdx.x;
    const int r = tid >> 2, c0 = 16 * (tid & 3);
    const int i = bi * 64 + r;
    const bool live = (!causal || bj <= bi) && i < S;
    float lse = 0.f, dl = 0.f;
    if (live) {
        lse = LSE[(size_t)bh * S + i];
        dl = dlt[(size_t)bh * S + i];
    }
    float sv[16], dpv[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) sv[e] = dpv[e] = 0.f;
    if (live) {
        const float4* s4 = reinterpret_cast<const float4*>(Sm + ((size_t)bh * S + i) * Sp + bj * 64 + c0);
        const float4* d4 = reinterpret_cast<const float4*>(dPm + ((size_t)bh * S + i) * Sp + bj * 64 + c0);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float4 a = s4[q], b = d4[q];
            sv[4 * q] = a.x, sv[4 * q + 1] = a.y, sv[4 * q + 2] = a.z, sv[4 * q + 3] = a.w;
            dpv[4 * q] = b.x, dpv[4 * q + 1] = b.y, dpv[4 * q + 2] = b.z, dpv[4 * q + 3] = b.w;
        }
    }
    uint32_t dsw[8];
#pragma unroll
    for (int e = 0; e < 16; e += 2) {
        _Float16 ph[2], dh[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int j = bj * 64 + c0 + e + u;
            const bool vis = live && j < S && (!causal || j <= i);
            // a masked entry may hold garbage (never written): select, not multiply
            const float p = vis ? __builtin_amdgcn_exp2f((sv[e + u] - lse) * kLog2e) : 0.f;
            const float ds = vis ? scale * p * (dpv[e + u] - dl) : 0.f;
            ph[u] = (_Float16)p;
            dh[u] = (_Float16)ds;
            tp[r * LD + c0 + e + u] = ph[u];
            td[r * LD + c0 + e + u] = dh[u];
        }
        dsw[e / 2] = (uint32_t)__builtin_bit_cast(uint16_t, dh[0]) |
                     ((uint32_t)__builtin_bit_cast(uint16_t, dh[1]) << 16);
    }
    if (i < S) {
        u32x4* dst = reinterpret_cast<u32x4*>(dS + ((size_t)bh * S + i) * Sp + bj * 64 + c0);
        dst[0] = u32x4{dsw[0], dsw[1], dsw[2], dsw[3]};
        dst[1] = u32x4{dsw[4], dsw[5], dsw[6], dsw[7]};
    }
    __syncthreads();
    // transposed: row r of the output tile is key j = bj*64 + r, columns are
    // the queries bi*64 + c0 .. +15
    const int j = bj * 64 + r;
    if (j < S) {
        uint32_t pw[8], tw[8];
#pragma unroll
        for (int e = 0; e < 16; e += 2) {
            pw[e / 2] = (uint32_t)__builtin_bit_cast(uint16_t, tp[(c0 + e) * LD + r]) |
                        ((uint32_t)__builtin_bit_cast(uint16_t, tp[(c0 + e + 1) * LD + r]) << 16);
            tw[e / 2] = (uint32_t)__builtin_bit_cast(uint16_t, td[(c0 + e) * LD + r]) |
                        ((uint32_t)__builtin_bit_cast(uint16_t, td[(c0 + e + 1) * LD + r]) << 16);
        }
        u32x4* pd = reinterpret_cast<u32x4*>(PT + ((size_t)bh * S + j) * Sp + bi * 64 + c0);
        u32x4* dd = reinterpret_cast<u32x4*>(dST + ((size_t)bh * S + j) * Sp + bi * 64 + c0);
        pd[0] = u32x4{pw[0], pw[1], pw[2], pw[3]};
        pd[1] = u32x4{pw[4], pw[5], pw[6], pw[7]};
        dd[0] = u32x4{tw[0], tw[1], tw[2], tw[3]};
        dd[1] = u32x4{tw[4], tw[5], tw[6], tw[7]};
    }
}

}  // namespace

int unfused_row_stride(int S) { return (S + 63) / 64 * 64; }

hipError_t launch_unfused(const FwdArgs& a, void* workspace) {
    const int S = a.S, Sp = unfused_row_stride(S);
    const int BH = a.B * a.H;
    float* Sm = reinterpret_cast<float*>(workspace);
    _Float16* P = reinterpret_cast<_Float16*>(Sm + (size_t)BH * S * Sp);
    const int TQ = (S + 63) / 64;
    const int kQkChunk = qk_chunk(a.D, BH, TQ);
    const dim3 qk_grid((unsigned)(BH * TQ * ((TQ + kQkChunk - 1) / kQkChunk)));
    const hipStream_t st = (hipStream_t)a.stream;
    const _Float16* q = (const _Float16*)a.q;
    const _Float16* k = (const _Float16*)a.k;
    if (a.D == 64)
        hipLaunchKernelGGL((qk_kernel<64>), qk_grid, dim3(256), 0, st, q, k, Sm, BH, S, Sp, 64, 0, a.causal, a.scale, kQkChunk);
    else if (a.D == 128)
        hipLaunchKernelGGL((qk_kernel<128>), qk_grid, dim3(256), 0, st, q, k, Sm, BH, S, Sp, 128, 0, a.causal, a.scale, kQkChunk);
    else {
        // two head-dim sub-tiles, summed into S before the softmax
        hipLaunchKernelGGL((qk_kernel<512>), qk_grid, dim3(256), 0, st, q, k, Sm, BH, S, Sp, 512, 0, a.causal, a.scale, kQkChunk);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int BHS = BH * S;
    const dim3 sm_grid((unsigned)((BHS + 3) / 4));
    // rows of up to 4096 entries are held in registers
    if (Sp <= 512)
        hipLaunchKernelGGL(softmax_reg_kernel<1>, sm_grid, dim3(256), 0, st, Sm, P, a.lse, BHS, S, Sp, a.causal);
    else if (Sp <= 1024)
        hipLaunchKernelGGL(softmax_reg_kernel<2>, sm_grid, dim3(256), 0, st, Sm, P, a.lse, BHS, S, Sp, a.causal);
    else if (Sp <= 2048)
        hipLaunchKernelGGL(softmax_reg_kernel<4>, sm_grid, dim3(256), 0, st, Sm, P, a.lse, BHS, S, Sp, a.causal);
    else if (Sp <= 4096)
        hipLaunchKernelGGL(softmax_reg_kernel<8>, sm_grid, dim3(256), 0, st, Sm, P, a.lse, BHS, S, Sp, a.causal);
    else
        hipLaunchKernelGGL(softmax_kernel, sm_grid, dim3(256), 0, st, Sm, P, a.lse, BHS, S, Sp, a.causal);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (a.D == 512) {
        pv512(st, P, (const _Float16*)a.v, (_Float16*)a.o, BH, S, Sp, a.causal);
        return hipGetLastError();
    }
    // 64-row tiles, two workgroups per CU
    const dim3 pv_grid((unsigned)(BH * ((a.S + 63) / 64)));
    if (a.D == 64)
        hipLaunchKernelGGL((pv_stream_kernel<64, 32>), pv_grid, dim3(256), 0, st, P,
                           (const _Float16*)a.v, (_Float16*)a.o, BH, S, Sp, a.causal);
    else
        hipLaunchKernelGGL((pv_stream_kernel<128, 64>), pv_grid, dim3(256), 0, st, P,
                           (const _Float16*)a.v, (_Float16*)a.o, BH, S, Sp, a.causal);
    return hipGetLastError();
}

}  // namespace attn

namespace attn {

size_t bwd512_workspace_bytes(int B, int H, int S) {
    const size_t bh = (size_t)B * H, n = (size_t)S * unfused_row_stride(S);
    // S, dP (fp32); dS, P^T, dS^T (fp16); Dlt (fp32 per row)
    return bh * n * (4 + 4 + 2 + 2 + 2) + bh * S * 4;
}

hipError_t launch_bwd512(const BwdArgs& a) {
    const int S = a.S, Sp = unfused_row_stride(S), BH = a.B * a.H;
    const size_t n = (size_t)BH * S * Sp;
    float* Sm = reinterpret_cast<float*>(a.workspace);
    float* dPm = Sm + n;
    _Float16* dS = reinterpret_cast<_Float16*>(dPm + n);
    _Float16* PT = dS + n;
    _Float16* dST = PT + n;
    float* dlt = reinterpret_cast<float*>(dST + n);
    const hipStream_t st = (hipStream_t)a.stream;
    const _Float16* q = (const _Float16*)a.q;
    const _Float16* k = (const _Float16*)a.k;
    const _Float16* v = (const _Float16*)a.v;
    const _Float16* dO = (const _Float16*)a.dout;
    const int TQ = (S + 63) / 64;
    const int kQkChunk = qk_chunk(512, BH, TQ);
    const dim3 qk_grid((unsigned)(BH * TQ * ((TQ + kQkChunk - 1) / kQkChunk)));
    hipLaunchKernelGGL((qk_kernel<512>), qk_grid, dim3(256), 0, st, q, k, Sm, BH, S, Sp, 512, 0, a.causal, a.scale, kQkChunk);
    hipLaunchKernelGGL((qk_kernel<512>), qk_grid, dim3(256), 0, st, dO, v, dPm, BH, S, Sp, 512, 0, a.causal, 1.0f, kQkChunk);
    const int BHS = BH * S;
    hipLaunchKernelGGL(bwd512_delta_kernel, dim3((unsigned)((BHS + 3) / 4)), dim3(256), 0, st, dO,
                       (const _Float16*)a.o, dlt, BHS);
    hipLaunchKernelGGL(bwd512_ds_kernel, dim3((unsigned)(BH * TQ * TQ)), dim3(256), 0, st, Sm, dPm,
                       a.lse, dlt, dS, PT, dST, S, Sp, TQ, a.causal, a.scale);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // dV = P^T dO, dK = dS^T Q (rows = keys; causal: the queries from the key
    // on), dQ = dS K (causal rows)
    pv512(st, PT, dO, (_Float16*)a.dv, BH, S, Sp, a.causal ? 2 : 0);
    pv512(st, dST, q, (_Float16*)a.dk, BH, S, Sp, a.causal ? 2 : 0);
    pv512(st, dS, k, (_Float16*)a.dq, BH, S, Sp, (int)a.causal);
    return hipGetLastError();
}

}  // namespace attn
