// Device helpers shared by the fused attention kernels (gfx950).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {
namespace detail {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __fp16 fp16x4_raw __attribute__((__vector_size__(4 * sizeof(__fp16))));
typedef __attribute__((address_space(3))) fp16x4_raw lds_half4;

constexpr float kNegInf = -__builtin_inff();
constexpr float kFltMax = 3.402823466e38f;
constexpr float kLn2 = 0.693147180559945309417f;
constexpr float kLazyTau = 8.0f;  // log2 headroom before the reference max moves

__device__ __forceinline__ void wait_lgkm0() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4) | (0 << 8));
    asm volatile("" ::: "memory");
}
// Workgroup barrier after this wave's LDS writes have landed.  No full memory
// fence: the global loads of later tiles stay in flight across it.
__device__ __forceinline__ void barrier() {
    wait_lgkm0();
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Both halves of the wave end up holding max / sum over lanes n and n+32.
__device__ __forceinline__ float max_halves(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                    false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_halves(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                    false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Online softmax of one 32-key x 32-query S^T accumulator block.
//
// Accumulator register r of lane (g, n) holds key 8(r/4) + 4g + r%4 (relative
// to the block) for query n.  Keys with 8(r/4) + r%4 > lim are masked (MASK
// only).  c = |scale| log2(e).  m is the running reference max in log2 units,
// l this lane's share of the row sum, o the NB output accumulator blocks.
// P is returned in fp16 (round to nearest even) as the B operand of the two
// 16-key P V steps: pf[h][e] = weight of accumulator register 8h + e.
//
// The weights are computed against the current reference max; only when a
// row max outgrows it by more than 2^kLazyTau is the output rescaled and the
// weights recomputed, so every weight is <= 2^kLazyTau and most blocks skip
// the rescale.  The result equals the eager rescale up to rounding.
template <bool MASK, int NB>
__device__ __forceinline__ void online_softmax(floatx16 s, int lim, float c, float& m, float& l,
                                               floatx16* o, half8* pf) {
    float mx = kNegInf;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        if (MASK && (8 * (r >> 2) + (r & 3)) > lim) s[r] = kNegInf;
        mx = fmaxf(mx, s[r]);
    }
    auto weights = [&](float mref) {
        float psum = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float t = __builtin_fmaf(s[r], c, -mref);
            if (MASK && (8 * (r >> 2) + (r & 3)) > lim) t = kNegInf;
            const float p = __builtin_amdgcn_exp2f(t);
            psum += p;
            pf[r >> 3][r & 7] = (_Float16)p;
        }
        return psum;
    };
    float psum = weights(m);
    mx = max_halves(mx);
    // fmaxf keeps the candidate finite when every key of the block is masked
    // (c * -inf) or c == 0 (0 * -inf).
    const float cand = fmaxf(c * mx, -kFltMax);
    if (__builtin_amdgcn_ballot_w64(cand > m + kLazyTau) != 0) {
        const float m_new = fmaxf(m, cand);
        const float alpha = __builtin_amdgcn_exp2f(m - m_new);
        m = m_new;
        l *= alpha;
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) o[b][r] *= alpha;
        psum = weights(m);
    }
    l += psum;
}

// Online softmax of one 32-key x 32-query S^T block (register r of lane
// (g, n): key 8(r/4) + 4g + r%4 of the block, query n; keys with
// 8(r/4) + r%4 > lim are masked when MASK).  c = |scale| log2(e); m: the
// running reference max (log2 units), l: this lane's share of the row sum,
// o: the output blocks.  P^T (fp16, round to nearest even) goes to pf as the
// B operand of the two 16-key P V steps.
//
// The weights are formed against the current reference max m without
// looking at the row max.  Every weight is at most the lane's sum of them, so
// while every lane's sum stays within 2^kLazyTau no weight exceeds it and
// nothing else is done; otherwise (or when the sum is NaN: m = -inf meeting a
// masked key) the row max is taken, the reference moves to it, the output and
// sum are rescaled and the weights formed again.  So the row-max tree runs
// only on the rare blocks that move the reference, and every weight stays
// <= 2^kLazyTau (fp16-safe) either way.  The sum runs as a tree (short
// dependence chains), and the speculative weights are pinned ahead of the
// branch so that they stay in the same scheduling region as the next tile's
// matrix instructions.
constexpr float kLazyBound = 256.0f;  // 2^kLazyTau
static_assert(kLazyTau == 8.0f, "kLazyBound = 2^kLazyTau");
template <bool MASK, int NB, bool PIPE, int NMF = 8, int NDS = 0>
__device__ __forceinline__ void softmax_block(floatx16 s, int lim, float c, float& m, float& l,
                                              floatx16* o, half8* pf) {
    if (MASK) {
#pragma unroll
        for (int r = 0; r < 16; ++r)
            if ((8 * (r >> 2) + (r & 3)) > lim) s[r] = kNegInf;
    }
    // weights against reference mref: P^T in fp16 into pf, and this lane's
    // sum in fp32 (four partial sums, then a tree)
    auto weights = [&](float mref) {
        float q[4];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float t = __builtin_fmaf(s[r], c, -mref);
            if (MASK && (8 * (r >> 2) + (r & 3)) > lim) t = kNegInf;
            const float e = __builtin_amdgcn_exp2f(t);
            if (r < 4)
                q[r] = e;
            else
                q[r & 3] += e;
            pf[r >> 3][r & 7] = (_Float16)e;
        }
        return (q[0] + q[1]) + (q[2] + q[3]);
    };
    float psum = weights(m);
    // keep the speculative weights ahead of the branch
    asm volatile("" : "+v"(psum));
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        u32x4 x = __builtin_bit_cast(u32x4, pf[h]);
        asm volatile("" : "+v"(x));
        pf[h] = __builtin_bit_cast(half8, x);
    }
    if (PIPE) {
        // interleave the next tile's Q K^T (NMF MFMAs and the NDS LDS reads
        // of their operands, issued by the caller in this region) with this
        // softmax's vector work, the reads running up to four ahead
        constexpr int pre = NDS < 4 ? NDS : 4;
        if (pre > 0) __builtin_amdgcn_sched_group_barrier(0x100, pre, 0);  // DS read
        __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);   // VALU
#pragma unroll
        for (int i = 0; i < NMF; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
            if (i + pre < NDS) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, 40 / NMF, 0);  // VALU
        }
    }
    // every weight is at most the lane's sum; the sum is NaN when m = -inf
    // meets a masked key (-inf + inf), and that too takes the branch
    if (__builtin_amdgcn_ballot_w64(!(psum <= kLazyBound)) != 0) {
        const float mx = fmaxf(fmaxf(fmaxf(fmaxf(s[0], s[1]), s[2]), fmaxf(fmaxf(s[3], s[4]), s[5])),
                               fmaxf(fmaxf(fmaxf(s[6], s[7]), s[8]),
                                     fmaxf(fmaxf(fmaxf(s[9], s[10]), s[11]),
                                           fmaxf(fmaxf(fmaxf(s[12], s[13]), s[14]), s[15]))));
        // fmaxf keeps the candidate finite when every key is masked
        // (c * -inf) or c == 0 (0 * -inf)
        const float cand = fmaxf(c * max_halves(mx), -kFltMax);
        const float m_new = fmaxf(m, cand);
        const float alpha = __builtin_amdgcn_exp2f(m - m_new);
        m = m_new;
        l *= alpha;
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) o[b][r] *= alpha;
        psum = weights(m);
    }
    l += psum;
}

}  // namespace detail
}  // namespace attn
