/*
 * attn.h - C ABI of the fused scaled-dot-product attention forward for
 * AMD Instinct MI355X (gfx950).
 *
 *   O = softmax(scale * Q K^T + causal mask) V
 *   LSE[i] = log( sum_{visible j} exp(scale * q_i . k_j) )      (natural log)
 *
 * The operation is the SDPA forward that "An Optimal Mapper Meets a Real GPU"
 * lowers and gates against PyTorch SDPA (section "Ground rules": FP16 in,
 * FP32 accumulate; section "Experiment one": query length equals key length,
 * causal or not).  The per-row log-sum-exp output and the head-dim-512 case,
 * whose two 256-wide halves of Q K^T are summed in logit space before the
 * softmax, follow the STAGE_D.md notes (sections "2. External k_sub Merge is
 * Mathematically Impossible", "4. Guard Dead Code" and "6. The k_tile
 * Parameter").
 *
 * Plain C (C99), no HIP or torch types: pointers, sizes and a stream handle.
 *
 * Data layout (all contiguous, row-major):
 *   q, k, v, o : fp16 (IEEE binary16 bit patterns), shape [B, H, S, D]
 *   lse        : fp32, shape [B, H, S]
 * All pointers are DEVICE pointers on the current HIP device.
 *
 * Semantics
 *   - causal != 0 hides key j from query i when j > i (query and key lengths
 *     are equal, so top-left and bottom-right alignment coincide).
 *   - scale multiplies the fp32 dot product before the softmax; any finite
 *     value is accepted (0 gives uniform weights, a negative value is applied
 *     exactly by negating Q).
 *   - Accumulation is fp32; P is rounded to fp16 (nearest even) before the
 *     P V product; O is rounded to fp16 (nearest even) once, after dividing
 *     by the row sum.
 *   - Any S >= 1 is accepted (up to the size limit below): ragged tails are
 *     masked, never read out of bounds.
 *   - Deterministic: the same inputs give the same output bytes (no atomics,
 *     fixed reduction order).  The kernel depends on the whole call: at
 *     D = 128 a call with B*H*ceil(S/128) >= 512 query tiles of 128 rows
 *     (>= 256 when not causal) runs the 128-row kernel, a smaller one the
 *     64-row kernel, so a (b, h)
 *     slice of a large call launched on its own agrees with its slice of the
 *     call to rounding (both within the parity gate), bit for bit only when
 *     both calls take the same kernel.
 *
 * Ownership and synchronisation
 *   The caller allocates and owns every buffer; the library never allocates
 *   or frees caller memory.  attn_fwd enqueues one kernel on `stream` and
 *   returns without waiting; the caller synchronises.  o and lse must not
 *   overlap the inputs or each other.
 *
 * Errors
 *   Every entry point validates its arguments BEFORE any HIP call and returns
 *   0 (ATTN_OK) or a negative ATTN_ERR_* code; nothing aborts or prints.
 *   ATTN_ERR_LAUNCH means the kernel launch itself failed; the HIP error code
 *   is kept per thread and returned by attn_last_hip_error().
 */
#ifndef ATTN_H
#define ATTN_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ATTN_OK 0
#define ATTN_ERR_NULL -1      /* a required pointer is NULL */
#define ATTN_ERR_SHAPE -2     /* B, H or S < 1, the sizes overflow 32-bit row
                                 indices, or one (batch, head) slice of an
                                 input or output is 4 GiB or more */
#define ATTN_ERR_HEAD_DIM -3  /* D is not a supported head dimension */
#define ATTN_ERR_SCALE -4     /* scale is NaN or infinite */
#define ATTN_ERR_LAUNCH -5    /* the HIP launch failed (see attn_last_hip_error) */
#define ATTN_ERR_WORKSPACE -6 /* workspace NULL or smaller than required */
#define ATTN_ERR_ALIAS -7     /* an output buffer overlaps another buffer */
#define ATTN_ERR_SPLITS -8    /* splits < 1 */
#define ATTN_ERR_SCRATCH -9   /* attn_fwd_decode_noalloc: the call needs more than
                                 ATTN_DECODE_NOALLOC_SCRATCH_BYTES of workspace */

/* Capacity of the static device scratch array behind attn_fwd_decode_noalloc
   (32 MiB per GPU). */
#define ATTN_DECODE_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)

/*
 * Fused forward: one kernel, scores kept on chip.
 *   q, k, v : device fp16 [B, H, S, D], read only
 *   o       : device fp16 [B, H, S, D], written
 *   lse     : device fp32 [B, H, S], written
 *   D       : 64, 128 or 512 (attn_head_dim_supported tells)
 *   stream  : a hipStream_t (NULL = the default stream)
 */
int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
             int B, int H, int S, int D, int causal, float scale, void* stream);

/*
 * Unfused three-kernel forward, kept as an ablation of the fused path: the
 * same result computed as the three-branch pipeline QK -> softmax -> AV with
 * its intermediates in global memory ("An Optimal Mapper Meets a Real GPU",
 * sections "Ground rules" and "The uncomfortable audit": a multi-kernel
 * pipeline with globally addressed workspaces).
 *   kernel 1: S = scale * Q K^T, fp32 [B, H, S, S] (D = 512: one pass over
 *             all 512 head dims; the two passes of option 2 of the STAGE_D.md
 *             notes, the second adding into S, measured slower);
 *   kernel 2: P = softmax rows of S, fp16 [B, H, S, S], and LSE;
 *   kernel 3: O = P V.
 * workspace: device memory of at least attn_fwd_unfused_workspace_bytes(B,H,S)
 * = B*H*S*Sp*6 bytes (Sp = S rounded up to a multiple of 64: S in fp32 and P
 * in fp16), owned by the caller, overwritten.  Other arguments as attn_fwd.
 * Three launches on `stream`, asynchronous like attn_fwd.
 */
size_t attn_fwd_unfused_workspace_bytes(int B, int H, int S);
int attn_fwd_unfused(const void* q, const void* k, const void* v, void* o,
                     float* lse, int B, int H, int S, int D, int causal,
                     float scale, void* workspace, size_t workspace_bytes,
                     void* stream);

/*
 * Split-KV forward, for shapes with few (batch, head) slices and long causal
 * rows, where one workgroup per query tile leaves most of the GPU idle.
 * D = 64 or 128: the decode kernel below with Sq = Sk = S (same arguments,
 * workspace and results as attn_fwd_decode; its chunks are 64-key tiles).
 * D = 512: the key range of every 64-row query tile is cut into
 * chunks of at most C = ceil(ceil(S/32) / splits) 32-key tiles; each chunk is
 * one workgroup that leaves its partial state (its own normalised O in fp16, row
 * max and row sum) in `workspace`, and a second kernel merges the chunks of
 * each row in chunk order (deterministic).  The merge over DISJOINT key sets
 * is exact up to rounding (STAGE_D.md notes, section "2. External k_sub Merge
 * is Mathematically Impossible": outputs over different token sets combine
 * through their weights); the partial write, re-read and reduction are the
 * split-k costs that "An Optimal Mapper Meets a Real GPU" (section
 * "Experiment one: ten mappings, forty handwritten kernels") says must be
 * paid.  Query tiles with a single chunk are written directly; splits = 1
 * gives the fused result bit for bit.
 *   D         : 64, 128 or 512 (else ATTN_ERR_HEAD_DIM)
 *   splits    : >= 1 (else ATTN_ERR_SPLITS)
 *   workspace : device memory of at least
 *               attn_fwd_splitkv_workspace_bytes(B, H, S, D, causal, splits)
 *               bytes, owned by the caller and overwritten; may be NULL when
 *               that size is 0 (no query tile is split).
 * Other arguments as attn_fwd.  One or two launches on `stream`,
 * asynchronous like attn_fwd.
 */
size_t attn_fwd_splitkv_workspace_bytes(int B, int H, int S, int D, int causal, int splits);
int attn_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse,
                     int B, int H, int S, int D, int causal, float scale, int splits,
                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * Decode form: Sq query rows against Sk keys, e.g. a few new tokens against a
 * long key/value cache (the decode kernel of "Validating Memory-Optimal
 * Transformer Kernels on Real Hardware", section 5).
 *   q, o : device fp16 [B, H, Sq, D]       k, v : device fp16 [B, H, Sk, D]
 *   lse  : device fp32 [B, H, Sq]
 *   D    : 64 or 128 (else ATTN_ERR_HEAD_DIM)
 *   causal != 0 aligns the mask bottom-right: query i is position
 *     i + Sk - Sq of the sequence, so key j is visible iff j <= i + Sk - Sq
 *     (with Sq = Sk this is attn_fwd's mask).  It needs Sq <= Sk, else
 *     ATTN_ERR_SHAPE (the first rows would see no key).
 *   splits : >= 1 (else ATTN_ERR_SPLITS).  The key range of every 64-row
 *     query tile is cut into chunks of at most ceil(ceil(Sk/64) / splits)
 *     64-key tiles, one workgroup each; chunks leave partial states in
 *     `workspace` and a second kernel merges them in chunk order
 *     (deterministic; exact up to rounding because the key sets are
 *     disjoint).  Query tiles with one chunk are written directly.
 *   workspace : device memory of at least attn_fwd_decode_workspace_bytes(...)
 *     bytes, owned by the caller and overwritten; may be NULL when that size
 *     is 0.
 * One or two launches on `stream`, asynchronous like attn_fwd.
 */
size_t attn_fwd_decode_workspace_bytes(int B, int H, int Sq, int Sk, int D, int causal,
                                       int splits);
int attn_fwd_decode(const void* q, const void* k, const void* v, void* o, float* lse,
                    int B, int H, int Sq, int Sk, int D, int causal, float scale, int splits,
                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * attn_fwd_decode for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments, results (bit for bit) and launches as attn_fwd_decode,
 * without the workspace: the chunks' partial states go to a static device
 * array of ATTN_DECODE_NOALLOC_SCRATCH_BYTES that each GPU holds from the
 * library's first use of it until the process ends.  Nothing is allocated
 * and nothing freed.
 *   - A call needing more than ATTN_DECODE_NOALLOC_SCRATCH_BYTES (see
 *     attn_fwd_decode_workspace_bytes) returns ATTN_ERR_SCRATCH before any
 *     launch.
 *   - All calls on one GPU share its array.  Calls whose execution overlaps
 *     on one GPU (e.g. on two unordered streams) race on it and give wrong
 *     results; calls ordered on one stream are safe.
 *   - The first call on a device looks up the array's device address (a
 *     HIP symbol query, no allocation); its failure is ATTN_ERR_LAUNCH.
 */
int attn_fwd_decode_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                            int B, int H, int Sq, int Sk, int D, int causal, float scale,
                            int splits, void* stream);

/*
 * Backward of attn_fwd for D = 64, 128 or 512: the gradients of L = sum(dO * O)
 * with respect to q, k and v ("Validating Memory-Optimal Transformer Kernels
 * on Real Hardware", abstract and section 4, which measures this backward and
 * its atomic-free rewrite):
 *   P  = exp(scale Q K^T + mask - LSE)       (recomputed, never stored)
 *   dV = P^T dO
 *   dS = P * (dO V^T - rowsum(dO * O))
 *   dQ = scale dS K,   dK = scale dS^T Q
 *
 *   q, k, v, o, dout : fp16 [B, H, S, D], device; o and lse are the outputs of
 *                      attn_fwd for the same q, k, v, causal and scale
 *   lse              : fp32 [B, H, S], device (natural log)
 *   dq, dk, dv       : fp16 [B, H, S, D], device, written; they must not
 *                      overlap each other or any input
 *   workspace        : device memory of at least
 *                      attn_bwd_workspace_bytes_d(B, H, S, D) bytes, owned
 *                      by the caller and overwritten: for D = 64, 128 one
 *                      float per row (= attn_bwd_workspace_bytes(B, H, S));
 *                      for D = 512 the materialised intermediates,
 *                      B H (14 S Sp + 4 S) bytes with Sp = S rounded up to 64
 * Accumulation is fp32; P and dS are rounded to fp16 before the products
 * that consume them.  No atomics, so the outputs are deterministic.
 * D = 64, 128: two launches (P recomputed, never stored).  D = 512: the
 * n x n scores and score gradients (S, dP in fp32; dS, P^T, dS^T in fp16)
 * are stored in the workspace and re-read by MFMA products, nine launches
 * (the same section of the paper measures this storing trade).  All on
 * `stream`, asynchronous like attn_fwd.  Returns the same status codes as
 * attn_fwd (ATTN_ERR_HEAD_DIM for D other than 64, 128 or 512,
 * ATTN_ERR_WORKSPACE for a missing or short workspace).
 */
size_t attn_bwd_workspace_bytes(int B, int H, int S);
size_t attn_bwd_workspace_bytes_d(int B, int H, int S, int D);
int attn_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
             const void* dout, void* dq, void* dk, void* dv, int B, int H, int S, int D,
             int causal, float scale, void* workspace, size_t workspace_bytes, void* stream);

/* 1 if attn_fwd accepts head dimension D, else 0. */
int attn_head_dim_supported(int D);

/* Static text for a status code; never NULL. */
const char* attn_status_string(int status);

/* The hipError_t of this thread's last ATTN_ERR_LAUNCH (0 if none). */
int attn_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_H */
