/*
 * fa.h — C ABI of libfa: exact scaled-dot-product attention on AMD Instinct
 * MI355X (gfx950), computed tile by tile with the online-softmax recurrence so
 * that the N x N score matrix never reaches device memory.
 *
 * Definition (handsonai.io "DL101 chapter 9", section 1.1 Key/Value Caching):
 *   O = softmax(scale * Q K^T [+ causal mask]) V,   scale normally 1/sqrt(d).
 * Recurrence (same page, section 3.3 FlashAttention; holysheep.ai Flash
 * Attention article, section 2.1 Online Softmax): a running row max m and
 * denominator l; when a new K/V block arrives the partial output and l are
 * rescaled by exp(m_old - m_new); one division by l at the end.
 * Backward (thienlv.com glossary "Flash Attention Là Gì?", section "Ba Kỹ Thuật
 * Chính", item 2): P is recomputed from Q, K and the saved logsumexp instead of
 * being stored.
 * Grouped K/V heads (DL101 chapter 9, sections 3.1 MQA and 3.2 GQA): query head
 * h reads K/V head h / (Hq / Hkv).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every tensor pointer is a DEVICE pointer to a contiguous row-major tensor,
 *   head dimension fastest: q/o/dq/do are [B][Hq][Nq][d]; k/v/dk/dv are
 *   [B][Hkv][Nk][d]; lse is [B][Hq][Nq] float32.
 * - dtype FA_BF16: q, k, v, o, do are bfloat16 (raw 16-bit storage); the
 *   kernels compute QK^T and PV on bf16 matrix cores with float32 accumulation
 *   and keep the softmax statistics in float32.  FA_F32: all of them are
 *   float32 and every step is float32.
 * - lse (logsumexp) of query row i is the natural log of sum_j exp(scale *
 *   q_i . k_j) over the keys row i may see.  A row that sees no key gets
 *   O = 0 and lse = -inf.
 * - causal != 0: key j is visible to query i iff j <= i + (Nk - Nq)
 *   (bottom-right aligned; equal to the lower triangle when Nq == Nk).
 *   Causal with Nq > Nk is rejected (rows without keys would be the norm).
 * - d must be 64 or 128.  Hq must be a multiple of Hkv.  All sizes >= 1 unless
 *   stated.  Tensor sizes are limited to 2^31 elements each.
 * - stream is a hipStream_t (NULL = the default stream).  Every call only
 *   enqueues work on that stream and returns; nothing is synchronised.
 * - Ownership: the caller allocates and owns every buffer, workspaces
 *   included.  The library allocates nothing, frees nothing and keeps no
 *   pointer after returning.  Its only global state is a per-device cache of
 *   facts looked up on first use (compute-unit count, LDS size, each kernel's
 *   dynamic-LDS attribute), filled idempotently and safe to race on, so calls
 *   on different streams or threads are independent; and the fixed device
 *   scratch of fa_decode_noalloc (declared below), whose calls on one device
 *   share it.  Outputs are fully overwritten.
 * - Errors: host-visible arguments are checked before anything is enqueued;
 *   on any error nothing is launched and a status != FA_OK is returned.  A
 *   failed kernel launch returns FA_ERR_HIP.  No exception crosses the ABI.
 */
#ifndef FA_H
#define FA_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FA_ABI_VERSION 1

typedef enum {
    FA_OK = 0,
    FA_ERR_NULL_PTR = 1,     /* a required pointer is NULL                      */
    FA_ERR_SHAPE = 2,        /* a size < 1, Hq % Hkv != 0, causal with Nq > Nk,  */
                             /* or a tensor above 2^31 elements                  */
    FA_ERR_DTYPE = 3,        /* dtype / grad_dtype not one of fa_dtype_t, or     */
                             /* FA_BF16 gradients asked of FA_F32 inputs         */
    FA_ERR_UNSUPPORTED = 4,  /* head dimension d other than 64 or 128           */
    FA_ERR_WORKSPACE = 5,    /* workspace NULL or smaller than the query says    */
    FA_ERR_HIP = 6,          /* the HIP runtime refused a launch                 */
    FA_ERR_ARG = 7,          /* scale not finite or not > 0                       */
    FA_ERR_SCRATCH = 8       /* fa_decode_noalloc: the shape needs more scratch   */
                             /* than its fixed device buffer holds                */
} fa_status_t;

typedef enum {
    FA_F32 = 0,
    FA_BF16 = 1,
    /* Not dtypes: these two give the type the range of a 32-bit int, so any
     * int a caller passes is a value of fa_dtype_t and an unknown one reaches
     * the FA_ERR_DTYPE check (with only 0 and 1 listed, C++ would make
     * reading 7 through this type undefined). */
    FA_DTYPE_RANGE_MIN_ = -0x7FFFFFFF - 1,
    FA_DTYPE_RANGE_MAX_ = 0x7FFFFFFF
} fa_dtype_t;

/* FA_ABI_VERSION of the built library. */
int fa_abi_version(void);

/* Static string naming a status code (never NULL). */
const char* fa_status_str(int status);

/*
 * Forward pass.
 *   q [B,Hq,Nq,d], k/v [B,Hkv,Nk,d] in dtype; o [B,Hq,Nq,d] in dtype (written);
 *   lse [B,Hq,Nq] float32 (written; needed by fa_bwd).
 */
fa_status_t fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                   int B, int Hq, int Hkv, int Nq, int Nk, int d,
                   fa_dtype_t dtype, float scale, int causal, void* stream);

/* Bytes of device workspace fa_bwd needs: two float32 per query row
 * (D_i = dO_i . O_i and lse_i log2 e), i.e. linear in Nq, never Nq x Nk. */
size_t fa_bwd_workspace_bytes(int B, int Hq, int Nq, int d);

/*
 * Backward pass: gradients of sum(O * dO) with respect to q, k, v.
 *   q, k, v, o (the forward output), dO in dtype, lse from fa_fwd;
 *   dq [B,Hq,Nq,d], dk/dv [B,Hkv,Nk,d] written in grad_dtype (FA_F32 is the
 *   default choice; FA_BF16 rounds the float32 result to bfloat16 and is
 *   accepted for FA_BF16 inputs only: FA_F32 inputs with FA_BF16 gradients
 *   return FA_ERR_DTYPE).  With
 *   grouped heads, dk/dv of a K/V head are the sums over its query heads.
 *   The result is deterministic (no atomics): repeated calls give the same bits.
 *   D_i = dO_i . O_i is formed from the o passed in, so the rounding of a
 *   stored (bf16) O enters the gradients: with delta_i = dO_i . (O_i -
 *   O_exact_i), |delta_i| <= 2^-9 |dO_i| |O_i| for bf16 O, dQ_i carries the
 *   extra term -scale delta_i sum_j P_ij k_j and dK_j the term -scale sum_i
 *   P_ij delta_i q_i (dV none).  These stay at the gradients' own bf16 level
 *   unless the values a query attends to are nearly equal (dP_ij - D_i then
 *   nearly cancels): with values equal up to a 2^-5 spread they are ~7% of
 *   dQ and ~6% of dK.
 *   workspace: device buffer of at least fa_bwd_workspace_bytes(...) bytes.
 */
fa_status_t fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dO,
                   const float* lse, void* dq, void* dk, void* dv, fa_dtype_t grad_dtype,
                   int B, int Hq, int Hkv, int Nq, int Nk, int d,
                   fa_dtype_t dtype, float scale, int causal,
                   void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of device workspace fa_decode needs for its partial results (float32
 * partial outputs and logsumexps of the pieces of each row that the streaming
 * waves computed, plus B + 1 integers).  Independent of Nmax; 0 for shapes
 * fa_decode would reject (Hq not a multiple of Hkv, non-positive sizes). */
size_t fa_decode_workspace_bytes(int B, int Hq, int Hkv, int Nmax, int d);

/*
 * Decode: one new query token per (b, h) against a KV cache.
 *   q [B,Hq,1,d]; k_cache/v_cache [B,Hkv,Nmax,d]; seqlens [B] int32 on the
 *   DEVICE: row b sees keys j < seqlens[b] (values are clamped to [0, Nmax];
 *   the cache beyond seqlens[b] is never read into the result and may hold
 *   anything, NaN included).  o [B,Hq,1,d] in dtype; lse [B,Hq] float32.
 *   seqlens[b] == 0 gives o = 0 and lse = -inf for that sequence.
 *   workspace: device buffer of at least fa_decode_workspace_bytes(...) bytes.
 */
fa_status_t fa_decode(const void* q, const void* k_cache, const void* v_cache,
                      const int* seqlens, void* o, float* lse,
                      int B, int Hq, int Hkv, int Nmax, int d,
                      fa_dtype_t dtype, float scale,
                      void* workspace, size_t workspace_bytes, void* stream);

/* Size of the fixed device scratch of fa_decode_noalloc (per device). */
#define FA_DECODE_NOALLOC_SCRATCH_BYTES (64u << 20)

/*
 * fa_decode without a workspace argument, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation.  Arguments, results and errors as fa_decode; the
 * partial results fa_decode keeps in the caller's workspace live instead in a
 * fixed buffer of FA_DECODE_NOALLOC_SCRATCH_BYTES (64 MiB) per device, which
 * the library reserves when its code is loaded on a device and holds until the
 * process ends.  The call itself allocates nothing and calls no allocating
 * routine.  Shapes whose fa_decode_workspace_bytes(B, Hq, Hkv, Nmax, d)
 * exceeds the buffer are refused with FA_ERR_SCRATCH (the decode workload
 * B16 Hq32 Hkv8 d128 needs 4.3 MiB; at d = 128 the buffer holds B * Hkv up to
 * 30465 with 4 query heads per K/V head, 14208 with 8, 2016 with 32; at
 * d = 64 about twice that).
 * Every call on a device shares that device's buffer, and its contents carry
 * over from call to call (nothing in it needs to start at zero), so calls
 * that can overlap on one device (concurrent streams, threads) race and must
 * be serialised by the caller; calls on different devices are independent.
 */
fa_status_t fa_decode_noalloc(const void* q, const void* k_cache, const void* v_cache,
                              const int* seqlens, void* o, float* lse,
                              int B, int Hq, int Hkv, int Nmax, int d,
                              fa_dtype_t dtype, float scale, void* stream);

/* Bytes of device workspace fa_decode_chunk needs: the same partial results
 * as fa_decode over Hq * Nq query rows.  0 for shapes fa_decode_chunk would
 * reject. */
size_t fa_decode_chunk_workspace_bytes(int B, int Hq, int Hkv, int Nq, int Nmax, int d);

/*
 * Chunk decode: Nq new query tokens per (b, h) against a KV cache that already
 * holds their keys and values, as when a large model checks several drafted
 * tokens in one pass or a prompt is prefilled in chunks (DL101 chapter 9,
 * section 1.2 Speculative Decoding, with the rule of section 1.1: token t
 * attends to the keys up to and including its own position).
 *   q [B,Hq,Nq,d]; k_cache/v_cache [B,Hkv,Nmax,d]; seqlens [B] int32 on the
 *   DEVICE (clamped to [0, Nmax]): sequence b's cache holds seqlens[b] keys,
 *   the last Nq of which belong to the new tokens.  o [B,Hq,Nq,d] in dtype;
 *   lse [B,Hq,Nq] float32.
 *   causal != 0: token t (0 <= t < Nq) sees keys j < seqlens[b] - (Nq - 1 - t),
 *   i.e. bottom-right aligned to the sequence's own length; a token whose
 *   range is empty (seqlens[b] < Nq - t) gets o = 0 and lse = -inf.
 *   causal == 0: every token sees keys j < seqlens[b].
 *   1 <= Nq <= 64; Nq == 1 is fa_decode.
 *   workspace: device buffer of at least fa_decode_chunk_workspace_bytes(...)
 *   bytes.  Other conventions as fa_decode.
 */
fa_status_t fa_decode_chunk(const void* q, const void* k_cache, const void* v_cache,
                            const int* seqlens, void* o, float* lse,
                            int B, int Hq, int Hkv, int Nq, int Nmax, int d,
                            fa_dtype_t dtype, float scale, int causal,
                            void* workspace, size_t workspace_bytes, void* stream);

/*
 * FP8 forward: exact attention of FP8 inputs (thienlv.com glossary "Flash
 * Attention Là Gì?", section "Flash Attention 2 và 3": FlashAttention-3 adds
 * FP8 support; format and scaling are this library's reading).
 *   q [B,Hq,Nq,d], k/v [B,Hkv,Nk,d]: OCP FP8 E4M3 codes (one byte each; 1 sign,
 *   4 exponent bits of bias 7, 3 mantissa bits, max 448, S.1111.111 = NaN);
 *   the value of an element is its E4M3 value times the tensor's descale
 *   (descale_q, descale_k, descale_v: finite, > 0).  o [B,Hq,Nq,d] bfloat16;
 *   lse [B,Hq,Nq] float32 = ln sum_j exp(scale * q_i . k_j) of those values.
 *   Both products run on FP8 matrix cores with float32 accumulation; the
 *   softmax weights are rounded to E4M3 (as 2^8 P, round to nearest even)
 *   for the second product, so O differs from exact attention by at most
 *   2^-4 max_j |v_j| (plus the bf16 rounding of O); lse does not see that
 *   rounding.  Other conventions as fa_fwd (causal bottom-right, GQA,
 *   d = 64 or 128).
 */
fa_status_t fa_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse,
                       int B, int Hq, int Hkv, int Nq, int Nk, int d,
                       float descale_q, float descale_k, float descale_v, float scale, int causal,
                       void* stream);

/* Bytes of device workspace fa_decode_paged needs (as fa_decode_chunk; it
 * does not depend on the cache).  0 for shapes fa_decode_paged would reject. */
size_t fa_decode_paged_workspace_bytes(int B, int Hq, int Hkv, int Nq, int d);

/*
 * Chunk decode against a paged KV cache: the keys and values of all sequences
 * live in a pool of fixed-size pages, and a block table names the page that
 * holds each run of page_size consecutive keys of a sequence (the cache layout
 * of vLLM's PagedAttention, which unite.ai "What is FlashAttention", section
 * "Nguồn chính để nghiên cứu FlashAttention", names as where the method meets
 * serving; the pages define nothing further, so the layout below is this
 * library's).  The result is exactly fa_decode_chunk's on the contiguous cache
 * the pages spell out.
 *   k_pages/v_pages [num_pages][Hkv][page_size][d] (each page holds page_size
 *   consecutive keys of every K/V head); block_table [B][max_pages] int32 on
 *   the DEVICE: key j of sequence b is row j % page_size of page
 *   block_table[b][j / page_size].  Entries are clamped to [0, num_pages) (an
 *   out-of-range entry gives wrong values, never an out-of-bounds read);
 *   entries past a sequence's last page are never read.
 *   seqlens [B] int32 on the DEVICE, clamped to [0, max_pages * page_size].
 *   q [B,Hq,Nq,d] (Nq = 1 is plain decode, up to 64 as fa_decode_chunk), o
 *   [B,Hq,Nq,d] in dtype, lse [B,Hq,Nq] float32; causal as fa_decode_chunk.
 *   page_size must be a multiple of 32 (FA_ERR_UNSUPPORTED otherwise).
 *   workspace: at least fa_decode_paged_workspace_bytes(...) bytes.
 */
fa_status_t fa_decode_paged(const void* q, const void* k_pages, const void* v_pages,
                            const int* block_table, const int* seqlens, void* o, float* lse,
                            int B, int Hq, int Hkv, int Nq, int num_pages, int page_size,
                            int max_pages, int d, fa_dtype_t dtype, float scale, int causal,
                            void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FA_H */
