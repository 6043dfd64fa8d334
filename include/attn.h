/*
 * attn.h -- C ABI of the MI355X (gfx950) fused attention library (libattn.so):
 * forward, split-KV decoding, backward and MLA decoding, and Mamba2
 * ChunkScan. Plain C types only; no C++ or framework types cross it.
 *
 * The operation (PipeThreader, OSDI'25 summary page, "FlashAttention-3"
 * paragraph and Fig 7; "PipeThreader and TileLang" page, section 4.1): for
 * every batch b and head h, with inputs Q, K, V,
 *     S = scale * Q K^T            (optionally causally masked)
 *     P = softmax(S) row by row,   O = P V,
 * computed in one fused kernel that streams K/V blocks (load_k, load_v),
 * multiplies (mma_qk, mma_pv) and keeps an online softmax with output
 * rescaling, so the N x N matrix never exists. The kernel also returns the
 * per-row log-sum-exp of the scaled logits.
 *
 * Readings where the pages are silent (stated once, used by every entry):
 *   - scale multiplies q.k before the softmax; callers usually pass
 *     1/sqrt(d) rounded to float32;
 *   - causal != 0: key j is visible to query i iff j <= i (square,
 *     top-left aligned, diagonal included); masked pairs get zero weight;
 *   - lse[i] = ln sum_{j visible} exp(scale * q_i . k_j)   (natural log).
 */
#ifndef ATTN_H
#define ATTN_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. Every entry point validates its arguments before any HIP
 * call; on a nonzero return nothing was launched and no output was written. */
enum attn_status {
  ATTN_OK = 0,
  ATTN_ERR_NULL_PTR = 1,   /* q, k, v, out or lse is NULL while B*H*N > 0        */
  ATTN_ERR_BAD_SHAPE = 2,  /* B, H or N negative, an element count overflows, or
                              (attn_fwd_variant / attn_variant_info) a variant id
                              out of range or serving another head dimension   */
  ATTN_ERR_HEAD_DIM = 3,   /* d is not a supported head dimension                 */
  ATTN_ERR_BAD_SCALE = 4,  /* scale is NaN or infinite                            */
  ATTN_ERR_MISALIGNED = 5, /* a pointer is misaligned: 16 bytes for every buffer
                              except lse (and the backward's lse), 4 bytes       */
  ATTN_ERR_HIP = 6,        /* the HIP runtime reported an error at launch         */
  /* 7 is not used */
  ATTN_ERR_WORKSPACE = 8,  /* decoding, backward, MLA decoding: workspace smaller
                              than the entry's workspace-size function reports  */
  ATTN_ERR_TOO_LARGE = 9   /* attn_fwd_decode_static: the shape needs more scratch
                              than attn_decode_static_max_bytes()               */
};

/*
 * attn_fwd -- fused attention forward on one GPU.
 *
 *   q, k, v : device pointers, bf16, dense row-major [B][H][N][d]
 *   out     : device pointer, float32, [B][H][N][d]; fully overwritten
 *   lse     : device pointer, float32, [B][H][N];   fully overwritten
 *   B, H, N : batch, heads, sequence length (N >= 1 any value; tails masked)
 *   d       : head dimension, one of 64, 128, 256
 *   causal  : 0 = every key visible, nonzero = key j visible to query i iff j <= i
 *   scale   : finite float32 multiplier of q.k (zero and negative values
 *             included: a zero scale gives uniform weights over the visible
 *             keys)
 *   stream  : hipStream_t to enqueue on (NULL = the default stream)
 *
 * Alignment: q, k, v and out 16 bytes, lse 4 bytes (else ATTN_ERR_MISALIGNED).
 * Ownership: the caller owns all five buffers; the library never allocates,
 * frees, copies or synchronises. The call is asynchronous: it enqueues the
 * kernel on `stream` and returns; device-side faults surface at the caller's
 * next synchronisation. B*H*N == 0 returns ATTN_OK and launches nothing.
 * Preconditions not checked: out and lse do not alias q, k, v or each other;
 * each buffer holds the stated number of elements.
 * Thread-safe and stateless: calls on different streams may run concurrently.
 */
int attn_fwd(const void* q, const void* k, const void* v, float* out, float* lse, int B, int H,
             int N, int d, int causal, float scale, void* stream);

/* Human-readable text for a status code (static storage; never NULL). */
const char* attn_strerror(int status);

/*
 * Kernel variants, for the tile/depth sweep (PipeThreader summary page,
 * "Profiler" paragraph and Fig 9: candidate schedules are filtered by an
 * on-chip memory check and the final one is chosen by measured whole-program
 * latency; "PipeThreader and TileLang" page, section 7: the autotuner runs a
 * correctness check before it profiles).
 *
 * attn_num_variants : number of compiled variants.
 * attn_variant_name : short description "d128_bm256_bn64_w8_..."; NULL if id
 *                     is out of range.
 * attn_variant_info : fills head_dim, block_m (query rows per workgroup),
 *                     block_n (keys per pipeline stage), waves per workgroup,
 *                     and lds_bytes; returns ATTN_ERR_BAD_SHAPE for a bad id.
 * attn_fwd_variant  : attn_fwd forced onto variant `id`; same arguments,
 *                     validation and semantics, plus ATTN_ERR_BAD_SHAPE when
 *                     id is out of range or the variant does not serve head
 *                     dimension d.
 * attn_default_variant : the variant attn_fwd picks for (d, causal), or -1.
 */
int attn_num_variants(void);
const char* attn_variant_name(int id);
int attn_variant_info(int id, int* head_dim, int* block_m, int* block_n, int* waves,
                      int* lds_bytes);
int attn_default_variant(int d, int causal);
int attn_fwd_variant(int id, const void* q, const void* k, const void* v, float* out, float* lse,
                     int B, int H, int N, int d, int causal, float scale, void* stream);

/*
 * Split-KV decoding (PipeThreader summary page, evaluation setup: the
 * FlashDecoding microbenchmark of the LLAMA3 models at (BS, SEQ) = (1, 1)
 * and (32, 1); the same operation as attn_fwd with a rectangular score
 * matrix). For every batch b and head h, Nq new query rows attend to a cache
 * of Nkv keys, every query seeing every key:
 *     S = scale * Q K^T  (Nq x Nkv),   O = softmax(S) V,
 *     lse[i] = ln sum_j exp(S_ij).
 * The keys of each (b, h) are split into chunks processed in parallel, each
 * giving a normalised partial (O_c, LSE_c) in the workspace; a second kernel
 * merges them: LSE = ln sum_c exp(LSE_c), O = sum_c exp(LSE_c - LSE) O_c.
 *
 *   q       : device, bf16, [B][H][Nq][d]
 *   k, v    : device, bf16, [B][H][Nkv][d]
 *   out     : device, float32, [B][H][Nq][d]; fully overwritten
 *   lse     : device, float32, [B][H][Nq];    fully overwritten
 *   Nq >= 0, Nkv >= 1 whenever B*H*Nq > 0; d one of 64, 128, 256
 *   scale   : finite float32 multiplier of q.k (as for attn_fwd)
 *   workspace, workspace_bytes : device scratch owned by the caller, 16-byte
 *             aligned, at least the size attn_decode_workspace_size reports
 *             for the same shape (else ATTN_ERR_WORKSPACE); its contents on
 *             entry do not matter and are overwritten
 *   stream  : hipStream_t (NULL = default stream); two kernels are enqueued
 *
 * Grouped K/V heads (G query heads sharing one K/V head, as in the LLAMA3
 * models): with k, v of Hkv = H / G heads, [B][Hkv][Nkv][d], query head h
 * reads K/V head h / G. The G query heads of a group are adjacent in q, out
 * and lse, so that operation is exactly this call with H replaced by Hkv and
 * Nq by G * Nq, on the same five buffers (and a workspace sized for that
 * shape); each K/V head is then read once per group.
 *
 * Same ownership, validation and asynchrony rules as attn_fwd; the library
 * allocates nothing. Calls sharing one workspace must not overlap.
 *
 * attn_decode_workspace_size : workspace bytes for a shape (0 when
 *             B*H*Nq == 0); same shape errors as attn_fwd_decode.
 */
int attn_decode_workspace_size(int B, int H, int Nq, int Nkv, int d, size_t* bytes);
int attn_fwd_decode(const void* q, const void* k, const void* v, float* out, float* lse, int B, int H,
                    int Nq, int Nkv, int d, float scale, void* workspace, size_t workspace_bytes,
                    void* stream);

/*
 * attn_fwd_decode_static -- attn_fwd_decode for callers that cannot allocate
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same operation, arguments and kernels without the
 * workspace. The chunk partials go to a fixed device array of
 * attn_decode_static_max_bytes() bytes (16 MiB) inside the library, one per
 * GPU, held until the process ends; the entry calls no allocator. A shape
 * whose attn_decode_workspace_size exceeds that returns ATTN_ERR_TOO_LARGE
 * before any HIP call. The array is looked up for the current device on the
 * first call there (hipGetSymbolAddress; make the stream's device current).
 * Every call on one GPU shares that GPU's array: calls that overlap on one
 * GPU (other streams, other threads) race and must be serialised by the
 * caller. No part of the array needs clearing between calls.
 */
size_t attn_decode_static_max_bytes(void);
int attn_fwd_decode_static(const void* q, const void* k, const void* v, float* out, float* lse, int B, int H,
                           int Nq, int Nkv, int d, float scale, void* stream);

/*
 * Attention backward (the backward pass the Twill software-pipelining
 * write-up schedules in its section 3.2; the pages do not restate it, so it is
 * the derivative of attn_fwd's definition). With dO the gradient of the loss
 * with respect to out (lse is taken to carry no gradient), per (b, h):
 *     P_ij  = exp(scale * q_i.k_j - lse_i) on visible pairs, else 0
 *     D_i   = sum_c dO_ic out_ic,      dS_ij = P_ij (dO_i.v_j - D_i)
 *     dv_j  = sum_i P_ij dO_i
 *     dk_j  = scale * sum_i dS_ij q_i,  dq_i = scale * sum_j dS_ij k_j
 *
 *   q, k, v, dout : device, bf16, [B][H][N][d]
 *   out, lse      : device, float32, the attn_fwd outputs for the same q, k,
 *                   v, causal and scale ([B][H][N][d] and [B][H][N])
 *   dq, dk, dv    : device, float32, [B][H][N][d]; fully overwritten
 *   d             : 64, 128 or 256
 *   causal, scale : as for attn_fwd
 *   workspace, workspace_bytes : device scratch owned by the caller, 16-byte
 *                   aligned, at least attn_bwd_workspace_size bytes (else
 *                   ATTN_ERR_WORKSPACE); its contents on entry do not matter
 *   stream        : hipStream_t (NULL = default stream); three kernels are
 *                   enqueued
 *
 * Same ownership, validation and asynchrony rules as attn_fwd; the library
 * allocates nothing and the result is deterministic (no atomics). Calls
 * sharing one workspace must not overlap. B*H*N == 0 returns ATTN_OK.
 *
 * attn_bwd_workspace_size : workspace bytes for a shape (256 bytes per 32
 *                   query rows of each head); same shape errors as attn_bwd.
 */
int attn_bwd_workspace_size(int B, int H, int N, int d, size_t* bytes);
int attn_bwd(const void* q, const void* k, const void* v, const float* out, const float* lse,
             const void* dout, float* dq, float* dk, float* dv, int B, int H, int N, int d, int causal,
             float scale, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Mamba2 ChunkScan (PipeThreader summary page, "Running example: Mamba2" and
 * Fig 6(a); the linear-attention microbenchmark derived from Mamba2-1.3B).
 * The sequence is cut into chunks of L steps; inside a chunk, cb is scaled
 * by the exponential decay built from dA and by dt, and its product with x
 * accumulates into the output. For step s (chunk c = s / L, m = s - cL):
 *     out[b][s][h][:] = sum_{k=0..m} cb[b][c][m][k]
 *                        * exp(dA_cumsum[b][h][c][m] - dA_cumsum[b][h][c][k])
 *                        * dt[b][h][c][k] * x[b][cL + k][h][:]
 * (only earlier-or-same steps of the same chunk; the contribution carried
 * across chunks by the state is a separate operation).
 *
 *   x          : device, bf16, [B][S][H][P]
 *   cb         : device, bf16, [B][nc][L][L]  (nc = ceil(S / L); one group,
 *                shared by all heads)
 *   dt, dA_cumsum : device, float32, [B][H][nc][L] (dA_cumsum: the running
 *                sum of dA within each chunk)
 *   out        : device, float32, [B][S][H][P]; fully overwritten
 *   P          : 64 (else ATTN_ERR_HEAD_DIM); L a multiple of 32 in [32, 256]
 *   stream     : hipStream_t (NULL = default stream)
 *
 * Same ownership, validation and asynchrony rules as attn_fwd (all five
 * pointers 16-byte aligned). B*S == 0 returns ATTN_OK and launches nothing.
 */
int chunk_scan(const void* x, const void* cb, const float* dt, const float* dA_cumsum, float* out, int B, int S,
               int H, int P, int L, void* stream);

/*
 * MLA decoding (multi-head latent attention in the absorbed form; the
 * decoding operator the PipeThreader summary page cites in its "Discussion"
 * paragraph, written there in about 80 lines against 500-plus by hand). Every query head of sequence b attends to one shared
 * cache of N latent rows of 576 values (512 latent + 64 rotary); a row's
 * first 512 values are its value:
 *     s_hj = scale * q_h . kv_j (576 products),  out_h = softmax_j(s_h) kv[:, 0:512],
 *     lse_h = ln sum_j exp(s_hj).
 *
 *   q   : device, bf16, [B][H][576];   kv : device, bf16, [B][N][576]
 *   out : device, float32, [B][H][512]; lse : device, float32, [B][H]; fully overwritten
 *   H   : a multiple of 64 (else ATTN_ERR_BAD_SHAPE); N >= 1 when B*H > 0
 *   scale : finite float32 (as for attn_fwd)
 *   workspace, workspace_bytes : device scratch owned by the caller, 16-byte
 *           aligned, at least mla_decode_workspace_size bytes (else
 *           ATTN_ERR_WORKSPACE); contents on entry do not matter
 *   stream : hipStream_t (NULL = default stream); two kernels are enqueued
 *
 * Same ownership, validation and asynchrony rules as attn_fwd_decode; the
 * library allocates nothing; calls sharing one workspace must not overlap.
 */
int mla_decode_workspace_size(int B, int H, int N, size_t* bytes);
int mla_decode(const void* q, const void* kv, float* out, float* lse, int B, int H, int N, float scale,
               void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_H */
