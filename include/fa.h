/*
 * fa.h - C ABI of the fused exact-attention library (libfa.so) for
 * AMD Instinct MI355X (gfx950).
 *
 * The library computes exact scaled dot-product attention
 *
 *     O = softmax(scale * Q K^T [+ causal mask]) V
 *
 * in one fused, tiled pass with an online softmax: each query row keeps a
 * running maximum, a running sum of exponentials and a rescaled output
 * accumulator, and the N x N score and probability matrices never leave
 * the chip. Sources, cited by page title and section:
 *   - "From Self-Attention to FlashAttention" (wmrh.cn), section 1 (the
 *     standard and flash data flows) and section 2 (online softmax);
 *   - "Flash Attention algorithm design and I/O optimisation" interview
 *     page (algomooc.com), "Positioning" (the result is exact up to
 *     floating-point ordering) and "Core mechanism" (tiling, online
 *     softmax, backward by recomputation from saved row statistics);
 *   - "FlashAttention in ops-transformer" (mhpn.cn), "Core idea",
 *     "Online softmax", "Complete operator" (causal and scale arguments,
 *     workspace query, asynchronous launch on a caller stream),
 *     "Pitfalls" (causal mask; fp32 softmax inside half-precision kernels)
 *     and "A surprise" (the backward keeps forward state).
 *
 * Conventions shared by every entry point
 *   Layout     Q, K, V, O, dO, dQ, dK, dV are contiguous row-major
 *              [B, H, N, D] tensors (batch, head, position, head dim) of the
 *              call's dtype. LSE is contiguous fp32 [B, H, N].
 *   Memory     Every tensor pointer is device memory owned by the caller,
 *              16-byte aligned. The library never allocates, frees or
 *              synchronises, and keeps no state between calls except the
 *              per-thread error text of fa_last_error and the static
 *              scratch array of fa_backward_noalloc.
 *   Stream     Work is enqueued on `stream` (a hipStream_t; NULL means the
 *              default stream) and runs asynchronously; a returned FA_OK
 *              means the launch was accepted.
 *   Causal     A query at position i sees keys 0..i (diagonal included).
 *   Scale      Any finite float; callers usually pass 1/sqrt(D).
 *   Errors     Arguments are validated before any device work. A rejected
 *              call returns a non-zero fa_status, writes nothing and sets
 *              the text returned by fa_last_error. Shapes outside the
 *              supported set return FA_ERR_UNSUPPORTED so the caller can
 *              fall back to another implementation.
 *   Threads    Calls are reentrant; calls that write the same buffers on
 *              different streams race, as any two kernels would.
 */
#ifndef FA_H
#define FA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum fa_dtype {
  FA_FP32 = 0, /* IEEE binary32 */
  FA_FP16 = 1, /* IEEE binary16 */
  FA_BF16 = 2  /* bfloat16 */
} fa_dtype;

typedef enum fa_status {
  FA_OK = 0,
  FA_ERR_INVALID_ARGUMENT = 1, /* null pointer, non-positive size, bad dtype,
                                  non-finite scale, misaligned pointer,
                                  index overflow */
  FA_ERR_UNSUPPORTED = 2,      /* valid request outside the supported set */
  FA_ERR_WORKSPACE = 3,        /* backward workspace missing or too small */
  FA_ERR_HIP = 4               /* the HIP runtime rejected a launch */
} fa_status;

/*
 * fa_forward - fused attention forward.
 *
 * Computes, for every batch b and head h,
 *   O[b,h]   = softmax(scale * Q[b,h] K[b,h]^T [+ causal mask]) V[b,h]
 *   LSE[b,h,i] = ln sum_j exp(scale * Q[b,h,i] . K[b,h,j])  over the keys j
 *                row i may see (natural log)
 * ("From Self-Attention to FlashAttention", sections 1-2; "FlashAttention in
 * ops-transformer", "Core idea" and "Online softmax"). LSE is the row
 * statistic the backward recomputes probabilities from.
 *
 *   q, k, v  in   [B, H, N, D] of `dtype`
 *   o        out  [B, H, N, D] of `dtype`, rounded to nearest even
 *   lse      out  [B, H, N] fp32 (required)
 *   B, H, N  >= 1
 *   D        head dim; supported: 64, 128
 *   scale    finite multiplier of Q K^T
 *   causal   0 = full attention, non-zero = causal (keys 0..i for row i)
 *   dtype    fa_dtype: FA_FP32, FA_FP16 or FA_BF16. Scores, softmax
 *            statistics and the output accumulator are fp32 for every
 *            dtype; for FA_FP16/FA_BF16 the probabilities are rounded to
 *            the dtype only as the operand of the P V product.
 *   stream   hipStream_t or NULL
 *
 * Returns FA_OK, FA_ERR_INVALID_ARGUMENT, FA_ERR_UNSUPPORTED or FA_ERR_HIP.
 */
fa_status fa_forward(const void* q, const void* k, const void* v, void* o, float* lse,
                     int64_t B, int64_t H, int64_t N, int64_t D, float scale, int causal,
                     int dtype, void* stream);

/*
 * fa_forward_dropout - fa_forward with dropout on the attention
 * probabilities (training).
 *
 * The dropout branch of "Flash Attention algorithm design and I/O
 * optimisation" (verification answer), read as the usual attention dropout:
 * P = softmax(scale * Q K^T [masked]) as in fa_forward (LSE is unchanged),
 * each P[i][j] kept or dropped by counter-based random bits, and
 *   O = (P * keep) V / (1 - thr / 256).
 * Element (i, j) of head bh = b * H + h is dropped when byte j % 4 of word
 * i % 4 of Philox4x32-10 (Salmon et al., SC 2011) with counter
 * (j / 4, i / 4, bh, offset) and key (seed mod 2^32, seed / 2^32) is below
 * thr = floor(256 * dropout_p + 0.5): the probability is rounded to a
 * multiple of 1/256. The same (seed, offset) in fa_backward_dropout
 * regenerates the same decisions; nothing is stored.
 *
 *   dropout_p  0 <= p < 255.5/256 (thr = 0 is exactly fa_forward)
 *   seed       any 64-bit value
 *   offset     below 2^32 (e.g. a per-step counter)
 *   dtype      FA_FP16 or FA_BF16 (FA_FP32 returns FA_ERR_UNSUPPORTED)
 *   other arguments as for fa_forward
 *
 * Returns FA_OK, FA_ERR_INVALID_ARGUMENT, FA_ERR_UNSUPPORTED or FA_ERR_HIP.
 */
fa_status fa_forward_dropout(const void* q, const void* k, const void* v, void* o, float* lse,
                             int64_t B, int64_t H, int64_t N, int64_t D, float scale, int causal,
                             int dtype, float dropout_p, uint64_t seed, uint64_t offset,
                             void* stream);

/*
 * fa_forward_gqa - fa_forward (and fa_forward_dropout) with grouped K/V
 * heads in the dense layout: H query heads share H_kv K/V heads, query head
 * h reading K/V head h / (H / H_kv) (MQA: H_kv = 1). Shared K/V heads are one
 * of the factors the decode and prefill gains depend on ("Flash Attention
 * algorithm design and I/O optimisation", "Training and inference value");
 * each query head is still exact attention against its K/V head.
 *
 *   q         in   [B, H, N, D] of `dtype`
 *   k, v      in   [B, H_kv, N, D] of `dtype`
 *   o, lse    out  as for fa_forward
 *   H_kv      divides H (H_kv = H is exactly fa_forward)
 *   dropout_p 0 = no dropout (any dtype); otherwise as for
 *             fa_forward_dropout (FA_FP16 or FA_BF16; the bits of query
 *             head h of batch b are those of head b * H + h)
 *   seed, offset  as for fa_forward_dropout (ignored when dropout_p = 0)
 *   other arguments as for fa_forward
 *
 * Returns FA_OK, FA_ERR_INVALID_ARGUMENT, FA_ERR_UNSUPPORTED or FA_ERR_HIP.
 */
fa_status fa_forward_gqa(const void* q, const void* k, const void* v, void* o, float* lse,
                         int64_t B, int64_t H, int64_t H_kv, int64_t N, int64_t D, float scale,
                         int causal, int dtype, float dropout_p, uint64_t seed, uint64_t offset,
                         void* stream);

/*
 * fa_forward_varlen - fused attention forward over a packed batch of
 * variable-length sequences, with grouped K/V heads (GQA/MQA).
 *
 * The variants named by "Flash Attention algorithm design and I/O
 * optimisation" in its deployment and verification answers: variable-length
 * batches and shared K/V heads. Sequence b is tokens [cu_seqlens[b],
 * cu_seqlens[b+1]) of the packed tensors and attends only within itself (a
 * causal query at position i of its sequence sees positions 0..i). Query
 * head h reads K/V head h / (H / H_kv). Per (sequence, head) the result is
 * that of fa_forward.
 *
 *   q, o        [total, H, D] of `dtype` (token-major, heads interleaved)
 *   k, v        [total, H_kv, D] of `dtype`
 *   lse         out [H, total] fp32, natural log
 *   cu_seqlens  device memory, batch + 1 int32 offsets, caller-owned; the
 *               caller guarantees 0 = cu[0] <= cu[1] <= ... <= cu[batch] =
 *               total and cu[b+1] - cu[b] <= max_seqlen. Offsets outside
 *               [0, total] are clamped and longer sequences truncated to
 *               max_seqlen rows, so no access leaves the tensors; tokens not
 *               covered by any sequence are not written.
 *   batch       number of sequences (>= 1)
 *   max_seqlen  longest sequence, 1 <= max_seqlen <= total
 *   H, H_kv     query and K/V heads; H_kv divides H
 *   D           64 or 128
 *   scale, causal, stream  as for fa_forward
 *   dtype       FA_FP16 or FA_BF16 (FA_FP32 returns FA_ERR_UNSUPPORTED)
 *
 * Returns FA_OK, FA_ERR_INVALID_ARGUMENT, FA_ERR_UNSUPPORTED or FA_ERR_HIP.
 */
fa_status fa_forward_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                            const int32_t* cu_seqlens, int64_t batch, int64_t max_seqlen,
                            int64_t total, int64_t H, int64_t H_kv, int64_t D, float scale,
                            int causal, int dtype, void* stream);

/*
 * fa_forward_varlen_dropout - fa_forward_varlen with dropout on the
 * attention probabilities, as fa_forward_dropout defines it for each
 * (sequence, query head): element (i, j) of query head h of sequence b, i
 * and j counted from the sequence's first token, takes the bits of head
 * b * H + h (exactly those of a dense batch of the same sequences).
 *
 *   dropout_p, seed, offset  as for fa_forward_dropout
 *   other arguments as for fa_forward_varlen
 *
 * Returns FA_OK, FA_ERR_INVALID_ARGUMENT, FA_ERR_UNSUPPORTED or FA_ERR_HIP.
 */
fa_status fa_forward_varlen_dropout(const void* q, const void* k, const void* v, void* o,
                                    float* lse, const int32_t* cu_seqlens, int64_t batch,
                                    int64_t max_seqlen, int64_t total, int64_t H, int64_t H_kv,
                                    int64_t D, float scale, int causal, int dtype,
                                    float dropout_p, uint64_t seed, uint64_t offset,
                                    void* stream);

/*
 * fa_backward_workspace_bytes - device workspace fa_backward needs for
 * this shape: two fp32 row statistics [B, H, N] (delta = rowsum(dO * O) and
 * LSE * log2(e)), each padded to 256 bytes (the two-phase workspace query of
 * "FlashAttention in ops-transformer", "Complete operator"). Returns 0 for
 * non-positive sizes or on overflow.
 */
size_t fa_backward_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t D);

/*
 * fa_backward - attention backward by recomputation.
 *
 * Given the forward's O and LSE and the upstream gradient dO, writes the
 * exact gradients of the forward definition:
 *   P  = exp(scale * Q K^T - LSE)        recomputed tile by tile, masked
 *   dV = P^T dO
 *   dP = dO V^T,  delta_i = sum_d dO[i,d] O[i,d]
 *   dS = P * (dP - delta)
 *   dQ = scale * dS K,   dK = scale * dS^T Q
 * P is never stored ("Flash Attention algorithm design and I/O
 * optimisation", "Core mechanism": save a few statistics, recompute local
 * blocks; "FlashAttention in ops-transformer", "A surprise"). No step uses
 * atomics: the gradients are bitwise reproducible from run to run (the
 * deterministic mode of "FlashAttention in ops-transformer", "Complete
 * operator", is the only mode).
 *
 *   q, k, v, o, dout  in   [B, H, N, D] of `dtype`; o from fa_forward
 *   lse               in   [B, H, N] fp32 from fa_forward
 *   dq, dk, dv        out  [B, H, N, D] of `dtype`
 *   workspace         device scratch of at least
 *                     fa_backward_workspace_bytes(B, H, N, D) bytes, owned by
 *                     the caller, 256-byte aligned; its contents on entry are
 *                     ignored and on return unspecified
 *   B, H, N, D, scale, causal, stream  as for fa_forward (same values)
 *   dtype             FA_FP16 or FA_BF16 (FA_FP32 returns FA_ERR_UNSUPPORTED)
 *
 * Returns FA_OK, FA_ERR_INVALID_ARGUMENT, FA_ERR_UNSUPPORTED,
 * FA_ERR_WORKSPACE or FA_ERR_HIP.
 */
fa_status fa_backward(const void* q, const void* k, const void* v, const void* o,
                      const void* dout, const float* lse, void* dq, void* dk, void* dv,
                      void* workspace, size_t workspace_bytes, int64_t B, int64_t H,
                      int64_t N, int64_t D, float scale, int causal, int dtype,
                      void* stream);

/*
 * fa_backward_dropout - backward of fa_forward_dropout: the same dropout
 * decisions are regenerated from (dropout_p, seed, offset), and
 *   Pd = P * keep / (1 - p'),  dV = Pd^T dO,
 *   dP = (dO V^T) * keep / (1 - p'),  delta_i = sum_d dO[i,d] O[i,d],
 *   dS = P * (dP - delta),  dQ = scale dS K,  dK = scale dS^T Q
 * (p' = thr / 256). o and lse must come from fa_forward_dropout with the
 * same arguments. Workspace, arguments and statuses as for fa_backward;
 * dropout arguments as for fa_forward_dropout. Deterministic (no atomics).
 */
fa_status fa_backward_dropout(const void* q, const void* k, const void* v, const void* o,
                              const void* dout, const float* lse, void* dq, void* dk, void* dv,
                              void* workspace, size_t workspace_bytes, int64_t B, int64_t H,
                              int64_t N, int64_t D, float scale, int causal, int dtype,
                              float dropout_p, uint64_t seed, uint64_t offset, void* stream);

/*
 * fa_backward_gqa - backward of fa_forward_gqa (with or without dropout).
 * Per query head the formulas of fa_backward (fa_backward_dropout when
 * dropout_p != 0) hold; a K/V head serves H / H_kv query heads, so its dK
 * and dV are the sums of their contributions (the chain rule through the
 * shared operand), accumulated in fp32 in a fixed order (deterministic).
 *
 *   q, o, dout, dq   [B, H, N, D] of `dtype`
 *   k, v, dk, dv     [B, H_kv, N, D] of `dtype`
 *   lse              [B, H, N] fp32 from fa_forward_gqa
 *   workspace        fa_backward_workspace_bytes(B, H, N, D) bytes
 *   dropout_p, seed, offset  the values given to fa_forward_gqa
 *   dtype            FA_FP16 or FA_BF16 (FA_FP32 returns FA_ERR_UNSUPPORTED)
 *   other arguments as for fa_backward
 *
 * Returns FA_OK, FA_ERR_INVALID_ARGUMENT, FA_ERR_UNSUPPORTED,
 * FA_ERR_WORKSPACE or FA_ERR_HIP.
 */
fa_status fa_backward_gqa(const void* q, const void* k, const void* v, const void* o,
                          const void* dout, const float* lse, void* dq, void* dk, void* dv,
                          void* workspace, size_t workspace_bytes, int64_t B, int64_t H,
                          int64_t H_kv, int64_t N, int64_t D, float scale, int causal, int dtype,
                          float dropout_p, uint64_t seed, uint64_t offset, void* stream);

/*
 * fa_backward_varlen - backward of fa_forward_varlen: the gradients of a
 * packed batch of variable-length sequences with grouped K/V heads.
 *
 * Per (sequence, query head) the formulas of fa_backward hold. A K/V head
 * is shared by the H / H_kv query heads h with h / (H / H_kv) equal to it,
 * so its dK and dV are the sums of their contributions (the chain rule
 * through the shared operand). No step uses atomics: the sums are taken in
 * a fixed order and the result is bitwise reproducible.
 *
 *   q, o, dout  in   [total, H, D] of `dtype`; o from fa_forward_varlen
 *   k, v        in   [total, H_kv, D] of `dtype`
 *   lse         in   [H, total] fp32 from fa_forward_varlen
 *   dq          out  [total, H, D] of `dtype`
 *   dk, dv      out  [total, H_kv, D] of `dtype`
 *   cu_seqlens, batch, max_seqlen, total, H, H_kv, D, scale, causal, stream
 *               as for fa_forward_varlen (same values); rows of tokens not
 *               covered by any sequence are not written
 *   workspace   device scratch of at least
 *               fa_backward_workspace_bytes(1, H, total, D) bytes, owned by
 *               the caller, 256-byte aligned; contents on entry ignored, on
 *               return unspecified
 *   dtype       FA_FP16 or FA_BF16 (FA_FP32 returns FA_ERR_UNSUPPORTED)
 *
 * Returns FA_OK, FA_ERR_INVALID_ARGUMENT, FA_ERR_UNSUPPORTED,
 * FA_ERR_WORKSPACE or FA_ERR_HIP.
 */
fa_status fa_backward_varlen(const void* q, const void* k, const void* v, const void* o,
                             const void* dout, const float* lse, void* dq, void* dk, void* dv,
                             const int32_t* cu_seqlens, void* workspace, size_t workspace_bytes,
                             int64_t batch, int64_t max_seqlen, int64_t total, int64_t H,
                             int64_t H_kv, int64_t D, float scale, int causal, int dtype,
                             void* stream);

/*
 * fa_backward_varlen_dropout - backward of fa_forward_varlen_dropout: the
 * formulas of fa_backward_dropout per (sequence, query head), dK and dV
 * summed over each K/V head's query heads as in fa_backward_varlen. The
 * dropout arguments must be those given to the forward. Workspace,
 * arguments and statuses as for fa_backward_varlen.
 */
fa_status fa_backward_varlen_dropout(const void* q, const void* k, const void* v, const void* o,
                                     const void* dout, const float* lse, void* dq, void* dk,
                                     void* dv, const int32_t* cu_seqlens, void* workspace,
                                     size_t workspace_bytes, int64_t batch, int64_t max_seqlen,
                                     int64_t total, int64_t H, int64_t H_kv, int64_t D,
                                     float scale, int causal, int dtype, float dropout_p,
                                     uint64_t seed, uint64_t offset, void* stream);

/*
 * fa_decode_workspace_bytes - device workspace fa_decode needs for these
 * sizes: per-chunk partial results (fp32 O and LSE of every output row for
 * every key chunk) when the cache is cut into more than one chunk, else 0.
 * Same arguments as fa_decode. Returns 0 also for invalid sizes.
 */
size_t fa_decode_workspace_bytes(int64_t batch, int64_t s_q, int64_t H, int64_t H_kv,
                                 int64_t max_seqlen_k, int64_t D);

/*
 * fa_decode - attention of new tokens against a key/value cache.
 *
 * The decode step of "Flash Attention algorithm design and I/O
 * optimisation" ("Training and inference value"): each step brings s_q new
 * tokens per sequence and reads the whole cache. Sequence b's cache holds
 * L_b = cache_seqlens[b] tokens, its new tokens being the last s_q of them;
 * new token t sees cache keys 0 .. L_b - s_q + t (causal), query head h reads
 * K/V head h / (H / H_kv). A row that sees no key gets O = 0 and
 * LSE = -inf. The cache is cut into chunks whose (O, LSE) results are merged
 * exactly by LSE (the online-softmax rescale of "From Self-Attention to
 * FlashAttention", section 2, applied to whole chunks).
 *
 *   q              [batch, s_q, H, D] of `dtype`
 *   k_cache, v_cache  [batch, cache_capacity, H_kv, D] of `dtype`
 *   cache_seqlens  device memory, batch int32 lengths, caller-owned; values
 *                  are clamped into [0, max_seqlen_k], so no access leaves
 *                  the caches
 *   o              out [batch, s_q, H, D] of `dtype`
 *   lse            out [batch, H, s_q] fp32, natural log
 *   workspace      device scratch of fa_decode_workspace_bytes(...) bytes,
 *                  256-byte aligned, caller-owned (may be NULL when that
 *                  size is 0); contents on entry ignored, on return
 *                  unspecified
 *   max_seqlen_k   upper bound of cache_seqlens used to cut the chunks,
 *                  0 <= max_seqlen_k <= cache_capacity
 *   H, H_kv        query and K/V heads; H_kv divides H and
 *                  (H / H_kv) * s_q <= 32 (else FA_ERR_UNSUPPORTED)
 *   D              64 or 128
 *   scale          any finite value (1/sqrt(D) is usual)
 *   dtype          FA_FP16 or FA_BF16 (FA_FP32 returns FA_ERR_UNSUPPORTED)
 *   stream         hipStream_t as void*; asynchronous, no allocation
 *
 * Returns FA_OK, FA_ERR_INVALID_ARGUMENT, FA_ERR_UNSUPPORTED,
 * FA_ERR_WORKSPACE or FA_ERR_HIP.
 */
fa_status fa_decode(const void* q, const void* k_cache, const void* v_cache,
                    const int32_t* cache_seqlens, void* o, float* lse, void* workspace,
                    size_t workspace_bytes, int64_t batch, int64_t s_q, int64_t cache_capacity,
                    int64_t max_seqlen_k, int64_t H, int64_t H_kv, int64_t D, float scale,
                    int dtype, void* stream);

/*
 * fa_backward_noalloc - fa_backward without a caller workspace, for callers
 * that cannot allocate device memory at all (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc).
 *
 * Same arguments, results and errors as fa_backward with dropout off, minus
 * workspace and workspace_bytes. The two fp32 row statistics the backward
 * needs live in a static 16 MiB array inside the library instead, one copy
 * per GPU, held until the process ends: B * H * N may be at most 2^21 rows
 * (the size fa_backward_workspace_bytes reports must not exceed 16 MiB);
 * larger calls return FA_ERR_UNSUPPORTED and write nothing. The call
 * allocates and frees nothing; its first call on a device looks up that
 * device's copy of the array (stream must run on the current device).
 * Every call on one GPU shares the array and leaves its contents behind
 * (each call writes every statistic it reads, so nothing needs clearing):
 * calls that overlap on one GPU, on different streams, race.
 *
 * Returns FA_OK, FA_ERR_INVALID_ARGUMENT, FA_ERR_UNSUPPORTED or FA_ERR_HIP.
 */
fa_status fa_backward_noalloc(const void* q, const void* k, const void* v, const void* o,
                              const void* dout, const float* lse, void* dq, void* dk, void* dv,
                              int64_t B, int64_t H, int64_t N, int64_t D, float scale, int causal,
                              int dtype, void* stream);

/*
 * fa_clock_probe - a measurement aid, not part of the attention path: the
 * shader clock the GPU runs at while other work occupies it, so that a
 * throughput can be set against the peak at the clock actually held. One
 * wave of one workgroup (no LDS) spins through `iters` dependent fused
 * multiply-adds between two reads of the shader cycle counter and of the
 * 100 MHz constant clock, and stores the deltas:
 *   out[0]  shader cycles over the spin
 *   out[1]  constant-clock ticks (10 ns each) over the spin
 *   out[2]  unspecified (keeps the spin from being optimised away)
 * The clock in MHz is out[0] / out[1] * 100. Launch it on a stream of its
 * own beside the work to be measured; 10^5 iterations take about 1.5 ms.
 *   out     device, 3 x uint64, 8-byte aligned; written by the kernel
 *   iters   >= 1
 *   stream  HIP stream (NULL: the default stream); asynchronous
 * Returns FA_ERR_INVALID_ARGUMENT (NULL or misaligned out, iters < 1) before
 * any HIP call, FA_ERR_HIP if the launch fails, else FA_OK.
 */
fa_status fa_clock_probe(uint64_t* out, int iters, void* stream);

/* fa_status_string - static, never-NULL name of a status code. */
const char* fa_status_string(int status);

/* fa_last_error - detail of the last failing call on the calling thread
 * ("" if none). Valid until the next call on that thread. */
const char* fa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_H */
