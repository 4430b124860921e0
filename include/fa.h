/*
 * fa.h — exact attention (FlashAttention-style forward and recompute backward) for AMD
 * Instinct MI355X (gfx950). C ABI: plain pointers and sizes, no framework types.
 *
 * What is computed (pages, cited by title and section):
 *   "FlashAttention 为什么不需要存下注意力矩阵" (jefxiong.cn) §03 3.1-3.3 and
 *   "FlashAttention V1 技术深度解析" (spark.aweffr.cn) §2.2, §3.2, §4.2.
 *
 *   Forward, per (b, h):  S = scale * Q K^T  (causal: S[i][j] = -inf for key j > query i),
 *                         P = softmax(S) row-wise,  O = P V,
 *                         LSE[i] = m_i + log(l_i) = log sum_j exp(S[i][j])   (natural log).
 *   Backward, given dO:   dV = P^T dO,  dP = dO V^T,  D_i = rowsum(dO * O)_i,
 *                         dS = P * (dP - D),  dQ = scale * dS K,  dK = scale * dS^T Q.
 *   P is never stored: the forward streams K/V tiles with a running max, a running sum and an
 *   unnormalised output accumulator rescaled by exp(m_old - m_new); the backward recomputes each
 *   P tile as exp(S - LSE).
 *
 * Layout: every tensor is contiguous [B, H, N, d] (d fastest), LSE and the internal row
 * vectors are contiguous [B, H, N]. Q, K and V share N (self-attention). Pointers must be
 * device pointers (hipMalloc'd or equivalent) aligned to 16 bytes.
 *
 * Supported: d in {32, 64, 96, 128}, and 256 for plain 16-bit attention only (fa_forward,
 * fa_forward_kv, fa_backward, fa_backward_kv); decoding: d in {64, 128}. N >= 1 (a ragged tail is masked);
 * B, H >= 1 with B*H*N*d < 2^31
 * and N*d < 2^30 (a head's fp32 rows then span less than 4 GiB, the reach of a buffer load's
 * 32-bit byte range; the same bound applies to Nk*d);
 * in_dtype in {FA_F32, FA_F16, FA_BF16}; any finite scale; causal in {0, 1}.
 * The backward supports all three input dtypes (fp32 inputs: O and the gradients in fp32, N = Nk,
 * no dropout or block mask, as the fp32 forward).
 *
 * Ownership: the caller owns every buffer and the stream. The library never allocates or frees
 * device memory; the backward takes a caller-provided workspace.
 *
 * Errors: arguments are validated before any launch. An unsupported combination returns
 * FA_ERR_UNSUPPORTED and an invalid one FA_ERR_INVALID_ARG; nothing is launched and there is no
 * fallback path. FA_ERR_HIP reports a failed HIP call or launch. The library never aborts,
 * prints or throws across this boundary. FA_ERR_RANGE is returned only by the optional debug
 * range check of the backward (FA_DEBUG_CHECKS=1, see the input range note below).
 *
 * Asynchrony: calls enqueue kernels on `stream` (a hipStream_t; NULL = the null stream) and
 * return without waiting. Calls on distinct streams may run concurrently from distinct threads.
 */
#ifndef FA_H
#define FA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum fa_status {
  FA_OK = 0,
  FA_ERR_INVALID_ARG = 1, /* null pointer, non-positive size, size overflow, non-finite scale */
  FA_ERR_UNSUPPORTED = 2, /* head dim, dtype combination or mode this build does not provide */
  FA_ERR_WORKSPACE = 3,   /* workspace missing or smaller than fa_backward_workspace_bytes() */
  FA_ERR_HIP = 4,         /* a HIP runtime call or kernel launch failed */
  FA_ERR_RANGE = 5        /* FA_DEBUG_CHECKS=1 only: a bf16 input of a backward call lies outside
                             the range of its fp16 operand copy (|x| >= 65536 or not finite) */
} fa_status;

typedef enum fa_dtype { FA_F32 = 0, FA_F16 = 1, FA_BF16 = 2 } fa_dtype;

/*
 * Forward pass ("FlashAttention 为什么不需要存下注意力矩阵" §03 3.2, §04 4.1: the tiled function
 * returns the normalised output and the per-row logsumexp).
 *
 *   q, k, v  [B,H,N,d] in in_dtype (read only)
 *   o        [B,H,N,d] in o_dtype, written: o_dtype is in_dtype, or FA_F32 for 16-bit inputs
 *   lse      [B,H,N] float32, written: natural-log logsumexp of the scaled scores per query row
 *   scale    multiplies Q K^T before the softmax (usually 1/sqrt(d)); any finite value
 *   causal   1: query i attends to keys 0..i; 0: to all N keys
 * Fully masked K/V tiles are skipped. Results are deterministic (no atomics).
 */
fa_status fa_forward(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                     int H, int N, int d, float scale, int causal, fa_dtype in_dtype,
                     fa_dtype o_dtype, void* stream);

/*
 * Forward pass with different query and key lengths (chunked prefill over a K/V cache, or
 * cross-attention): Nq query rows per head against Nk keys. Same computation as fa_forward, with
 *   q, o     [B,H,Nq,d];  k, v [B,H,Nk,d];  lse [B,H,Nq]
 *   causal   1: the queries are the LAST Nq positions of the key sequence, so query row i sees
 *            keys 0 .. Nk - Nq + i (the top-left rule of fa_forward when Nq = Nk); requires
 *            Nq <= Nk (otherwise FA_ERR_INVALID_ARG). 0: every query sees all Nk keys.
 * in_dtype must be FA_F16 or FA_BF16 (FA_ERR_UNSUPPORTED otherwise); other errors as fa_forward.
 */
fa_status fa_forward_kv(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                        int H, int Nq, int Nk, int d, float scale, int causal, fa_dtype in_dtype,
                        fa_dtype o_dtype, void* stream);

/*
 * Bytes of device workspace fa_backward needs for these sizes and dtypes: the row vector
 * D = rowsum(dO * O) (float32 [B,H,N]), a per-head dO scale (float32 [B,H]), room for 256
 * partial maxima of |dO| per head, a flag word, the scaled fp16 copy of dO ([B,H,N,d] 16-bit)
 * and, when in_dtype is FA_BF16, fp16 copies of Q, K and V (3 x [B,H,N,d] 16-bit) used as the
 * MFMA operands.
 * grad_dtype does not change the size but is validated. Returns 0 for arguments fa_backward would
 * reject (e.g. an in_dtype / grad_dtype pair it does not provide).
 */
size_t fa_backward_workspace_bytes(int B, int H, int N, int d, fa_dtype in_dtype,
                                   fa_dtype grad_dtype);

/*
 * Input range of every backward entry point (fa_backward, fa_backward_kv, fa_backward_dropout,
 * fa_backward_blocksparse). The five products run on fp16 MFMA operands with fp32 accumulation:
 *   - Q, K and V: bf16 inputs are converted to fp16, which is exact for 2^-14 <= |x| <= 65504 and
 *     changes smaller values by less than 2^-25. PRECONDITION: |Q|, |K|, |V| < 65520 elementwise
 *     (larger bf16 values would become infinities). fp16 inputs are used as they are.
 *   - dO: scaled per (b, h) by a power of two 2^s before its fp16 copy is taken, chosen from the
 *     head's largest |dO| (s = 0 while that lies in [1/2, 16], so ordinary gradients keep their
 *     bits; otherwise it is brought into [8, 16)). dP, D and dS scale along with it and stay
 *     inside fp16's range for upstream gradients of any magnitude; the results are multiplied by
 *     2^-s, which is exact. No precondition on dO beyond being finite.
 * With FA_DEBUG_CHECKS=1 in the environment, a backward call with bf16 inputs first checks the
 * precondition on the device, waits for the answer and returns FA_ERR_RANGE (launching no
 * backward kernel) when it fails. The check needs no more workspace than the call itself.
 */

/*
 * Backward pass ("FlashAttention 为什么不需要存下注意力矩阵" §03 3.3; "FlashAttention V1 技术深度解析"
 * §4.2: recompute each P tile from the saved statistics instead of storing P).
 *
 *   q, k, v    [B,H,N,d] in in_dtype (FA_F32, FA_F16 or FA_BF16), the forward's inputs
 *   o          [B,H,N,d] in o_dtype (in_dtype or FA_F32), the forward's output
 *   dout       [B,H,N,d] in in_dtype, the upstream gradient dL/dO
 *   lse        [B,H,N] float32, the forward's logsumexp
 *   dq, dk, dv [B,H,N,d] in grad_dtype (in_dtype or FA_F32), written
 *   workspace  device buffer of at least fa_backward_workspace_bytes(B,H,N,d,in_dtype,grad_dtype)
 *              bytes,
 *              16-byte aligned; contents on entry are ignored and clobbered
 * Four kernels run on the stream: a max pass (per-head max |dO|, fp16 copy of bf16 Q), a
 * row-wise preprocess (dO scale, D, scaled fp16 dO), a keys-outer kernel for dK and dV, and a
 * queries-outer kernel for dQ. Every product uses fp16 MFMA operands with fp32 accumulation
 * (input range above). fp32 inputs instead run three kernels (D, dK/dV, dQ) on true-fp32 MFMA
 * with no operand copies and no scaling. No atomics: all outputs are deterministic.
 */
fa_status fa_backward(const void* q, const void* k, const void* v, const void* o,
                      const void* dout, const float* lse, void* dq, void* dk, void* dv, int B,
                      int H, int N, int d, float scale, int causal, fa_dtype in_dtype,
                      fa_dtype o_dtype, fa_dtype grad_dtype, void* workspace,
                      size_t workspace_bytes, void* stream);

/*
 * Bytes of device workspace fa_backward_kv needs: D (float32 [B,H,Nq]), the per-head dO scale and
 * partial maxima, a flag word, the scaled fp16 copy of dO ([B,H,Nq,d]) and, when in_dtype is
 * FA_BF16, fp16 copies of Q ([B,H,Nq,d]) and of K and V ([B,H,Nk,d] each). Equal to
 * fa_backward_workspace_bytes when Nq = Nk. Returns 0 for arguments fa_backward_kv would reject.
 */
size_t fa_backward_kv_workspace_bytes(int B, int H, int Nq, int Nk, int d, fa_dtype in_dtype,
                                      fa_dtype grad_dtype);

/*
 * Backward pass of fa_forward_kv (same gradients as fa_backward, over Nq queries and Nk keys):
 *   q, o, dout, dq  [B,H,Nq,d];  k, v, dk, dv [B,H,Nk,d];  lse [B,H,Nq]
 *   causal          as in fa_forward_kv (queries are the last Nq positions; Nq <= Nk)
 *   workspace       at least fa_backward_kv_workspace_bytes(B,H,Nq,Nk,d,in_dtype,grad_dtype)
 * Keys that no query sees get dK = dV = 0. Dtypes, workspace rules and errors as fa_backward.
 */
fa_status fa_backward_kv(const void* q, const void* k, const void* v, const void* o,
                         const void* dout, const float* lse, void* dq, void* dk, void* dv, int B,
                         int H, int Nq, int Nk, int d, float scale, int causal,
                         fa_dtype in_dtype, fa_dtype o_dtype, fa_dtype grad_dtype,
                         void* workspace, size_t workspace_bytes, void* stream);

/*
 * Forward pass with dropout on the attention probabilities ("FlashAttention 为什么不需要存下注意力矩阵"
 * §05, fourth difference: the kernel keeps no mask, only the random generator's seed and
 * offset, and the backward pass regenerates the same mask from them).
 *
 *   O = (P * Z / q) V  with P the softmax above, Z in {0, 1} the keep mask, q the keep rate;
 *   LSE is that of the undropped softmax. Arguments as fa_forward, plus:
 *   dropout_p  drop probability, finite, 0 <= p < 1 (otherwise FA_ERR_INVALID_ARG)
 *   seed       64-bit generator key; offset  32-bit stream selector (e.g. a step counter)
 * Mask: for head index bh = b*H + h, query i and key j, Philox-4x32-10 (Salmon et al., SC'11)
 * with counter (j / 8, i, bh, offset) and key (seed low word, seed high word) yields eight 16-bit
 * values (w0 low half, w0 high half, w1 low half, ... w3 high half) for keys 8*(j/8) .. +7;
 * Z[i][j] = 1 iff the value for j is below T = floor((1 - p) * 65536 + 1/2), and q = T / 65536.
 * The same (seed, offset) must be passed to fa_backward_dropout. in_dtype must be FA_F16 or
 * FA_BF16 (FA_F32 returns FA_ERR_UNSUPPORTED).
 */
fa_status fa_forward_dropout(const void* q, const void* k, const void* v, void* o, float* lse,
                             int B, int H, int N, int d, float scale, int causal,
                             fa_dtype in_dtype, fa_dtype o_dtype, float dropout_p, uint64_t seed,
                             uint32_t offset, void* stream);

/*
 * Backward pass of fa_forward_dropout, regenerating the same keep mask Z from (dropout_p, seed,
 * offset): dV = (P * Z / q)^T dO, dP = (dO V^T) * Z / q, D = rowsum(dO * O), dS = P * (dP - D),
 * dQ = scale * dS K, dK = scale * dS^T Q. Arguments, workspace and errors as fa_backward; o must
 * be the dropout forward's output.
 */
fa_status fa_backward_dropout(const void* q, const void* k, const void* v, const void* o,
                              const void* dout, const float* lse, void* dq, void* dk, void* dv,
                              int B, int H, int N, int d, float scale, int causal,
                              fa_dtype in_dtype, fa_dtype o_dtype, fa_dtype grad_dtype,
                              float dropout_p, uint64_t seed, uint32_t offset, void* workspace,
                              size_t workspace_bytes, void* stream);

/* Block size of the block-sparse masks: one mask byte covers 128 queries x 128 keys. */
#define FA_SPARSE_BLOCK 128
/* Longest sequence the block-sparse entry points accept. */
#define FA_SPARSE_MAX_N 65536

/*
 * Block-sparse forward pass ("FlashAttention 为什么不需要存下注意力矩阵" §06: once attention is cut
 * into blocks, whole blocks can be skipped; the causal case of §04 4.5 generalised to any
 * pattern of blocks is block-sparse attention).
 *
 *   block_mask  device array of mask_heads x nb x nb bytes, nb = ceil(N / FA_SPARSE_BLOCK),
 *               row-major: block_mask[(hm * nb + qb) * nb + kb] != 0 lets queries
 *               128*qb .. 128*qb + 127 see keys 128*kb .. 128*kb + 127 (read only, caller-owned)
 *   mask_heads  1 (one mask for every (b, h)) or B*H (mask of head b*H + h at index b*H + h)
 * Query i sees key j iff its block is nonzero (and j <= i when causal). Blocks that are zero are
 * never loaded or computed. A query that sees no key gets O = 0 and LSE = -inf. Other arguments
 * as fa_forward; in_dtype must be FA_F16 or FA_BF16 and N <= FA_SPARSE_MAX_N
 * (FA_ERR_UNSUPPORTED otherwise); a NULL mask or another mask_heads is FA_ERR_INVALID_ARG.
 */
fa_status fa_forward_blocksparse(const void* q, const void* k, const void* v, void* o,
                                 float* lse, int B, int H, int N, int d, float scale, int causal,
                                 fa_dtype in_dtype, fa_dtype o_dtype, const uint8_t* block_mask,
                                 int mask_heads, void* stream);

/*
 * Backward pass of fa_forward_blocksparse with the same mask: invisible keys have P = 0 and only
 * live blocks are visited; queries that saw no key (LSE = -inf) contribute nothing. Arguments,
 * workspace and errors as fa_backward plus the mask arguments of fa_forward_blocksparse.
 */
fa_status fa_backward_blocksparse(const void* q, const void* k, const void* v, const void* o,
                                  const void* dout, const float* lse, void* dq, void* dk,
                                  void* dv, int B, int H, int N, int d, float scale, int causal,
                                  fa_dtype in_dtype, fa_dtype o_dtype, fa_dtype grad_dtype,
                                  const uint8_t* block_mask, int mask_heads, void* workspace,
                                  size_t workspace_bytes, void* stream);

/*
 * Bytes of device workspace fa_decode_forward needs for these sizes: per (head, key chunk, query)
 * an fp32 partial output of d elements and its running maximum and sum. Returns 0 for sizes
 * fa_decode_forward would reject.
 */
size_t fa_decode_workspace_bytes(int B, int H, int Nq, int Nk, int d);

/*
 * Split-KV decoding forward: Nq query rows per head, the LAST Nq positions of a sequence of Nk
 * keys (Flash-Decoding, named in "FlashAttention V1 技术深度解析" (conclusion) and
 * "Flash Attention：一个数学技巧把内存省 5 倍" §七; the merge is the rescale of
 * "FlashAttention 为什么不需要存下注意力矩阵" §03 3.2 applied to whole chunks of keys).
 *
 *   q        [B,H,Nq,d] in in_dtype (FA_F16 or FA_BF16), 1 <= Nq <= 4 and Nq <= Nk
 *   k, v     [B,H,Nk,d] in in_dtype (e.g. a KV cache)
 *   o        [B,H,Nq,d] in o_dtype (in_dtype or FA_F32), written
 *   lse      [B,H,Nq] float32, written (natural-log logsumexp of the scaled scores)
 *   causal   1: query i (0-based among the Nq) sees keys 0 .. Nk - Nq + i; 0: all Nk keys
 *   workspace  device buffer of at least fa_decode_workspace_bytes(B, H, Nq, Nk, d) bytes,
 *            16-byte aligned; contents ignored and clobbered
 * Two kernels run on the stream: one workgroup per (head, chunk of keys) writes a partial result,
 * then one workgroup per (head, query) merges the partials. Deterministic (no atomics).
 * Errors as fa_forward; Nq > 4 returns FA_ERR_UNSUPPORTED, Nq > Nk FA_ERR_INVALID_ARG.
 */
fa_status fa_decode_forward(const void* q, const void* k, const void* v, void* o, float* lse,
                            int B, int H, int Nq, int Nk, int d, float scale, int causal,
                            fa_dtype in_dtype, fa_dtype o_dtype, void* workspace,
                            size_t workspace_bytes, void* stream);

/* Bytes of device scratch that fa_decode_forward_noalloc has on each GPU. */
#define FA_DECODE_SCRATCH_BYTES (8u << 20)

/*
 * fa_decode_forward without a workspace, for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid allocation. Same arguments
 * (minus the workspace), computation, kernels and results as fa_decode_forward. The per-chunk
 * partials live in a device array of FA_DECODE_SCRATCH_BYTES that the library holds on each GPU
 * it runs on until the process ends; the call itself allocates nothing (no hipMalloc, no
 * allocating library routine). Calls needing more scratch than that, i.e. with
 * fa_decode_workspace_bytes(B, H, Nq, Nk, d) > FA_DECODE_SCRATCH_BYTES, return FA_ERR_WORKSPACE
 * before any launch. Every call on one GPU uses that GPU's single array: calls that may overlap
 * in time on one GPU (different streams, different threads) race on it and must be serialised
 * by the caller. Nothing needs clearing between calls (every partial is written before it is
 * read). Other errors as fa_decode_forward.
 */
fa_status fa_decode_forward_noalloc(const void* q, const void* k, const void* v, void* o,
                                    float* lse, int B, int H, int Nq, int Nk, int d, float scale,
                                    int causal, fa_dtype in_dtype, fa_dtype o_dtype,
                                    void* stream);

/*
 * fa_backward with a measurement aid that leaves the results unchanged (the same kernels and
 * arithmetic as fa_backward on the same arguments). It records `ev_before` on `stream` right
 * before the dK/dV kernel is launched and `ev_after` right after it. The caller can then time
 * that kernel, the longest of the backward, with hipEventElapsedTime. Both are hipEvent_t handles
 * the caller owns; the library keeps no reference to them after the call.
 * 16-bit inputs only (FA_F32 returns FA_ERR_UNSUPPORTED). A NULL event returns
 * FA_ERR_INVALID_ARG. Other arguments and errors are as for fa_backward.
 */
fa_status fa_backward_timed(const void* q, const void* k, const void* v, const void* o,
                            const void* dout, const float* lse, void* dq, void* dk, void* dv,
                            int B, int H, int N, int d, float scale, int causal,
                            fa_dtype in_dtype, fa_dtype o_dtype, fa_dtype grad_dtype,
                            void* workspace, size_t workspace_bytes, void* stream,
                            void* ev_before, void* ev_after);

/* A static, human-readable description of a status code (never NULL). */
const char* fa_status_string(fa_status s);

#ifdef __cplusplus
}
#endif

#endif /* FA_H */
