/*
 * fa.h — C ABI of the exact tiled attention library (libfa.so, gfx950).
 *
 * What it computes: exact scaled-dot-product attention in the FlashAttention
 * style.  The forward pass tiles Q, K and V, forms S = scale * Q K^T one tile
 * at a time, runs the online softmax (running row max m and row sum l, with
 * the partial output rescaled by e^{m_old - m_new}) and accumulates P V
 * without ever writing the N x N matrix; it stores O and the per-row
 * log-sum-exp.  The backward pass recomputes P from that log-sum-exp instead
 * of reading a stored P and forms dV, dK and dQ, each accumulated in fp32
 * by the one workgroup that owns it.
 *   - three-step definition S = QK^T, P = softmax(S), O = PV: lab write-up
 *     "FlashAttention" (dpshk.com), section 2.1;
 *   - tiling, online softmax and recomputation: the same write-up,
 *     sections 3.1, 3.2 and 3.3;
 *   - argument set (q, k, v, dropout_p, softmax_scale, causal), the
 *     [batch, seq, heads, head_dim] layout, fp16/bf16 only: the write-up's
 *     section 4.2 and the FlashAttention library overview's usage example;
 *   - variable-length batches (cu_seqlens): the varlen interface named in
 *     section 4.2 of the write-up;
 *   - packed QKV ([B, N, 3, H, d]): the qkvpacked example of the tiemojia.cn
 *     article, reached here through the row stride ld_qkv.
 *
 * Conventions shared by every entry point:
 *   - All tensor pointers are DEVICE pointers owned by the caller.  The
 *     library never allocates, frees, synchronizes or aborts.  Work is
 *     enqueued on `stream` (a hipStream_t passed as void*; NULL = the null
 *     stream) and runs asynchronously.
 *   - Fixed length (cu_seqlens == NULL): q, k, v and their gradients are
 *     [B, N, H, d] with consecutive tokens ld_qkv elements apart (ld_qkv == 0
 *     means H*d, i.e. contiguous; packed QKV passes 3*H*d).  o and dout are
 *     always contiguous [B, N, H, d].  lse is float32 [B, N, H].
 *   - Varlen (cu_seqlens != NULL): cu_seqlens is a DEVICE int32 array of
 *     B + 1 prefix sums (cu_seqlens[0] = 0, non-decreasing); sequence b holds
 *     tokens cu_seqlens[b] .. cu_seqlens[b+1]-1 of [total, H, d] tensors, and
 *     lse is [total, H].  N must be >= every sequence length (it sizes the
 *     grid).  Causal masking and dropout indices are local to each sequence;
 *     queries never see another sequence.  Its contents are a precondition
 *     the library does not read on the host.  The kernels clamp them so that
 *     no access leaves [0, min(cu_seqlens[B], B*N)) tokens: a sequence longer
 *     than N is cut to its first N tokens (its later rows are not written),
 *     and prefix sums that are negative, decreasing or past B*N give empty or
 *     shortened sequences (outputs unspecified, never an out-of-bounds
 *     access).
 *   - Causal: query i sees keys j <= i (queries and keys have equal length).
 *   - scale multiplies Q K^T before the softmax (1/sqrt(d) is the usual value).
 *   - Dropout (0 < dropout_p < 1) drops entries of the normalised P before
 *     the P V product and scales kept entries by 1/(1 - dropout_p); the
 *     log-sum-exp excludes dropout.  Philox-4x32-10 (Salmon et al., SC'11)
 *     with key (seed low 32 bits, seed high 32 bits) and counter
 *     (i, j / 8, h, b) gives four 32-bit words, read as eight 16-bit values
 *     (value v: low half of word v/2 for even v, high half for odd v);
 *     element (b, h, i, j) is kept iff value j mod 8 is
 *     >= floor(dropout_p * 2^16), so the drop probability is that threshold
 *     / 2^16 (within 2^-16 of dropout_p).  Forward and backward must get the
 *     same seed and dropout_p.  dropout_p == 0 runs the no-dropout kernels.
 *   - dtype is FA_DTYPE_F16 or FA_DTYPE_BF16 for every tensor except lse and
 *     the workspace (float32).  d must be 32, 64, 96, 128, 160, 192 or 256.
 *     Up to 128 is the fused-kernel range in the tiemojia.cn article's list
 *     of when the fused kernel applies (its engineering-considerations
 *     part); the larger heads run with one wave per SIMD (the output tile
 *     needs the whole register file), and at 256 the key-side kernel
 *     recomputes S and dP once per half of dK, dV's columns, so those
 *     heads run at a lower rate -- the lab write-up, section 5.3, warns
 *     that kernels degrade past 192.
 *   - Pointers must be 16-byte aligned and ld_qkv a multiple of 8; the
 *     token stride (ld_qkv, or H*d) may not exceed FA_MAX_TOKEN_STRIDE
 *     elements (FA_ERR_UNSUPPORTED otherwise: the kernels address a tile of
 *     64 tokens through a 32-bit byte range).
 *   - Outputs must not alias inputs; dq, dk and dv may point into one packed
 *     [B, N, 3, H, d] buffer when ld_qkv = 3*H*d.
 *   - Every argument is checked on the host before any HIP call; a failed
 *     check returns a nonzero FA_ERR_* code and enqueues nothing.  A launch
 *     error returns FA_ERR_HIP.
 */
#ifndef FA_H_
#define FA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Largest token stride (elements between consecutive tokens) of q, k, v,
 * dq, dk, dv, o and dout that fa_forward / fa_backward accept. */
#define FA_MAX_TOKEN_STRIDE (1 << 24)

enum fa_dtype { FA_DTYPE_F16 = 0, FA_DTYPE_BF16 = 1 };

enum fa_status {
    FA_OK = 0,
    FA_ERR_NULL_POINTER = 1,   /* a required pointer is NULL */
    FA_ERR_BAD_SHAPE = 2,      /* B, H or N < 1, or a size overflows */
    FA_ERR_UNSUPPORTED = 3,    /* d not in {32, 64, 96, 128, 160, 192, 256}, unknown dtype,
                                  or N above FA_MASK_MAX_N for a block-sparse call or a
                                  stored-keep-bit call with dropout */
    FA_ERR_BAD_ARGUMENT = 4,   /* scale not finite, dropout_p not in [0, 1) */
    FA_ERR_ALIGNMENT = 5,      /* pointer not 16-byte aligned or bad ld_qkv */
    FA_ERR_WORKSPACE = 6,      /* workspace (or keep-bit buffer) NULL or smaller than required */
    FA_ERR_HIP = 7,            /* a HIP launch reported an error */
    FA_ERR_SCRATCH_LIMIT = 8   /* fa_backward_noalloc: B*N*H above FA_NOALLOC_MAX_ROWS */
};

/* Forward pass.
 *   q, k, v : input, layout above, row stride ld_qkv.
 *   o       : output, contiguous [tokens, H, d], dtype.
 *   lse     : output, float32 [tokens, H]: natural-log log-sum-exp of the
 *             scaled scores of each query row over its visible keys.
 * Lab write-up sections 3.1-3.2 (tiling + online softmax); library overview
 * usage example (flash_attn_func arguments). */
int fa_forward(const void* q, const void* k, const void* v, void* o, float* lse,
               int B, int H, int N, int d, float scale, int causal,
               const int32_t* cu_seqlens, float dropout_p, uint64_t seed, void* stream,
               int dtype, int64_t ld_qkv);

/* Bytes of device workspace fa_backward needs for B sequences of at most N
 * tokens with H heads of size d: two fp32 [B*N, H] arrays, each rounded up
 * to 256 bytes, the row terms D = rowsum(dO * O) and lse * log2(e) (written
 * by the query-side kernel, read by the key-side kernel).  The size depends
 * on the token count B*N only (d is accepted for symmetry), so a caller that
 * counts tokens T may ask for (1, T, H, d); for packed variable-length
 * input that T must be B*max_seqlen, the bound fa_backward checks against
 * (it cannot read cu_seqlens on the host).  Returns 0 if the size overflows.
 * Host-only, never fails otherwise. */
size_t fa_backward_workspace_size(int B, int N, int H, int d);

/* Backward pass (recomputation from lse, lab write-up section 3.3).
 *   q, k, v, o, lse : what fa_forward was given / produced.
 *   dout            : contiguous [tokens, H, d] gradient of the loss wrt o.
 *   dq, dk, dv      : outputs, row stride ld_qkv.
 *   workspace       : device memory of at least fa_backward_workspace_size
 *                     bytes, 16-byte aligned; no initialisation needed; its
 *                     contents are overwritten.
 * Enqueues two kernels: the query-side kernel (D = rowsum(dO * O) into the
 * workspace, then dQ, accumulated in fp32 registers over every key block a
 * query sees) and the key-side kernel (dK and dV, accumulated in fp32
 * registers over every query block that sees a key; reads D).  Both
 * recompute S and P from lse; no atomics are used, so results are
 * deterministic. */
int fa_backward(const void* q, const void* k, const void* v, const void* o, const float* lse,
                const void* dout, void* dq, void* dk, void* dv,
                int B, int H, int N, int d, float scale, int causal,
                const int32_t* cu_seqlens, float dropout_p, uint64_t seed, void* stream,
                int dtype, int64_t ld_qkv, void* workspace, size_t workspace_bytes);

/* One of the two kernels fa_backward enqueues, for callers that time or
 * schedule them separately: stage 0 = query-side kernel (D into the
 * workspace, dQ), 1 = key-side kernel (dK, dV; reads D from the workspace).
 * Stages 0 then 1 enqueued on one stream with identical arguments do exactly
 * what fa_backward does.  Arguments and errors as fa_backward; a stage
 * outside 0..1 returns FA_ERR_BAD_ARGUMENT. */
int fa_backward_stage(int stage, const void* q, const void* k, const void* v, const void* o,
                      const float* lse, const void* dout, void* dq, void* dk, void* dv,
                      int B, int H, int N, int d, float scale, int causal,
                      const int32_t* cu_seqlens, float dropout_p, uint64_t seed, void* stream,
                      int dtype, int64_t ld_qkv, void* workspace, size_t workspace_bytes);

/* The backward for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation):
 * fa_backward without the workspace arguments.  Its two row arrays live in a
 * fixed array of FA_NOALLOC_SCRATCH_BYTES (32 MiB) in device memory, one per
 * GPU, which the library holds from the first call on a GPU until the
 * process ends; the call itself allocates and frees nothing.
 *   Arguments, layout and errors as fa_backward, plus FA_ERR_SCRATCH_LIMIT
 *   when B*N*H > FA_NOALLOC_MAX_ROWS (checked before any HIP call).
 *   The GPU is the stream's (the current GPU for the null stream);
 *   FA_ERR_UNSUPPORTED for a device ordinal >= FA_NOALLOC_MAX_DEVICES.
 * Every call on one GPU shares that GPU's array: calls that overlap on one
 * GPU (other streams, other threads) race and must be serialised by the
 * caller.  Nothing needs clearing between calls: each call writes every row
 * its own kernels read. */
#define FA_NOALLOC_MAX_ROWS (1 << 22)
#define FA_NOALLOC_SCRATCH_BYTES ((size_t)2 * FA_NOALLOC_MAX_ROWS * 4)
#define FA_NOALLOC_MAX_DEVICES 64
int fa_backward_noalloc(const void* q, const void* k, const void* v, const void* o, const float* lse,
                        const void* dout, void* dq, void* dk, void* dv,
                        int B, int H, int N, int d, float scale, int causal,
                        const int32_t* cu_seqlens, float dropout_p, uint64_t seed, void* stream,
                        int dtype, int64_t ld_qkv);

/* ---------------------------------------------------------- block-sparse
 * Block-sparse attention: the block-sparse mode the coreui.cn
 * FlashAttention-2 how-to names in section 5.2 (with masks converted to
 * block format, its section 2.3).  A block mask switches whole FA_MASK_BLOCK x FA_MASK_BLOCK blocks of
 * the score matrix on or off; the kernels skip the tiles of blocks that are
 * off, so work and time scale with the number of blocks that are on.
 *   block_mask : DEVICE uint8 [B, H, nb, nb], nb = ceil(N / FA_MASK_BLOCK),
 *                owned by the caller.  Entry (b, h, r, c) nonzero lets the
 *                queries r*FA_MASK_BLOCK .. +FA_MASK_BLOCK-1 of sequence b,
 *                head h see the keys c*FA_MASK_BLOCK .. +FA_MASK_BLOCK-1
 *                (positions local to the sequence for varlen).  With
 *                causal, j <= i applies as well.
 *   A query that sees no key gets O = 0 and lse = -inf, and contributes no
 *   gradient.  N must be <= FA_MASK_MAX_N (FA_ERR_UNSUPPORTED otherwise);
 *   a NULL block_mask returns FA_ERR_NULL_POINTER.  Every other argument,
 *   layout and error is as for fa_forward / fa_backward, which the calls
 *   below equal when every mask entry is nonzero. */
#define FA_MASK_BLOCK 128
#define FA_MASK_MAX_N 65536

int fa_forward_block_sparse(const void* q, const void* k, const void* v, void* o, float* lse,
                            int B, int H, int N, int d, float scale, int causal,
                            const int32_t* cu_seqlens, float dropout_p, uint64_t seed, void* stream,
                            int dtype, int64_t ld_qkv, const uint8_t* block_mask);

int fa_backward_block_sparse(const void* q, const void* k, const void* v, const void* o,
                             const float* lse, const void* dout, void* dq, void* dk, void* dv,
                             int B, int H, int N, int d, float scale, int causal,
                             const int32_t* cu_seqlens, float dropout_p, uint64_t seed,
                             void* stream, int dtype, int64_t ld_qkv, void* workspace,
                             size_t workspace_bytes, const uint8_t* block_mask);

/* One of the two kernels fa_backward_block_sparse enqueues (stage 0: D and
 * dQ, stage 1: dK and dV), as fa_backward_stage is for fa_backward. */
int fa_backward_block_sparse_stage(int stage, const void* q, const void* k, const void* v,
                                   const void* o, const float* lse, const void* dout, void* dq,
                                   void* dk, void* dv, int B, int H, int N, int d, float scale,
                                   int causal, const int32_t* cu_seqlens, float dropout_p,
                                   uint64_t seed, void* stream, int dtype, int64_t ld_qkv,
                                   void* workspace, size_t workspace_bytes,
                                   const uint8_t* block_mask);

/* ---------------------------------------------------- stored dropout bits
 * Dropout, which the coreui.cn FlashAttention-2 how-to (section 2.3) singles
 * out for special handling, is drawn by fa_forward / fa_backward from a
 * counter-based hash in each of the three kernels, in the spirit of the lab
 * write-up's section 3.3 (the backward recomputes rather than stores N x N
 * intermediates).  These calls trade memory for that hashing: the forward
 * stores the keep decisions it draws, one bit per (query, key) pair (N^2/8
 * bytes per head, against 2 N^2 for a stored 16-bit P), and the backward
 * reads them instead of hashing again.
 * Results are bitwise those of fa_forward / fa_backward with the same
 * arguments.  Dense and packed variable-length input only (no block mask).
 *
 * Layout of keep_bits (DEVICE, 32-bit words, caller-owned): with Np = N
 * rounded up to a multiple of 4, word
 *   (((b * H + h) * ceil(N/64) + t) * 2 + w) * Np + i
 * holds in bit k the decision for query i against key 64 t + 32 w + k of
 * sequence b, head h (local indices; 1 = kept), i.e. Np * ceil(N/64) * 8
 * bytes per (b, h).  The forward writes the words of the key tiles it
 * computes for each query (at least up to the query's causal diagonal, and
 * only rows of real queries) and leaves the others as they were; the
 * backward also reads some unwritten words, but only for pairs the causal
 * mask or the sequence end hides, whose bits have no effect. */

/* Bytes of keep_bits for B sequences of at most N tokens with H heads.
 * Returns 0 for N > FA_MASK_MAX_N (a head's bits must fit one 32-bit
 * buffer range) or sizes that overflow.  Host-only. */
size_t fa_dropout_bits_size(int B, int N, int H);

/* fa_forward, storing its dropout decisions into keep_bits (16-byte
 * aligned, keep_bits_bytes >= fa_dropout_bits_size(B, N, H)).  With
 * dropout_p == 0 it is exactly fa_forward and keep_bits is not touched (it
 * may be NULL).  Errors: those of fa_forward; FA_ERR_NULL_POINTER (NULL
 * keep_bits with dropout), FA_ERR_WORKSPACE (keep_bits_bytes too small),
 * FA_ERR_ALIGNMENT, FA_ERR_UNSUPPORTED (N > FA_MASK_MAX_N with dropout). */
int fa_forward_keep(const void* q, const void* k, const void* v, void* o, float* lse,
                    int B, int H, int N, int d, float scale, int causal,
                    const int32_t* cu_seqlens, float dropout_p, uint64_t seed, void* stream,
                    int dtype, int64_t ld_qkv, uint32_t* keep_bits, size_t keep_bits_bytes);

/* fa_backward, reading the dropout decisions from keep_bits as
 * fa_forward_keep wrote them for the same shapes, cu_seqlens, dropout_p and
 * seed (the seed is then unused).  With dropout_p == 0 it is exactly
 * fa_backward.  Errors: those of fa_backward and of fa_forward_keep. */
int fa_backward_keep(const void* q, const void* k, const void* v, const void* o, const float* lse,
                     const void* dout, void* dq, void* dk, void* dv, int B, int H, int N, int d,
                     float scale, int causal, const int32_t* cu_seqlens, float dropout_p,
                     uint64_t seed, void* stream, int dtype, int64_t ld_qkv, void* workspace,
                     size_t workspace_bytes, const uint32_t* keep_bits, size_t keep_bits_bytes);

/* One of the two kernels of fa_backward_keep (stage 0: D and dQ, stage 1: dK
 * and dV), as fa_backward_stage is for fa_backward. */
int fa_backward_keep_stage(int stage, const void* q, const void* k, const void* v, const void* o,
                           const float* lse, const void* dout, void* dq, void* dk, void* dv, int B, int H,
                           int N, int d, float scale, int causal, const int32_t* cu_seqlens,
                           float dropout_p, uint64_t seed, void* stream, int dtype, int64_t ld_qkv,
                           void* workspace, size_t workspace_bytes, const uint32_t* keep_bits,
                           size_t keep_bits_bytes);

/* ------------------------------------------------------ KV-cache decode
 * One decode step of inference with a KV cache (lab write-up, section 6.1):
 * nq new query tokens of each sequence attend to that sequence's cached keys
 * and values, the new tokens being the last nq positions of the sequence.
 *   q, o        : [B, nq, H, d] contiguous (o: output, dtype).
 *   k_cache,
 *   v_cache     : [B, nk_max, H, d] contiguous; the first seqlens_k[b]
 *                 tokens of sequence b are valid (all nk_max if seqlens_k is
 *                 NULL).
 *   seqlens_k   : DEVICE int32 [B] or NULL; values are clamped to
 *                 [0, nk_max].
 *   lse         : output, float32 [B, nq, H] (natural log).
 *   causal      : query t (0 <= t < nq) sees keys j <= L - nq + t
 *                 (bottom-right alignment); otherwise every valid key.  A
 *                 query that sees no key gets O = 0, lse = -inf.
 *   workspace   : DEVICE memory of fa_decode_workspace_size() bytes, 16-byte
 *                 aligned, no initialisation needed (fp32 partial results of
 *                 the 1024-key chunks).
 * 1 <= nq <= FA_DECODE_MAX_Q, d in {64, 128}, nk_max >= 1.  Errors as for
 * fa_forward (FA_ERR_WORKSPACE for a missing or short workspace).  Enqueues
 * a split kernel (one workgroup per sequence, head and 1024-key chunk) and a
 * merge kernel (log-sum-exp weighted sum of the chunks, the online-softmax
 * rule of section 3.2 of the lab write-up). */
#define FA_DECODE_MAX_Q 8

size_t fa_decode_workspace_size(int B, int H, int nq, int nk_max, int d);

int fa_decode(const void* q, const void* k_cache, const void* v_cache, const int32_t* seqlens_k,
              void* o, float* lse, int B, int H, int nq, int nk_max, int d, float scale,
              int causal, void* stream, int dtype, void* workspace, size_t workspace_bytes);

/* The same decode step over a paged cache: the keys and values of all
 * sequences live in two pools of fixed-size pages, and a block table maps
 * each sequence's cache positions to pages, so that caches can grow page by
 * page without being copied.  The attention computed is exactly that of
 * fa_decode on the cache the table describes.
 *   k_pages,
 *   v_pages     : [num_pages, page_size, H, d] contiguous (16-byte aligned).
 *   block_table : DEVICE int32 [B, max_pages]: cache position j of sequence
 *                 b is token j % page_size of page
 *                 block_table[b * max_pages + j / page_size].  Only the
 *                 entries covering positions below seqlens_k[b] are read.
 *                 Entries must lie in [0, num_pages); an entry outside is
 *                 clamped into that range (every read stays inside the
 *                 pools, the output is then unspecified).
 *   seqlens_k   : DEVICE int32 [B] or NULL (every sequence holds
 *                 max_pages * page_size tokens); clamped to
 *                 [0, max_pages * page_size].
 *   page_size   : a power of two.
 * q, o, lse, causal, scale, dtype and the limits on nq and d are those of
 * fa_decode; the workspace is fa_decode_workspace_size(B, H, nq,
 * max_pages * page_size, d) bytes.  Errors as for fa_decode, and
 * FA_ERR_UNSUPPORTED for a page size that is not a power of two. */
int fa_decode_paged(const void* q, const void* k_pages, const void* v_pages, const int32_t* block_table,
                    const int32_t* seqlens_k, void* o, float* lse, int B, int H, int nq, int num_pages,
                    int page_size, int max_pages, int d, float scale, int causal, void* stream, int dtype,
                    void* workspace, size_t workspace_bytes);

/* Dropout keep mask of a single (b, h) head as the fused kernels draw it:
 * keep[i * N + j] = 1 if element (i, j) is kept, 0 if dropped, for
 * 0 <= i, j < N (both local indices; causal masking is NOT applied).  keep
 * is a device buffer of N*N bytes.  The decision for (i, j) depends on
 * (seed, b, h, i, j) only, not on N, so for packed variable-length input
 * the mask of sequence s is this call with b = s and N = its length (its
 * top-left L x L block for any larger N).  Exposes the kernels' hash so
 * that tests can compare it bit for bit with an independent implementation;
 * a full [B, H, N, N] export is not offered (at 16 sequences of 4096 tokens
 * and 32 heads it would be 8.6 GB of bytes). */
int fa_dropout_mask(uint8_t* keep, int b, int h, int N, float dropout_p, uint64_t seed,
                    void* stream);

/* Static description of an error code (never NULL). */
const char* fa_strerror(int code);

#ifdef __cplusplus
}
#endif

#endif /* FA_H_ */
