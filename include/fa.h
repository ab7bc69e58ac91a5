/*
 * fa.h — C ABI of the fused exact-attention library for AMD Instinct MI355X (gfx950).
 *
 * What it computes, per (batch b, head h), with queries i and keys j in [0, N):
 *
 *     S_ij  = softmax_scale * <Q_i, K_j>            (scaled dot products)
 *     S_ij  = -inf where key j is hidden from query i (causal / sliding window)
 *     O_i   = sum_j softmax_j(S_i) V_j
 *     LSE_i = ln sum_j exp(S_ij)                    (natural log, over visible keys)
 *
 * This is the formula softmax(QK^T / sqrt(d_k)) V of the page "PyTorch-CUDA-v2.9镜像中使用
 * FlashAttention提升训练速度" (section "FlashAttention：不只是更快的 Attention"), computed the
 * way the page "告别OOM和训练慢：用Flash Attention加速你的PyTorch大模型（含A100环境配置）"
 * describes in §2.1 (tiling) and §2.2 (running max / running sum, keeping only the
 * normalisation statistics for the backward pass): one fused kernel, the N x N score
 * matrix never reaches device memory.  The argument set is the one of that page's §4.2
 * (softmax_scale, causal, window_size) and of the SDPA call of "Flash Attention 3.7 核心原理与
 * 实战：加速Transformer模型训练与推理" §3.2 ((batch, num_heads, seq_len, head_dim) tensors).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  Layout     Q, K, V, O, dO, dQ, dK, dV are dense row-major [B, H, N, d] arrays of
 *             `dtype` elements (last dimension contiguous, no padding).  LSE is a dense
 *             [B, H, N] float32 array; the backward workspace holds two of them.
 *  Memory     Every pointer is a device pointer the caller allocated (hipMalloc or any
 *             allocator handing out device memory).  The library allocates nothing and
 *             keeps no per-call state; it never takes ownership.  Array pointers must be
 *             16-byte aligned.  Outputs must not be the same buffer as an input.
 *  Shapes     B, H, N >= 0 (a zero makes the call a no-op that returns FA_OK; pointers
 *             may then be NULL).  head_dim (d) must be 64 or 128.  N * d must be below
 *             2^30 and B * H * N below 2^31.
 *  Masks      causal != 0 hides keys j > i.  window_left / window_right >= 0 hide keys
 *             j < i - window_left / j > i + window_right (bounds inclusive); -1 means
 *             unbounded; values below -1 are rejected.  Causal and window combine (AND).
 *  Scale      any finite float (0 gives the plain mean over visible keys).  Callers who
 *             want the default use 1/sqrt(head_dim).
 *  Precision  inputs fp16 or bf16; products accumulate in fp32; the probabilities are
 *             rounded once to the input type (round to nearest even) before the P·V
 *             product; O (and dQ, dK, dV) are rounded to the input type at the end.
 *  Streams    `stream` is a hipStream_t (NULL = the default stream).  Calls only
 *             enqueue work and return; the caller orders and synchronises.
 *  Errors     Arguments are validated on the host before any HIP call; an invalid call
 *             returns its status and enqueues nothing.  A failed launch returns
 *             FA_ERR_HIP (details from fa_last_error_detail()).  There is no silent
 *             fallback to another algorithm or device.
 *  Results    are deterministic: identical inputs give bit-identical outputs.
 */
#ifndef FA_H_
#define FA_H_

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum fa_status {
  FA_OK = 0,
  FA_ERR_NULL_PTR = 1,            /* a required pointer is NULL                        */
  FA_ERR_BAD_SHAPE = 2,           /* negative or too large B, H, N                     */
  FA_ERR_UNSUPPORTED_HEAD_DIM = 3,/* head_dim not in {64, 128}                          */
  FA_ERR_BAD_DTYPE = 4,           /* dtype not FA_F16 / FA_BF16                         */
  FA_ERR_BAD_WINDOW = 5,          /* window bound below -1                              */
  FA_ERR_MISALIGNED = 6,          /* a pointer is not 16-byte aligned                   */
  FA_ERR_BAD_SCALE = 7,           /* softmax_scale is NaN or infinite                   */
  FA_ERR_WORKSPACE = 8,           /* backward workspace NULL or smaller than required   */
  FA_ERR_HIP = 9,                 /* the HIP runtime reported an error                  */
  FA_ERR_ALIAS = 10,              /* an output buffer is also an input buffer           */
  FA_ERR_BAD_STAGES = 11,         /* fa_bwd_stages: empty mask or unknown stage bits     */
  FA_ERR_BAD_DROPOUT = 12,        /* dropout_p outside [0, 1)                           */
  FA_ERR_TOO_LARGE = 13           /* fa_bwd_noalloc: the shape needs more than its
                                     static scratch holds                               */
} fa_status;

typedef enum fa_dtype { FA_F16 = 0, FA_BF16 = 1 } fa_dtype;

/* Version of this ABI (major * 100 + minor). */
int fa_version(void);

/* Forward pass.
 *   q, k, v  in:  [B, H, N, d] dtype
 *   o        out: [B, H, N, d] dtype
 *   lse      out: [B, H, N] float32, ln sum_j exp(S_ij) per query (may be NULL when the
 *            caller needs no backward pass; the backward pass requires it)
 * Every query has at least its own key visible (the diagonal), so O and LSE are always
 * finite for finite inputs. */
fa_status fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                 int batch, int heads, int seqlen, int head_dim, fa_dtype dtype,
                 float softmax_scale, int causal, int window_left, int window_right,
                 void* stream);

/* Bytes of device workspace fa_bwd needs for this shape: float32 per-query statistics,
 * -LSE / sigma and -rowsum(dO * O) (sigma is softmax_scale moved at least 1e-30 away from
 * zero), stored per (batch, head) in blocks of 32 queries (32 of each, 256 bytes per block,
 * the last block padded with zeros): 8 * B * H * ceil(N / 32) * 32 bytes.  Returns 0 for
 * invalid or empty shapes. */
size_t fa_bwd_workspace_size(int batch, int heads, int seqlen, int head_dim);

/* Backward pass by recomputation: P is rebuilt tile by tile from Q, K and the saved LSE
 * (the forward's own output), so neither S nor P is ever stored — the recomputation
 * the page "PyTorch-CUDA-v2.9镜像中使用FlashAttention提升训练速度" names as its third
 * technique ("3. 重计算策略（Recomputation）").
 *   q, k, v, o, dout  in:  [B, H, N, d] dtype (o and lse from fa_fwd on the same inputs)
 *   lse               in:  [B, H, N] float32
 *   dq, dk, dv        out: [B, H, N, d] dtype, gradients of sum(dout * o)
 *   workspace         scratch of at least fa_bwd_workspace_size() bytes, 16-byte aligned;
 *                     its contents on entry do not matter and are clobbered.
 * Masks and scale must be those of the forward call. */
fa_status fa_bwd(const void* q, const void* k, const void* v, const void* o,
                 const void* dout, const float* lse, void* dq, void* dk, void* dv,
                 void* workspace, size_t workspace_bytes,
                 int batch, int heads, int seqlen, int head_dim, fa_dtype dtype,
                 float softmax_scale, int causal, int window_left, int window_right,
                 void* stream);

/* The backward pass has three stages.  fa_bwd runs all of them; fa_bwd_stages runs the
 * subset in `stages` (a bitwise OR of the values below), for callers that time or schedule
 * them one by one.  Same arguments as fa_bwd.  The stages depend on each other through the
 * workspace and the outputs: a call for a later stage must follow (on the same stream, with
 * the same arguments and workspace) the calls for every earlier stage.
 *   FA_BWD_DELTA  workspace <- -lse / sigma and -rowsum(dout * o) per query
 *   FA_BWD_DKDV   dk, dv    (reads workspace)
 *   FA_BWD_DQ     dq        (reads workspace)
 * A call that holds FA_BWD_DELTA and FA_BWD_DQ (fa_bwd's among them) runs them, on the main
 * kernels, as one kernel that forms the statistics of its queries, writes them to the workspace
 * and computes dq; FA_BWD_DKDV then follows it.  The workspace and every output are the same,
 * bit for bit, as those of the stages run one by one. */
typedef enum fa_bwd_stage {
  FA_BWD_DELTA = 1,
  FA_BWD_DKDV = 2,
  FA_BWD_DQ = 4,
  FA_BWD_ALL = 7
} fa_bwd_stage;

fa_status fa_bwd_stages(const void* q, const void* k, const void* v, const void* o,
                        const void* dout, const float* lse, void* dq, void* dk, void* dv,
                        void* workspace, size_t workspace_bytes,
                        int batch, int heads, int seqlen, int head_dim, fa_dtype dtype,
                        float softmax_scale, int causal, int window_left, int window_right,
                        unsigned stages, void* stream);

/* ---- Backward pass without allocation ---------------------------------------------------
 * For callers that cannot allocate device memory or pass a workspace: code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation.  fa_bwd_noalloc is fa_bwd
 * with its per-query statistics kept in a static device array of FA_NOALLOC_SCRATCH_BYTES
 * bytes that the library holds on each GPU it runs on until the process ends; it calls no
 * allocator.  Arguments, results and errors are those of fa_bwd without the workspace
 * arguments, plus FA_ERR_TOO_LARGE when fa_bwd_workspace_size() of the shape exceeds
 * FA_NOALLOC_SCRATCH_BYTES (16 MiB: B * H * ceil(N / 32) * 32 <= 2^21 query slots, e.g.
 * B * H = 128 heads of N = 16384).  The array of the calling thread's current device is used
 * (the stream must belong to that device); its address is looked up on the first call on each
 * device.  Every call on one device shares that device's array, so calls that may overlap on
 * one device (different streams, different host threads) race and must be ordered by the
 * caller.  Results are bit-identical to fa_bwd's. */
#define FA_NOALLOC_SCRATCH_BYTES (16u << 20)

fa_status fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                         const void* dout, const float* lse, void* dq, void* dk, void* dv,
                         int batch, int heads, int seqlen, int head_dim, fa_dtype dtype,
                         float softmax_scale, int causal, int window_left, int window_right,
                         void* stream);

/* Padded batches: sequence b is rows 0 .. L_b - 1 of its N rows (every head of batch b), the
 * remaining rows are padding.  This is the per-sample actual length the page "告别OOM和训练慢：
 * 用Flash Attention加速你的PyTorch大模型（含A100环境配置）" passes to its length-grouped batch
 * attention (§6), on the padded [B, H, N, d] layout whose keys the page "Flash Attention 3.7
 * 核心原理与实战：加速Transformer模型训练与推理" hides with a key padding mask (§4.2).  Each
 * sample is attention over its own L_b rows alone:
 *   - keys j >= L_b are hidden from every query;
 *   - rows i >= L_b are written as O_i = 0 and LSE_i = -inf (fa_fwd_varlen), and as zero
 *     dQ_i, dK_i, dV_i (fa_bwd_varlen); their Q, K, V, O and dO rows are never used.
 *   seqlens  in: device int32[B], the lengths L_b.  Read by the kernels, so it is not
 *            checked on the host: a value below 0 counts as 0 and one above N as N.  It must
 *            be 4-byte aligned and must not be an output buffer (FA_ERR_ALIAS).
 * Every other argument, convention and error is that of fa_fwd / fa_bwd_stages (`stages` as
 * there: FA_BWD_ALL for the whole backward pass); seqlens NULL gives FA_ERR_NULL_PTR.  A row
 * i < L_b sees at least its own key, as in fa_fwd.  The backward call needs the forward's o
 * and lse of the same seqlens, and the workspace size of fa_bwd. */
fa_status fa_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                        const int* seqlens, int batch, int heads, int seqlen, int head_dim,
                        fa_dtype dtype, float softmax_scale, int causal, int window_left,
                        int window_right, void* stream);

fa_status fa_bwd_varlen(const void* q, const void* k, const void* v, const void* o,
                        const void* dout, const float* lse, void* dq, void* dk, void* dv,
                        void* workspace, size_t workspace_bytes, const int* seqlens, int batch,
                        int heads, int seqlen, int head_dim, fa_dtype dtype, float softmax_scale,
                        int causal, int window_left, int window_right, unsigned stages,
                        void* stream);

/* Packed batches: the sequences of a batch concatenated per head, with no padding.  This is
 * the per-sample actual length of the A100 page (§6) on the (batch, num_heads, seq_len,
 * head_dim) layout of the FA3.7 page's SDPA call (§3.2) with the batch folded into the
 * sequence axis:
 *   q, k, v, o, dout, dq, dk, dv  [H, total, head_dim] of dtype, dense: head h holds the
 *            `total` rows of every sequence, sequence b being rows cu_seqlens[b] ..
 *            cu_seqlens[b+1] - 1;
 *   lse      [H, total] float32;
 *   cu_seqlens  device int32[B + 1], the sequences' start rows and the end of the last one
 *            (4-byte aligned, not an output).  Read by the kernels, so not checked on the
 *            host: each offset is clamped to [0, total], each sequence to [cu[b], cu[b+1])
 *            and to at most max_seqlen rows.
 *   max_seqlen  the longest sequence (sizes the grid and the backward workspace,
 *            fa_bwd_workspace_size(batch, heads, max_seqlen, head_dim) bytes).
 * Each sequence is attention over its own rows alone, with the masks of fa_fwd; rows no
 * sequence covers are neither read nor written.  Other arguments, conventions and errors are
 * those of fa_fwd / fa_bwd_stages (`stages` as there); total < 0, total * head_dim >= 2^30 or
 * heads * total >= 2^31 give FA_ERR_BAD_SHAPE, and total = 0 is a no-op.  The results are
 * bit-identical to fa_fwd_varlen / fa_bwd_varlen on the same sequences laid out padded. */
fa_status fa_fwd_packed(const void* q, const void* k, const void* v, void* o, float* lse,
                        const int* cu_seqlens, int batch, int heads, int total, int max_seqlen,
                        int head_dim, fa_dtype dtype, float softmax_scale, int causal,
                        int window_left, int window_right, void* stream);

fa_status fa_bwd_packed(const void* q, const void* k, const void* v, const void* o,
                        const void* dout, const float* lse, void* dq, void* dk, void* dv,
                        void* workspace, size_t workspace_bytes, const int* cu_seqlens, int batch,
                        int heads, int total, int max_seqlen, int head_dim, fa_dtype dtype,
                        float softmax_scale, int causal, int window_left, int window_right,
                        unsigned stages, void* stream);

/* Queries and keys of different lengths, and operands of any layout.
 *
 * N_q queries attend to N_k keys, and the queries are the LAST N_q positions of the key
 * sequence: query i sits at key position p_i = i + (N_k - N_q), and every mask is applied to
 * positions (causal hides keys j > p_i; the window hides j < p_i - window_left and
 * j > p_i + window_right).  A decode step of a language model (N_q = 1) over its KV cache
 * thus sees every cached key, and a block of new queries sees the cache and its own causal
 * prefix — the inference use the page "Flash Attention 3.7 核心原理与实战：加速Transformer模型训练
 * 与推理" names (§1.3) over the KV cache that the page "PyTorch-CUDA-v2.9镜像中使用
 * FlashAttention提升训练速度" mentions in its closing section.  With N_q = N_k this is fa_fwd.
 * A query that sees no key (possible when N_q > N_k under causal, or with a window) gets
 * O_i = 0 and LSE_i = -inf.
 *
 *   q, o     [B, H, N_q, head_dim], k, v [B, H, N_k, head_dim], dtype, each with its own
 *            strides (below); lse out: dense [B, H, N_q] float32, or NULL.
 *   strides  NULL for dense [B, H, N, d] arrays, else an array of four fa_strides, for q, k,
 *            v and o in that order.  Element (b, h, r, c) of an operand is at
 *            base + b * batch + h * head + r * row + c (in elements).  Every stride must be
 *            >= 0 and a multiple of 8 elements (16 bytes); (rows + 256) * row * 2 must be
 *            below 2^31 for each operand.  A stride of 0 shares rows: k and v with head
 *            stride 0 serve every head from one key/value head.  The (batch, seq, heads,
 *            head_dim) layout behind the transposed views of that page's §4.2 module has
 *            strides {N H d, d, H d}.  The elements of o must not overlap one another (not
 *            checked).
 *   workspace  device scratch of at least fa_fwd_kv_workspace_size() bytes (16-byte aligned;
 *            NULL allowed when that size is 0).  Long key sequences are split into parts that
 *            run in parallel; each part's normalised output and LSE go here and are merged by
 *            the log-sum-exp rule.  Its contents on entry do not matter.
 * N_q = 0 (or B = 0, H = 0) is a no-op; N_k = 0 writes O = 0 and LSE = -inf (k and v may be
 * NULL then).  Other conventions and errors as in fa_fwd; FA_ERR_BAD_SHAPE also reports a
 * stride outside the rules above.  Results depend on the shape only (not on the device).
 * Precision: with N_q <= 4 the probabilities stay in float32 for the P V sum (no rounding to
 * the input type); otherwise as in fa_fwd.
 *
 * ALiBi: alibi_slopes is a device float32 array [heads] (4-byte aligned, not an output), or
 * NULL for none.  Head h then subtracts slope_h * |p_i - j| from every scaled score before
 * the mask and the softmax: S_ij = softmax_scale * <Q_i, K_j> - slope_h * |p_i - j|, a penalty
 * linear in the distance between the query's and the key's positions.  These are the "linear
 * bias coefficients" the page "告别OOM和训练慢：用Flash Attention加速你的PyTorch大模型（含A100环境配置）"
 * lists as alibi_slopes in §4.2 (and the ALiBi relative position encoding "Flash Attention
 * 3.7 核心原理与实战" names for very long sequences in §6).  The values are read by the kernels
 * and not checked: they must be finite.  fa_bwd_kv takes the same slopes.
 *
 * Dropout: with dropout_p in (0, 1) the weights that multiply V are P_ij * M_ij / r, M_ij in
 * {0, 1} kept with probability r (about 1 - p), so that their expectation is P_ij, as the
 * dropout_p argument of the attention calls of the A100 page (§4.2)
 * and of the SDPA call of the FA3.7 page (§3.2) and the F.dropout of that page's §4.2 module
 * (applied to the softmax weights before V) describe; LSE is that of the softmax before
 * dropout.  M comes from Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel Random
 * Numbers: As Easy as 1, 2, 3", SC 2011), so a call is reproducible: one generator call with
 * counter (j >> 2, i >> 1, batch * heads + head, dropout_offset) and key dropout_seed (low
 * word first) draws 16 bits for each of queries 2 (i >> 1) + {0, 1} and keys
 * 4 (j >> 2) + {0 .. 3}; pair (i, j) takes half-word t = 4 (i & 1) + (j & 3) (word t >> 1,
 * its high half when t is odd) and is kept when that value is at least floor(p 2^16).  The
 * keep probability is thus r = (2^16 - floor(p 2^16)) / 2^16, and kept weights are scaled by
 * 1 / r = 2^16 / (2^16 - floor(p 2^16)) (rounded to float32).  dropout_p = 0 is no dropout;
 * values outside [0, 1) give FA_ERR_BAD_DROPOUT.  fa_bwd_kv must get the forward's p, seed and
 * offset.  With dropout, calls with N_q <= 4 take the MFMA kernel.
 *
 * Block-sparse attention: block_mask is a device uint8 array [heads][ceil(N_q / 64)]
 * [ceil(N_k / 64)] (dense, C order), or NULL for none.  Entry (h, a, c) nonzero selects the
 * block of queries 64 a .. 64 a + 63 and keys 64 c .. 64 c + 63 of head h (every batch); a pair
 * in an unselected block is hidden like a masked pair (its score is -inf), and unselected
 * blocks are skipped, not computed.  This is the block-sparse FlashAttention the A100 page
 * lists among its next steps (§6) and the sparse attention the FA3.7 page names for very long
 * sequences (§6); neither fixes a pattern.  It combines with causal, window, ALiBi and dropout;
 * a query whose row selects no visible key gets O = 0, LSE = -inf.  It must not be an output
 * buffer; fa_bwd_kv must get the forward's mask.
 *
 * Key padding mask: key_padding_mask is a device uint8 array [batch][N_k] (dense, C order), or
 * NULL for none.  Entry (b, j) nonzero marks key j of batch entry b as padding: it is hidden
 * from every query of that entry in every head (its scores are -inf), as the key_padding_mask
 * argument of the attention module in §4.2 of the FA3.7 page hides padding keys before the
 * softmax (the PyTorch-CUDA-v2.9 page, section "如何集成 FlashAttention：从安装到应用", names the
 * same argument).  Padding keys may sit anywhere, not only at the end of a sequence; it
 * combines with every other mask, ALiBi and dropout; a query left with no visible key gets
 * O = 0, LSE = -inf, and a padding key gets dK = dV = 0.  Key tiles made only of padding keys
 * are skipped.  It must not be an output buffer; fa_bwd_kv must get the forward's mask. */
typedef struct fa_strides {
  long long batch, head, row;
} fa_strides;

size_t fa_fwd_kv_workspace_size(int batch, int heads, int seqlen_q, int seqlen_k, int head_dim);

fa_status fa_fwd_kv(const void* q, const void* k, const void* v, void* o, float* lse,
                    const fa_strides* strides, int batch, int heads, int seqlen_q, int seqlen_k,
                    int head_dim, fa_dtype dtype, float softmax_scale, int causal,
                    int window_left, int window_right, const float* alibi_slopes,
                    const unsigned char* block_mask, const unsigned char* key_padding_mask,
                    float dropout_p, unsigned long long dropout_seed, unsigned dropout_offset,
                    void* workspace, size_t workspace_bytes, void* stream);

/* Backward pass of fa_fwd_kv (by recomputation, as fa_bwd): gradients of sum(dout * o) for
 * N_q queries over N_k keys with the queries at the end of the key sequence.
 *   q, o, dout, dq   [B, H, N_q, head_dim]; k, v, dk, dv [B, H, N_k, head_dim]; dtype
 *   lse              in: dense [B, H, N_q] float32 from fa_fwd_kv (-inf for rows without keys)
 *   strides          NULL for dense arrays, else eight fa_strides for q, k, v, o, dout, dq, dk,
 *                    dv in that order, under the rules of fa_fwd_kv.  Inputs may share rows
 *                    (e.g. head stride 0 for k, v); the elements of each output must not
 *                    overlap, so with shared key/value heads dk and dv hold one gradient per
 *                    query head, which the caller sums.
 *   workspace        at least fa_bwd_workspace_size(batch, heads, seqlen_q, head_dim) bytes,
 *                    16-byte aligned; contents on entry do not matter.
 * A row without keys has dQ = 0; with N_q = 0, dK = dV = 0 (and q, o, dout, lse, dq may be
 * NULL); with N_k = 0, dQ = 0 (k, v, dk, dv may be NULL).  Masks, scale, alibi_slopes,
 * block_mask, key_padding_mask and the dropout arguments must be those of the forward call.
 * Errors as in fa_bwd and fa_fwd_kv. */
fa_status fa_bwd_kv(const void* q, const void* k, const void* v, const void* o, const void* dout,
                    const float* lse, void* dq, void* dk, void* dv, const fa_strides* strides,
                    void* workspace, size_t workspace_bytes, int batch, int heads, int seqlen_q,
                    int seqlen_k, int head_dim, fa_dtype dtype, float softmax_scale, int causal,
                    int window_left, int window_right, const float* alibi_slopes,
                    const unsigned char* block_mask, const unsigned char* key_padding_mask,
                    float dropout_p, unsigned long long dropout_seed, unsigned dropout_offset,
                    void* stream);

/* ---- Decode steps over an FP8 key/value cache ------------------------------------------
 * fa_fwd_kv (no ALiBi, dropout or block mask; key_padding_mask as there) with K and V held as
 * FP8 E4M3 codes: the OCP
 * 8-bit floating-point format of sign, 4 exponent bits (bias 7) and 3 mantissa bits, largest
 * finite magnitude 448, smallest subnormal 2^-9, no infinities, codes 0x7F and 0xFF NaN.
 * Key element (b, h, r, c) is k_descale * value(code), value element v_descale * value(code).
 * The A100 page lists FP8 support among its next steps (§6); the cache a decode step reads is
 * the KV cache of the LLM inference the FA3.7 page names (§1.3) and that PagedAttention pages
 * through memory (closing section of the PyTorch-CUDA-v2.9 page).  A decode step is bound by
 * the bytes it reads, and one-byte keys and values halve them.  The scores and the output are
 * computed in fp32 from the exact decoded values, as in fa_fwd_kv.
 *
 *   q, o       [B, H, N_q, head_dim] of dtype (fp16 or bf16); lse out: dense [B, H, N_q]
 *              float32 or NULL.
 *   k, v       [B, H, N_k, head_dim] FP8 E4M3 codes, one byte per element.
 *   strides    NULL (dense) or four fa_strides for q, k, v, o, in elements (one byte for k and
 *              v), each >= 0 and a multiple of 8; the bounds of fa_fwd_kv apply.
 *   seqlen_q   0 .. 4; a larger N_q gives FA_ERR_BAD_SHAPE.
 *   k_descale, v_descale  finite and > 0, else FA_ERR_BAD_SCALE.
 *   workspace  at least fa_fwd_kv_workspace_size() bytes for the same sizes (16-byte aligned);
 *              it holds the partial results of key splits.
 * NaN codes in k or v are outside the domain (not checked).  The reading of positions, masks,
 * rows without keys and the other errors are those of fa_fwd_kv. */
fa_status fa_fwd_kv_fp8(const void* q, const void* k, const void* v, void* o, float* lse,
                        const fa_strides* strides, int batch, int heads, int seqlen_q,
                        int seqlen_k, int head_dim, fa_dtype dtype, float softmax_scale,
                        float k_descale, float v_descale, int causal, int window_left,
                        int window_right, const unsigned char* key_padding_mask, void* workspace,
                        size_t workspace_bytes, void* stream);

/* ---- Forward over FP8 E4M3 queries, keys and values -----------------------------------
 * fa_fwd with Q, K and V held as E4M3 codes (the format of fa_fwd_kv_fp8 above: the OCP 8-bit
 * floating-point format, sign / 4 exponent bits with bias 7 / 3 mantissa bits, largest
 * magnitude 448, 0x7F and 0xFF NaN) and one descale factor per tensor: query element
 * (b, h, i, c) is q_descale * value(code), and likewise for keys and values.  The attention is
 * fa_fwd's over those exact values:
 *     S_ij = softmax_scale * q_descale * k_descale * sum_c value(Q_ic) value(K_jc),
 *     O_i = v_descale * sum_j softmax_j(S_i) value(V_j),  LSE_i = ln sum_j exp(S_ij),
 * with fa_fwd's masks.  FP8 support is among the next steps the page "告别OOM和训练慢：用Flash
 * Attention加速你的PyTorch大模型（含A100环境配置）" lists (§6).  Both products run on gfx950's
 * FP8 matrix instruction with fp32 accumulation; the probabilities enter the second product
 * rounded to E4M3 (after an exact power-of-two scaling that keeps them in its normal range),
 * so each output carries a relative rounding of up to 2^-4 per weight on top of fa_fwd's;
 * the row sums and LSE use the unrounded probabilities in fp32.
 *   q, k, v    in:  [B, H, N, head_dim] E4M3 codes, one byte per element, dense, 16-byte aligned
 *   o          out: [B, H, N, head_dim] of out_dtype (FA_F16 or FA_BF16)
 *   lse        out: [B, H, N] float32, or NULL
 *   q_descale, k_descale, v_descale  finite and > 0, else FA_ERR_BAD_SCALE
 * NaN codes are outside the domain (not checked).  Other arguments, conventions and errors are
 * those of fa_fwd. */
fa_status fa_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse,
                     int batch, int heads, int seqlen, int head_dim, fa_dtype out_dtype,
                     float softmax_scale, float q_descale, float k_descale, float v_descale,
                     int causal, int window_left, int window_right, void* stream);

/* Static, human-readable name of a status code. */
const char* fa_status_string(fa_status s);

/* Text of the last HIP error seen by this thread (empty if none); valid until the next
 * call on this thread. */
const char* fa_last_error_detail(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_H_ */
