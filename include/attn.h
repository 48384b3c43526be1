/*
 * attn.h -- C ABI of libattn.so: exact attention on AMD MI355X (gfx950).
 *
 * The attention entry points are FA-2 style tiled computation that never writes
 * the N x N score or probability matrix to device memory:
 *
 *   attn_fwd                O = softmax(scale * Q K^T) V and the per-row
 *                           log-sum-exp.
 *   attn_fwd_splitk_decode  the same for a single query row against a long
 *                           key/value cache, split into chunks whose partial
 *                           (U, m, l) states are merged afterwards.
 *   attn_fwd_splitk_decode_paged
 *                           the same decode over a paged cache addressed
 *                           through a per-sequence block table.
 *   attn_fwd_merge          the forward combined in place with a running (O, LSE).
 *   attn_bwd                dQ, dK, dV by recomputing P from the saved LSE.
 *   attn_bwd_atomic_dq      the same with dQ accumulated by atomic adds.
 *   attn_quantize_fp8, attn_fwd_fp8
 *                           FP8 (E4M3) storage with per-block scales, and
 *                           the forward on it.
 *   attn_merge              (O, LSE) over two disjoint key sets -> over
 *                           their union (Ring Attention's per-shard update).
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers, owned by the caller.  The
 *     library never allocates, frees or retains them beyond the call.
 *   - Tensors are dense, row-major [B, H, rows, d] with d fastest
 *     (the [batch, heads, sequence, head_dim] layout of PyTorch's
 *     scaled_dot_product_attention, described on the "FlashAttention" page of
 *     xuesongtap.github.io, section 6), and 16-byte aligned.
 *   - Every call only enqueues kernels on `stream` (a hipStream_t; NULL is the
 *     null stream) and returns; the caller synchronises.  Argument checks run
 *     on the host before any HIP call, so an error status means nothing was
 *     launched.  No C++ exception crosses the ABI.
 *   - `scale` multiplies Q K^T before the softmax and must be finite and > 0;
 *     the usual value is 1/sqrt(d).
 *   - `causal` != 0 masks key index j > query index i (square problem,
 *     top-left aligned): "FlashAttention" (xuesongtap), section 2.2.
 *   - LSE values are natural-log log-sum-exp of the scaled scores,
 *     LSE_i = m_i + ln(l_i) (xuesongtap, section 3), stored as fp32.
 *   - Supported: dtype ATTN_BF16 with d in {64, 128}; dtype ATTN_F32 with
 *     d == 64 (forward only).  Other combinations return
 *     ATTN_ERR_UNSUPPORTED.  Accumulation is always fp32; outputs in the
 *     input dtype are rounded to nearest even.
 */
#ifndef ATTN_H
#define ATTN_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ATTN_OK = 0,
  ATTN_ERR_INVALID_ARG = 1, /* null/misaligned pointer, bad size, bad scale */
  ATTN_ERR_UNSUPPORTED = 2, /* dtype/head_dim combination not built */
  ATTN_ERR_WORKSPACE = 3,   /* workspace missing or smaller than required */
  ATTN_ERR_HIP = 4,         /* a HIP launch reported an error */
  ATTN_ERR_SCRATCH = 5      /* a no-allocation call needs more than the fixed scratch */
} attn_status;

typedef enum { ATTN_F32 = 0, ATTN_BF16 = 1 } attn_dtype;

/* Human-readable name of a status code (static storage, never NULL). */
const char* attn_status_string(attn_status s);

/* Version of this ABI (incremented on incompatible changes). */
int attn_abi_version(void);

/*
 * attn_fwd -- exact attention forward.
 *
 * Computes, per (b, h), S = scale * Q K^T (masked if causal), P = softmax(S)
 * row-wise, O = P V, and LSE_i = log sum_j exp(S_ij): the definition in
 * "FlashAttention" (xuesongtap), section 1, evaluated with the FA-2 loop of
 * its sections 2.1-2.2 (outer loop over query tiles kept on chip, inner loop
 * over K/V tiles with the running state (m, l, U), O = U / l at the end) and
 * the LSE of its section 3.
 *
 *   q, k, v : [B, H, N, d] in `dtype` (read only)
 *   o       : [B, H, N, d] in `dtype` (written)
 *   lse     : [B, H, N] fp32 (written; may be NULL when not needed)
 *   B, H, N : >= 1;  B*H <= 2^31-1, N <= 2^24
 *
 * Errors: ATTN_ERR_INVALID_ARG for a NULL or non-16-byte-aligned q/k/v/o, a
 * 4-byte-misaligned lse, a size out of range or a bad scale;
 * ATTN_ERR_UNSUPPORTED for an unsupported (dtype, d);  ATTN_ERR_HIP when the
 * launch fails.
 */
attn_status attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                     int B, int H, int N, int d, attn_dtype dtype, float scale, int causal,
                     void* stream);

/*
 * Workspace size in bytes that attn_fwd_splitk_decode needs for the given
 * shape: B*H*num_splits*(d + 2) fp32 values.  Returns 0 for invalid sizes.
 */
size_t attn_decode_workspace_bytes(int B, int H, int d, int num_splits);

/*
 * attn_fwd_splitk_decode -- FlashDecoding split-K attention for one query
 * row per (b, h).
 *
 * The cache of length L is cut into `num_splits` chunks; chunk c covers keys
 * [floor(c*L/S), floor((c+1)*L/S)).  For each chunk a partial state is
 * computed (the map step of FlashDecoding, cnblogs article on FlashAttention
 * tiling, section 3 scenario B; the partial (m, l, O) of "FlashAttention 1 和
 * FlashAttention 2 的区别", section 6):
 *     m_c = max_j s_j,  l_c = sum_j e^(s_j - m_c),  U_c = sum_j e^(s_j - m_c) V_j
 * with s = scale * K_c q, and the partials are merged (the reduce step):
 *     m = max_c m_c, l = sum_c e^(m_c - m) l_c, U = sum_c e^(m_c - m) U_c,
 *     O = U / l,  LSE = m + ln l.
 * An empty chunk (S > L) has m_c = -inf, l_c = 0, U_c = 0 and weight 0.
 * There is no causal flag: the single query sees the whole cache.
 *
 *   q        : [B, H, 1, d] in `dtype`
 *   k_cache  : [B, H, L, d] in `dtype`;  v_cache : [B, H, L, d]
 *   o        : [B, H, 1, d] in `dtype` (written)
 *   lse      : [B, H] fp32 (written; may be NULL)
 *   workspace: device buffer of at least attn_decode_workspace_bytes(...)
 *              bytes, 16-byte aligned.  On return (after the stream
 *              completes) it holds the partials, fp32, in this order:
 *              U [B, H, S, d], then m [B, H, S] (natural-log units of the
 *              scaled score), then l [B, H, S].
 *   num_splits: 1 <= S <= 65535;  L <= 2^30.
 *
 * Supported: ATTN_BF16 with d in {64, 128}.
 * Errors as attn_fwd, plus ATTN_ERR_WORKSPACE for a NULL or short workspace.
 */
attn_status attn_fwd_splitk_decode(const void* q, const void* k_cache, const void* v_cache,
                                   void* o, float* lse, void* workspace, size_t workspace_bytes,
                                   int B, int H, int L, int d, int num_splits, attn_dtype dtype,
                                   float scale, void* stream);

/* Size of the fixed per-device scratch of attn_fwd_splitk_decode_noalloc. */
#define ATTN_DECODE_SCRATCH_BYTES ((size_t)32 << 20)

/*
 * attn_fwd_splitk_decode_noalloc -- attn_fwd_splitk_decode for callers that
 * cannot allocate device memory (code under HIP graph capture, allocation-free
 * serving loops, harnesses that forbid hipMalloc).
 *
 * Same operation, arguments and result as attn_fwd_splitk_decode, without the
 * workspace: the chunk partials go to a fixed scratch array of
 * ATTN_DECODE_SCRATCH_BYTES (32 MiB) that the library keeps on each device it
 * runs on until the process ends.  The call allocates nothing and uses the
 * scratch of the CURRENT device (hipGetDevice); `stream` must belong to that
 * device.  The scratch is not readable by the caller.
 *
 * Every call on a device shares that device's scratch: calls whose kernels
 * may overlap on one device (on different streams without ordering between
 * them) race and give undefined results.  Calls on one stream are ordered.
 *
 * Limit: attn_decode_workspace_bytes(B, H, d, num_splits) must not exceed
 * ATTN_DECODE_SCRATCH_BYTES, i.e. B*H*num_splits*(d + 2) <= 8388608; for
 * B*H = 512 and d = 128 that is up to 126 splits.
 *
 * Errors as attn_fwd_splitk_decode (no workspace errors), plus
 * ATTN_ERR_SCRATCH when the partials would not fit in the scratch (checked on
 * the host; nothing is launched).
 */
attn_status attn_fwd_splitk_decode_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                           void* o, float* lse, int B, int H, int L, int d,
                                           int num_splits, attn_dtype dtype, float scale, void* stream);

/*
 * attn_fwd_splitk_decode_paged -- the split-K decode of
 * attn_fwd_splitk_decode over a paged key/value cache.
 *
 * "FlashAttention 1 和 FlashAttention 2 的区别", section 13, names the paged
 * block table as a KV-cache layout that decode kernels are tuned for; the
 * layout is fixed here as follows.  The cache is a pool of `num_blocks`
 * blocks of `block_size` token rows per head; sequence b has
 * seq_lens[b] tokens, and its token t is row (t mod block_size) of pool block
 * block_table[b][t / block_size].  For every (b, h) the result is that of
 * attn_fwd_splitk_decode on the gathered cache of length L_b = seq_lens[b]:
 * chunk c covers tokens [floor(c*L_b/S), floor((c+1)*L_b/S)), and the chunk
 * partials are merged as described there.  A sequence with L_b = 0 gives
 * O = 0 and LSE = -inf.
 *
 *   q          : [B, H, 1, d] in `dtype`
 *   k_pool     : [num_blocks, H, block_size, d] in `dtype`;  v_pool likewise
 *   block_table: [B, max_blocks_per_seq] int32, DEVICE memory; entries past
 *                ceil(L_b / block_size) are not read
 *   seq_lens   : [B] int32, DEVICE memory
 *   o, lse, workspace, num_splits: as attn_fwd_splitk_decode (the workspace
 *                size is attn_decode_workspace_bytes(B, H, d, num_splits))
 *   block_size : a power of two, 1 <= block_size;
 *                max_blocks_per_seq * block_size <= 2^30
 *
 * The device-side values are not validated on the host (they are never
 * read there): a length outside [0, max_blocks_per_seq * block_size] is
 * clamped into it and a block id outside [0, num_blocks) is clamped into
 * it, so no access leaves the pool, but the result is then unspecified.
 *
 * Supported: ATTN_BF16 with d in {64, 128}.
 * Errors as attn_fwd_splitk_decode; ATTN_ERR_INVALID_ARG also for a NULL or
 * 4-byte-misaligned block_table or seq_lens, num_blocks < 1,
 * max_blocks_per_seq < 1 or a block_size that is not a power of two.
 */
attn_status attn_fwd_splitk_decode_paged(const void* q, const void* k_pool, const void* v_pool,
                                         const int* block_table, const int* seq_lens, void* o,
                                         float* lse, void* workspace, size_t workspace_bytes, int B,
                                         int H, int d, int num_blocks, int block_size,
                                         int max_blocks_per_seq, int num_splits, attn_dtype dtype,
                                         float scale, void* stream);

/*
 * attn_quantize_fp8 -- block quantisation of a bf16 tensor to FP8 (E4M3),
 * the storage format of attn_fwd_fp8 ("8. FlashAttention 实战",
 * triton-tutorial.pages.dev, sections 8.9.3-8.9.4, and 8.9.5 for the
 * rotation).
 *
 * Rows of each (b, h) are grouped into blocks of `block_rows` (the last one
 * may be shorter).  Optionally every row is first rotated,
 * y = (x o signs) H / sqrt(d) with H the Sylvester Hadamard matrix (an
 * orthogonal map: rotating Q and K with the same signs leaves Q K^T
 * unchanged).  Each block gets the page's scale max|y| / 448 (an fp32
 * division, correctly rounded; 1 for an all-zero block), and its values
 * become e4m3(clamp(y / scale, -448, 448)), y / scale again an fp32 division,
 * rounded to nearest even.
 *
 *   x          : [B, H, N, d] bf16
 *   signs      : d floats, each +1 or -1, DEVICE memory; NULL = no rotation
 *   x8         : [B, H, N, d] bytes (E4M3 bit patterns, written)
 *   scales     : [B, H, ceil(N / block_rows)] fp32 (written)
 *   block_rows : >= 1 (attn_fwd_fp8 takes 32 for Q and 64 for K and V)
 *
 * Supported: d in {64, 128}; the rotation for d == 64 only.
 * Errors: ATTN_ERR_INVALID_ARG for NULL or misaligned pointers (x, x8 16
 * bytes; scales, signs 4 bytes) or sizes out of range; ATTN_ERR_UNSUPPORTED
 * for another d or a rotation with d != 64.
 */
attn_status attn_quantize_fp8(const void* x, const float* signs, void* x8, float* scales, int B, int H,
                              int N, int d, int block_rows, void* stream);

/*
 * attn_fwd_fp8 -- attention forward on FP8 (E4M3) inputs with per-block
 * scales, the method of "8. FlashAttention 实战", section 8.9.3 and the
 * listing of section 8.9.6: both products run on FP8 with fp32
 * accumulation, the softmax statistics in fp32, and the probabilities are
 * requantised to FP8 with one scale per block before the second product.
 *
 * Query rows are taken in blocks of BLOCK_M = 32 and keys in blocks of
 * BLOCK_N = 64.  With q = q8 sq, k = k8 sk, v = v8 sv (each row's E4M3 value
 * times its block's scale), for every (query block, key block) with a
 * visible pair and every row of it, with the running state (m, l, U):
 *     s       = scale * q . k                       (masked if causal)
 *     m_new   = max(m, max s),  alpha = e^(m - m_new),  p = e^(s - m_new)
 *     l       = alpha l + sum p
 *     scale_p = (largest p of the block, over its rows below N) / 448
 *     U       = alpha U + (e4m3(p / scale_p) v8) scale_p sv
 * and O = U / l, LSE = m + ln l.  (The page's listing multiplies the whole
 * accumulator by scale_p scale_v after the product; it is read as scaling the
 * block's own product.)
 *
 *   q8, k8, v8 : [B, H, N, d] E4M3 bytes (as written by attn_quantize_fp8)
 *   q_scale    : [B, H, ceil(N / 32)] fp32;  k_scale, v_scale:
 *                [B, H, ceil(N / 64)] fp32; every scale positive and finite
 *   o          : [B, H, N, d] bf16 (written);  lse: [B, H, N] fp32 or NULL
 *   block_m, block_n : the scale block sizes; 32 and 64 are supported
 *
 * Supported: d == 64, block_m == 32, block_n == 64.
 * Errors as attn_fwd; ATTN_ERR_UNSUPPORTED for other d or block sizes.
 */
attn_status attn_fwd_fp8(const void* q8, const void* k8, const void* v8, const float* q_scale,
                         const float* k_scale, const float* v_scale, void* o, float* lse, int B, int H,
                         int N, int d, int block_m, int block_n, float scale, int causal, void* stream);

/*
 * attn_merge -- combine attention results over two disjoint key sets.
 *
 * Given (O_a, LSE_a) over keys A and (O_b, LSE_b) over keys B for the same
 * query rows, writes the result over A u B: per row,
 *     L = log(e^LSE_a + e^LSE_b),
 *     O = e^(LSE_a - L) O_a + e^(LSE_b - L) O_b,   LSE = L,
 * the partial-state merge of "FlashAttention 1 和 FlashAttention 2 的区别",
 * section 6, for normalised outputs.  It is the update a GPU makes for each
 * K/V shard that reaches it in Ring Attention ("FlashAttention",
 * xuesongtap.github.io, section 5): attn_fwd on (its queries, the arriving
 * shard) -- causal on the diagonal shard, non-causal below it -- then this
 * merge into its running result.  A side with LSE = -inf contributes nothing
 * (its O is not read); both empty give O = 0, LSE = -inf.
 *
 *   o_a, o_b, o  : [B, H, N, d] in `dtype`;  lse_a, lse_b, lse: [B, H, N] fp32
 *   o may be o_a or o_b and lse may be lse_a or lse_b (in place); other
 *   overlaps are not allowed.
 *
 * Supported: ATTN_BF16 and ATTN_F32 with d in {64, 128}.
 * Errors: ATTN_ERR_INVALID_ARG for NULL or misaligned pointers (o's 16
 * bytes, lse's 4) or sizes out of range; ATTN_ERR_UNSUPPORTED for another d.
 */
attn_status attn_merge(const void* o_a, const float* lse_a, const void* o_b, const float* lse_b,
                       void* o, float* lse, int B, int H, int N, int d, attn_dtype dtype,
                       void* stream);

/*
 * attn_fwd_merge -- the forward over this call's keys, combined in place with
 * a running result over other keys: one step of Ring Attention ("FlashAttention",
 * xuesongtap.github.io, section 5) with attn_merge's combination fused into
 * the forward's epilogue.
 *
 * On entry (o, lse) hold the result over a key set A (rows with lse = -inf
 * have seen no key; their o is not read); k, v hold further keys disjoint
 * from A.  On return (o, lse) hold the result over A and the new keys:
 *     L = log(e^lse + e^LSE_new),
 *     o = e^(lse - L) o + e^(LSE_new - L) O_new,  lse = L,
 * with (O_new, LSE_new) what attn_fwd would compute (O_new is combined in
 * fp32, before rounding; o is read as stored).  With lse = -inf on entry the
 * result is attn_fwd's bit for bit.  `causal` masks key j > query i within
 * this call's block (the diagonal block of a causal sequence).
 *
 *   q, k, v : [B, H, N, d] bf16
 *   o       : [B, H, N, d] bf16, read and written
 *   lse     : [B, H, N] fp32, read and written (not NULL)
 *
 * Supported: ATTN_BF16 with d in {64, 128}.
 * Errors as attn_fwd; lse NULL is ATTN_ERR_INVALID_ARG.
 */
attn_status attn_fwd_merge(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                           int N, int d, attn_dtype dtype, float scale, int causal, void* stream);

/*
 * Workspace size in bytes that attn_bwd needs: 24 bytes per query row
 * (B*H*N rows) for the per-row terms of the backward -- D = rowsum(dO o O)
 * in fp32, -LSE*log2(e) in fp32, and -D and -LSE/scale each split into three
 * bf16 parts whose sum is the value to about fp32 precision.  Returns 0 for
 * invalid sizes.
 */
size_t attn_bwd_workspace_bytes(int B, int H, int N);

/*
 * attn_bwd -- exact attention backward by recomputation.
 *
 * With P rebuilt tile by tile as P_ij = exp(S_ij - LSE_i) from the saved LSE
 * ("8. FlashAttention 实战", triton-tutorial.pages.dev, section 8.8.2), and
 * D_i = sum_d dO_i o O_i from the saved O (section 8.8.3):
 *     dV = P^T dO,  dP = dO V^T,  dS = P o (dP - D),
 *     dQ = scale * dS K,  dK = scale * dS^T Q          (sections 8.8.1, 8.8.3)
 * computed in two deterministic phases without atomics (section 8.8.4):
 * dK/dV with key tiles outer, then dQ with query tiles outer.
 *
 *   q, k, v, o, dO : [B, H, N, d] in `dtype` (o is attn_fwd's output)
 *   lse            : [B, H, N] fp32 from attn_fwd with the same arguments
 *   dq, dk, dv     : [B, H, N, d] in `dtype` (written)
 *   workspace      : >= attn_bwd_workspace_bytes(B, H, N) bytes, 16-byte
 *                    aligned; its first B*H*N fp32 values hold D on return.
 *
 * Supported: ATTN_BF16 with d in {64, 128}.
 * Errors as attn_fwd, plus ATTN_ERR_WORKSPACE.
 */
attn_status attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dO,
                     const float* lse, void* dq, void* dk, void* dv, void* workspace,
                     size_t workspace_bytes, int B, int H, int N, int d, attn_dtype dtype,
                     float scale, int causal, void* stream);

/*
 * Workspace size in bytes that attn_bwd_atomic_dq needs: the 24 bytes per
 * query row of attn_bwd_workspace_bytes, rounded up to 256 bytes, then an
 * fp32 dQ accumulator of B*H*N*d values.  Returns 0 for invalid sizes.
 */
size_t attn_bwd_atomic_workspace_bytes(int B, int H, int N, int d);

/*
 * attn_bwd_atomic_dq -- the same backward with dQ accumulated by atomic adds
 * in the dK/dV pass (the single-kernel alternative to the split into a dK/dV
 * and a dQ pass, "8. FlashAttention 实战", triton-tutorial.pages.dev,
 * section 8.8.4): every key tile adds its dS K into an fp32 accumulator in
 * the workspace, which a last pass multiplies by scale into dq.  The results
 * are those of attn_bwd up to the order of the fp32 additions into dQ; that
 * order depends on timing, so dq is not bitwise reproducible (dk and dv are).
 *
 *   q, k, v, o, dO, lse, dq, dk, dv : as attn_bwd
 *   workspace      : >= attn_bwd_atomic_workspace_bytes(B, H, N, d) bytes,
 *                    16-byte aligned; its first B*H*N fp32 values hold D on
 *                    return, the accumulator holds dQ / scale.
 *
 * Supported: ATTN_BF16 with d in {64, 128}.
 * Errors as attn_bwd.
 */
attn_status attn_bwd_atomic_dq(const void* q, const void* k, const void* v, const void* o, const void* dO,
                               const float* lse, void* dq, void* dk, void* dv, void* workspace,
                               size_t workspace_bytes, int B, int H, int N, int d, attn_dtype dtype,
                               float scale, int causal, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_H */
