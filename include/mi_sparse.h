/*
 * mi_sparse.h -- C ABI of an MI355X (gfx950) library for MInference-style
 * dynamic sparse prefill attention.
 *
 * The method (arXiv 2407.02490, "MInference 1.0: Accelerating Pre-filling for
 * Long-Context LLMs via Dynamic Sparse Attention", abstract): every attention
 * head is assigned offline to one of three sparse patterns -- A-shape,
 * Vertical-Slash, Block-Sparse -- and at prefill time a sparse index is built
 * online from the input for that pattern, then attention runs only on the
 * indexed keys.  The four compute entry points below are the stages of that
 * path: two online estimates, the conversion of their output into per-query-
 * block work lists, and the sparse attention itself.
 *
 * Conventions for every call
 *  - All tensor pointers are DEVICE pointers owned by the caller.  The library
 *    never allocates, frees or synchronises; it enqueues kernels on `stream`
 *    (a hipStream_t; NULL means the default stream) and returns.
 *  - Small arrays documented as HOST arrays (`heads`, `head_pattern`) are read
 *    during the call and copied by value into kernel arguments.
 *  - Arguments are validated on the host before anything is enqueued.  On any
 *    error the call returns a non-zero mi_status, enqueues nothing and leaves
 *    every output untouched; mi_last_error() then holds a one-line reason for
 *    the calling thread.  MI_ERR_LAUNCH reports a failed kernel launch (work
 *    enqueued before it may have run).  Faults inside kernels surface at the
 *    caller's next synchronisation, as with any HIP kernel.
 *  - Calls are stateless and re-entrant.  Two calls that write the same output
 *    or workspace on different streams race; nothing else is shared.
 *  - Token block size is fixed at 64 (MI_BLOCK): seq_len must be a multiple of
 *    64.  Query block a holds query rows [64a, 64a+64); nb = seq_len / 64.
 *  - Tensors Q, K, V, O are laid out [batch, head, token, head_dim] with
 *    head_dim contiguous and arbitrary element strides for (batch, head, token)
 *    given in mi_attn_desc.  Query head h reads key/value head
 *    h / (heads_q / heads_kv) (grouped-query attention).
 */
#ifndef MI_SPARSE_H
#define MI_SPARSE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MI_BLOCK 64
#define MI_MAX_HEADS 256

typedef enum {
    MI_OK = 0,
    MI_ERR_NULL = 1,      /* a required pointer is NULL */
    MI_ERR_SHAPE = 2,     /* unsupported size, stride or alignment */
    MI_ERR_BUDGET = 3,    /* a budget, forced count or list capacity is out of range */
    MI_ERR_DTYPE = 4,     /* unknown dtype */
    MI_ERR_WORKSPACE = 5, /* workspace smaller than mi_workspace_bytes() */
    MI_ERR_LAUNCH = 6,    /* a kernel launch failed */
    MI_ERR_PATTERN = 7    /* bad head list or pattern code */
} mi_status;

typedef enum { MI_F32 = 0, MI_BF16 = 1 } mi_dtype;

/* Per-head pattern codes.  MI_DENSE (plain causal attention) is not one of the
 * method's patterns; it is the comparator the sparse kernel is measured
 * against and a safe choice for heads that fit no pattern.  MI_VSLASH runs a
 * Vertical-Slash head on whole aligned 64x64 tiles (the tiles its slash lines
 * cross) plus gathered vertical columns; MI_VSLASH_EXACT runs it on the same
 * tiles masked element by element to the pattern's exact key set (aifetchly
 * guide, "The Vertical-Slash Pattern": vertical keys every later query
 * attends to, slash lines at fixed offsets i - j). */
typedef enum { MI_ASHAPE = 0, MI_VSLASH = 1, MI_BSPARSE = 2, MI_DENSE = 3, MI_VSLASH_EXACT = 4 } mi_pattern;

/* Workspace-sized operations for mi_workspace_bytes(). */
typedef enum {
    MI_OP_VS_ESTIMATE = 0,
    MI_OP_BLOCK_ESTIMATE = 1,
    MI_OP_SPARSE_PREFILL = 2,
    MI_OP_ANTIDIAG_ESTIMATE = 3
} mi_op;

typedef struct {
    int32_t batch, heads_q, heads_kv, seq_len, head_dim; /* head_dim in {64, 128} */
    int32_t dtype;        /* mi_dtype of Q, K, V and O (f32 or bf16) */
    float scale;          /* softmax scale applied to q.k, normally 1/sqrt(head_dim) */
    int64_t q_stride[3];  /* element strides of (batch, head, token); head_dim contiguous */
    int64_t k_stride[3];  /* strides must be multiples of 8 elements (16-byte rows) */
    int64_t v_stride[3];
    int64_t o_stride[3];
} mi_attn_desc;

/* Per-query-block work lists (device memory, caller-owned).
 *   block_count [batch, heads_q, nb]             number of key blocks of query block a
 *   block_idx   [batch, heads_q, nb, block_cap]  key-block ids, ascending, padded with -1
 *   col_count   [batch, heads_q, nb]             number of gathered key columns
 *   col_idx     [batch, heads_q, nb, col_cap]    key positions, ascending, padded with -1
 *   vs_bits     [batch, heads_q, 2, MI_VS_BITS_WORDS(seq_len)] uint32, or NULL
 *               when no head is MI_VSLASH_EXACT: per exact head, a map of its
 *               vertical keys (bit 64 + j) then a map of its slash offsets
 *               (bit 64 + o); the first 64 bits of each map are zero
 * Query block a of a head attends, for each row i, to the keys j <= i that lie
 * in a listed key block or are listed columns (MI_VSLASH_EXACT heads: inside
 * listed key blocks, only keys j that are vertical keys or whose offset i - j
 * is a slash offset).  A listed column never lies in a listed key block. */
#define MI_VS_BITS_WORDS(seq_len) ((seq_len) / 32 + 4)
typedef struct {
    int32_t* block_count;
    int32_t* block_idx;
    int32_t* col_count;
    int32_t* col_idx;
    int32_t block_cap;
    int32_t col_cap;
    uint32_t* vs_bits;
} mi_index;

/* Bytes of workspace an operation needs.  op = MI_OP_VS_ESTIMATE: p0 = number
 * of listed heads; MI_OP_BLOCK_ESTIMATE and MI_OP_ANTIDIAG_ESTIMATE: p0 = number
 * of listed heads;
 * MI_OP_SPARSE_PREFILL: the attention item schedule, which mi_sparse_prefill
 * builds in ws with a kernel on the stream before the attention reads it
 * (optional: with ws = NULL the attention uses its default order).  Returns
 * 0 for an invalid desc. */
size_t mi_workspace_bytes(const mi_attn_desc* desc, int32_t op, int32_t p0, int32_t p1);

/* Vertical-Slash index estimate (hotpaper.ai summary of arXiv 2407.02490, key
 * idea: Vertical-Slash heads use the last last_q queries against the keys to
 * find globally important positions; aifetchly guide, "The Vertical-Slash
 * Pattern": vertical lines are keys every later query attends to, slash lines
 * are fixed offsets o = i - j).
 *
 * For each listed query head h and batch b, with rows i_r = N - last_q + r:
 *   P[r, j]       = softmax over keys j <= i_r of scale * q_{i_r} . k_j
 *   vertical[j]   = sum_r P[r, j]            j in [0, N)
 *   slash[o]      = sum_r P[r, i_r - o]      o in [0, N), terms i_r - o < 0 omitted
 *   vertical_idx  = {0..force_vertical-1} plus the highest-scoring other keys,
 *                   n_vertical in total (clamped to N), ascending
 *   slash_idx     = {0..force_slash-1} plus the highest-scoring other offsets,
 *                   n_slash in total (clamped to N), ascending
 * Equal scores rank the lower index first.  Selection uses the fp32 scores as
 * written to vertical_score / slash_score.
 *   heads          HOST int32[n_heads], strictly increasing q-head ids
 *   vertical_idx   int32 [batch, heads_q, n_vertical]; rows of listed heads written,
 *                  entries beyond the clamped budget set to -1
 *   slash_idx      int32 [batch, heads_q, n_slash], likewise
 *   vertical_score float [batch, heads_q, seq_len] or NULL (then kept in ws)
 *   slash_score    float [batch, heads_q, seq_len] or NULL
 *   ws             >= mi_workspace_bytes(desc, MI_OP_VS_ESTIMATE, n_heads, 0) bytes
 * Requires 1 <= last_q <= 64, last_q <= seq_len, 1 <= force_vertical <=
 * n_vertical and 1 <= force_slash <= n_slash. */
mi_status mi_vs_estimate(const mi_attn_desc* desc, const void* q, const void* k,
                         const int32_t* heads, int32_t n_heads, int32_t last_q,
                         int32_t n_vertical, int32_t n_slash,
                         int32_t force_vertical, int32_t force_slash,
                         int32_t* vertical_idx, int32_t* slash_idx,
                         float* vertical_score, float* slash_score,
                         void* ws, size_t ws_bytes, void* stream);

/* Block-Sparse index estimate (hotpaper.ai summary, key idea: 64-token mean
 * pooling gives block-level attention weights; aifetchly guide, "2. The
 * Block-Sparse Kernel Mechanics": mean key of each 64-token block, dot products
 * with the query block, top-k key blocks kept).
 *
 * For each listed query head h and batch b, with Qbar_a, Kbar_c the fp32 means
 * of the 64 query rows of block a and the 64 key rows of block c:
 *   z[a, c] = scale * Qbar_a . Kbar_c for c <= a
 *   w[a, c] = softmax over c <= a of z[a, c];  w[a, c] = 0 for c > a
 *   block_idx[a] = {0, a} plus the highest-weight other blocks c <= a,
 *                  min(top_blocks, a + 1) in total, ascending, padded with -1
 *   heads        HOST int32[n_heads], strictly increasing q-head ids
 *   block_idx    int32 [batch, heads_q, nb, top_blocks]
 *   block_count  int32 [batch, heads_q, nb]
 *   block_score  float [batch, heads_q, nb, nb] (w) or NULL: w is then formed
 *                only where the selection needs it and never stored; with
 *                nb <= 512 the scores z stay on chip as well (one fused
 *                kernel); longer rows keep z in ws between two kernels
 *   ws           >= mi_workspace_bytes(desc, MI_OP_BLOCK_ESTIMATE, n_heads, 0)
 * Requires top_blocks >= 2 and 16-byte aligned q and k.  Equal weights rank
 * the lower block first; the lists do not depend on whether block_score is
 * given. */
mi_status mi_block_estimate(const mi_attn_desc* desc, const void* q, const void* k,
                            const int32_t* heads, int32_t n_heads, int32_t top_blocks,
                            int32_t* block_idx, int32_t* block_count, float* block_score,
                            void* ws, size_t ws_bytes, void* stream);

/* Block-Sparse index from antidiagonal block scores (hysenlabs review of the
 * MInference repository, "How MInference differs from xAttention, FlexPrefill
 * and RetrievalAttention": xAttention scores blocks by antidiagonal sums to
 * decide which to keep).  The score of query block a and key block c is the
 * sum of the scaled logits along the 64x64 block's main antidiagonal,
 *   x[a, c] = scale * sum_{r<64} q[64a + r] . k[64c + 63 - r]   for c < a,
 * and over its causal half (r >= 32) for c = a; weights and lists then follow
 * mi_block_estimate: w = softmax over c <= a of x, block_idx[a] = {0, a} plus
 * the highest-weight other causal blocks, min(top_blocks, a + 1) in total,
 * ascending, padded with -1.  The output lists feed mi_build_index as
 * MI_BSPARSE lists.
 *   heads, block_idx, block_count, block_score: as for mi_block_estimate
 *   ws   >= mi_workspace_bytes(desc, MI_OP_ANTIDIAG_ESTIMATE, n_heads, 0): the
 *        score rows [batch, n_heads, nb, nb] fp32 (256 bytes when block_score
 *        is given: the scores are then formed in block_score itself)
 * Requires top_blocks >= 2.  Errors as for mi_block_estimate. */
mi_status mi_antidiag_estimate(const mi_attn_desc* desc, const void* q, const void* k,
                               const int32_t* heads, int32_t n_heads, int32_t top_blocks,
                               int32_t* block_idx, int32_t* block_count, float* block_score,
                               void* ws, size_t ws_bytes, void* stream);

/* Conversion of the estimates into per-query-block work lists (aifetchly
 * guide, "1. The Vertical-Slash Kernel Mechanics": verticals are read as
 * coalesced chunks; "2. The Block-Sparse Kernel Mechanics": only active
 * 64x64 tiles run on the matrix units).  Writes `out` for every head, by
 * head_pattern[h] (HOST int32[heads_q]):
 *   MI_VSLASH, MI_VSLASH_EXACT :
 *               slash offsets S (slash_idx row, -1 entries ignored) become the
 *               tile distances T = {floor(o/64), ceil(o/64) : o in S};
 *               block list of a = {a - t : t in T, t <= a};
 *               column list of a = {j in V : j <= 64a + 63, block of j not
 *               listed}, V = vertical_idx row.
 *               MI_VSLASH_EXACT heads also get their vs_bits maps (out->vs_bits
 *               must then be non-NULL).
 *   MI_BSPARSE: block list = bs_block_idx[b, h, a, :bs_block_count], no columns.
 *   MI_ASHAPE : block list = key blocks c <= a holding a sink key (64c <
 *               sink_tokens) or within the local window of some row
 *               (64(a - c) - 63 < local_tokens); no columns.
 *   MI_DENSE  : block_count = a + 1, col_count = 0, lists not written (the
 *               attention treats dense heads as all causal blocks).
 * Pointers for patterns no head uses may be NULL.  Capacities: block_cap >=
 * min(nb, 2 n_slash) if any VS head, >= top_blocks if any BS head, >= the
 * A-shape maximum min(nb, ceil(sink/64) + floor((local + 126)/64)) if any
 * A-shape head; col_cap >= min(n_vertical, seq_len) if any VS head. */
mi_status mi_build_index(const mi_attn_desc* desc, const int32_t* head_pattern,
                         const int32_t* vertical_idx, int32_t n_vertical,
                         const int32_t* slash_idx, int32_t n_slash,
                         const int32_t* bs_block_idx, const int32_t* bs_block_count,
                         int32_t top_blocks, int32_t sink_tokens, int32_t local_tokens,
                         const mi_index* out, void* stream);

/* Sparse prefill attention (arXiv 2407.02490 abstract: sparse attention with
 * the per-head pattern and online index; aifetchly guide, "1. The
 * Vertical-Slash Kernel Mechanics": online softmax keeps a running max and
 * normaliser so no score matrix is written).
 *
 * For each batch b, query head h and row i:
 *   o_i = sum_{j in A(i)} softmax_j(scale * q_i . k_j) v_j
 *   lse_i = log sum_{j in A(i)} exp(scale * q_i . k_j)      (natural log)
 * with A(i) from head h's pattern:
 *   MI_VSLASH, MI_BSPARSE: keys j <= i in the listed blocks or listed columns of
 *                          the row's query block (idx);
 *   MI_VSLASH_EXACT: keys j <= i that are vertical keys or lie on a slash line
 *              (i - j a slash offset), from idx's lists and vs_bits maps;
 *   MI_ASHAPE: keys j <= i with j < sink_tokens or i - j < local_tokens (idx
 *              holds the block list; edges are masked per element);
 *   MI_DENSE : all keys j <= i (idx not read).
 * head_pattern == NULL runs every head as MI_DENSE (the dense comparator; idx
 * may then be NULL).  A row whose A(i) is empty (an index with no block and
 * no column for its query block) gets o_i = 0 and lse_i = -inf.  O is written in desc->dtype; bf16 inputs use bf16 MFMA
 * with fp32 softmax and accumulation, f32 inputs use fp32 MFMA.
 *   o    [batch, heads_q, seq_len, head_dim] with desc->o_stride
 *   lse  float [batch, heads_q, seq_len] or NULL
 *   ws   NULL, or >= mi_workspace_bytes(desc, MI_OP_SPARSE_PREFILL, 0, 0)
 *        bytes of 16-byte aligned device memory: the call then enqueues a
 *        small kernel that writes the item schedule of mi_attn_schedule()
 *        into ws, and the attention runs its work items in that order (the
 *        results are bit-identical either way).  ws is overwritten by every
 *        call; two calls sharing it on different streams race.
 * A launch whose heads are all MI_BSPARSE, with 4 * idx->block_cap <= nb,
 * runs a schedule in which each half of a work item walks its own two
 * blocks' lists; its results are bit-identical to the common schedule's.
 * The call enqueues kernels only (no memset, copy or allocation), so it may
 * be captured in a HIP graph. */
mi_status mi_sparse_prefill(const mi_attn_desc* desc, const void* q, const void* k,
                            const void* v, const int32_t* head_pattern, const mi_index* idx,
                            int32_t sink_tokens, int32_t local_tokens, void* o, float* lse,
                            void* ws, size_t ws_bytes, void* stream);

/* mi_sparse_prefill for callers that cannot allocate device memory (code
 * under HIP graph capture, serving loops or harnesses that forbid hipMalloc):
 * the same computation, arguments and errors as mi_sparse_prefill with a
 * workspace, except that the item schedule is built in a buffer inside the
 * library instead of a caller workspace.  The buffer holds
 * MI_NOALLOC_SCHEDULE_ENTRIES int32 entries (1 MiB) per GPU, in the
 * library's device globals, kept until the process ends; a call whose
 * schedule needs more entries (about batch * heads_q * seq_len / 256) returns
 * MI_ERR_WORKSPACE and enqueues nothing.  The call allocates nothing.  Every
 * call on one GPU writes the same buffer (each call writes every entry it
 * reads, so nothing needs clearing): calls that overlap on one GPU, on
 * different streams, race. */
#define MI_NOALLOC_SCHEDULE_ENTRIES (1 << 18)
mi_status mi_sparse_prefill_noalloc(const mi_attn_desc* desc, const void* q, const void* k,
                                    const void* v, const int32_t* head_pattern, const mi_index* idx,
                                    int32_t sink_tokens, int32_t local_tokens, void* o, float* lse,
                                    void* stream);

/* The attention item schedule that mi_sparse_prefill builds in its ws on
 * the device, computed here on the host (host call, no device work, no
 * state kept between calls).  Items are runs of four 64-row query blocks
 * of one (batch, query head), packed as (b * heads_q + h) * nruns + run with
 * nruns = ceil(seq_len / 256); -1 marks padding.  Consecutive groups of four
 * entries hold items of one kv group and one pattern class (Vertical-Slash
 * and dense / A-shape / Block-Sparse), in run order, so that the heads a
 * group of four runs together stream the same K/V tiles; groups are ordered
 * by estimated length, longest first.  head_pattern as in mi_sparse_prefill
 * (NULL = all dense); block_cap bounds the Block-Sparse estimate.  Writes
 * min(cap, length) entries to out (may be NULL) and returns the length, or
 * -1 for an invalid desc or pattern code. */
int32_t mi_attn_schedule(const mi_attn_desc* desc, const int32_t* head_pattern, int32_t sink_tokens,
                         int32_t local_tokens, int32_t block_cap, int32_t* out, int32_t cap);

/* Static text of a status code. */
const char* mi_status_str(mi_status s);

/* Reason for the last non-MI_OK status returned on the calling thread. */
const char* mi_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* MI_SPARSE_H */
