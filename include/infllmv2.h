/*
 * infllmv2.h -- C ABI of an MI355X (gfx950) implementation of InfLLM v2
 * trainable block-sparse attention.
 *
 * What the method computes (sources are web pages about CPM.cu / MiniCPM4):
 *   - the KV context is split into fixed-size blocks of tokens (64 on the page
 *     "MiniCPM 4.0 ..." (shadowrocket9.top), section on native sparsity /
 *     InfLLM v2; 128 on "MiniCPM4: running LLMs on phones and PCs"
 *     (xugj520.cn), section 1.1 and the CPM_cu class sketch in section 2.1);
 *   - keys are compressed into parameter-free "semantic kernels": overlapping
 *     32-token units with stride 16 (xugj520.cn, section 1.1);
 *   - each query scores the kernels, the scores are pooled to blocks and the
 *     query keeps its top-k blocks (top-64 on shadowrocket9.top, top-6 on
 *     xugj520.cn), always including the initial tokens and a sliding local
 *     window (xugj520.cn, section 1.1);
 *   - attention then runs over the kept blocks only;
 *   - contexts shorter than dense_len = 8192 use dense attention
 *     (shadowrocket9.top, InfLLM v2 section; the sparse_config dict in its
 *     deployment section holds topk / block_size / dense_len);
 *   - the attention mask for tree speculative decoding is packed in uint64
 *     words (xugj520.cn, section 1.1 technical notes; pomoai.com CPM.cu
 *     article, section 2).
 * Where the pages disagree (block 64 vs 128, top-64 vs top-6) the value is a
 * run-time parameter.
 *
 * Conventions shared by every entry point
 *   - Pointers are DEVICE pointers unless a comment says "host".  The caller
 *     allocates and owns every buffer (inputs, outputs, workspaces); the
 *     library never allocates, frees or synchronises, so every call can be
 *     captured into a HIP graph.  Buffers must stay alive until the work
 *     queued on `stream` has finished.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *   - Work is queued asynchronously.  Arguments are validated on the host
 *     before anything is launched; an invalid call returns a non-zero status
 *     and queues nothing.  A failed launch returns INFLLMV2_ERR_HIP.  Faults
 *     inside queued work surface at the caller's next synchronisation.
 *   - Nothing aborts, throws or prints.  The library is stateless and
 *     reentrant, except infllmv2_sparse_attn_decode_noalloc, whose calls on
 *     one GPU share that GPU's fixed scratch array.
 *   - dtype selects the element type of q, k, v, compressed keys and outputs:
 *     INFLLMV2_F32 (float) or INFLLMV2_BF16 (bfloat16, stored as uint16).
 *     Accumulation is float32 in both cases.
 *   - Layouts (row-major, innermost last):
 *       queries      q        [rows][h_q][d]
 *       KV caches    k, v     [batch][h_kv][cap][d]   (batch = 1 for prefill
 *                                                      and tree verification)
 *       compressed   ck       [batch][h_kv][nc_cap][d] (dtype of k)
 *       block scores scores   [rows][h_kv][nb_cap]  float32
 *       selections   block_idx[rows][h_kv][topk]    int32, ascending, -1 pad
 *       outputs      out      [rows][h_q][d]; lse [rows][h_q] float32 (ln)
 *   - Query head h reads KV head floor(h * h_kv / h_q) (GQA groups of
 *     G = h_q / h_kv consecutive heads).
 *   - Supported: d in {64, 128}; h_q % h_kv == 0; for bf16 attention
 *     G in {1, 2, 4, 8, 16, 32}; block_size a multiple of 32 up to 256;
 *     kernel_stride <= kernel_size; 1 <= topk <= 128;
 *     init_blocks + local_blocks <= topk; n_draft <= 64.
 */
#ifndef INFLLMV2_H
#define INFLLMV2_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  INFLLMV2_OK = 0,
  INFLLMV2_ERR_INVALID_ARG = 1,   /* NULL pointer, bad size, inconsistent args */
  INFLLMV2_ERR_UNSUPPORTED = 2,   /* valid but outside the supported range    */
  INFLLMV2_ERR_WORKSPACE = 3,     /* workspace missing or too small           */
  INFLLMV2_ERR_HIP = 4            /* a kernel launch failed                   */
} infllmv2_status;

typedef enum { INFLLMV2_F32 = 0, INFLLMV2_BF16 = 1 } infllmv2_dtype;

/* Sparse-attention parameters.  Names of topk / block_size / dense_len follow
 * the sparse_config dict on shadowrocket9.top (deployment section). */
typedef struct {
  int32_t block_size;     /* B: tokens per KV block (default 64)                 */
  int32_t kernel_size;    /* ks: tokens per semantic kernel (default 32)         */
  int32_t kernel_stride;  /* s: token stride between kernels (default 16)        */
  int32_t topk;           /* blocks kept per (query, KV head), forced ones
                             included (default 64)                                */
  int32_t init_blocks;    /* leading blocks always kept (default 1)              */
  int32_t local_blocks;   /* the query's own block and the local_blocks-1 before
                             it are always kept (default 2)                       */
  int32_t dense_len;      /* a sequence with fewer than dense_len keys uses dense
                             causal attention (default 8192)                      */
  float scale;            /* softmax scale; 0 selects 1/sqrt(d)                  */
  int32_t score_mode;     /* how a KV group's query heads make one window score
                             (the pages do not say; see infllmv2_block_scores):
                             0 = scaled dot product with the group's summed
                             query (default), 1 = sum over the group's heads of
                             each head's softmax over the visible windows     */
} infllmv2_params;

/* host: fill *p with the defaults 64 / 32 / 16 / 64 / 1 / 2 / 8192 / 0 / 0. */
void infllmv2_default_params(infllmv2_params* p);

/* host: static string for a status code (never NULL). */
const char* infllmv2_status_string(int status);

/* host: library ABI version (major * 100 + minor). */
int infllmv2_version(void);

/*
 * Semantic-kernel key compression (xugj520.cn, section 1.1: 32-token units,
 * stride 16, no parameters; pooling = arithmetic mean).
 *
 *   ck[b][g][m][:] = round_to_dtype( mean_{t = m*s .. m*s+ks-1} k[b][g][t][:] )
 *
 * for every sequence b < batch, KV head g < h_kv and window m in
 * [m_begin, m_end) whose tokens all lie inside the sequence
 * (m*s + ks <= seqlens[b]).  Other windows are left untouched, so a decode
 * loop can append new windows as the cache grows.  Sum in float32, one
 * rounding (to nearest, ties to even) to the storage dtype.
 *   k        [batch][h_kv][cap][d]     seqlens  int32 [batch]
 *   ck       [batch][h_kv][nc_cap][d]  requires m_end <= nc_cap and
 *            (m_end-1)*s + ks <= cap.
 */
int infllmv2_compress_keys(int dtype, const void* k, int32_t batch, int32_t h_kv,
                           int64_t cap, int32_t d, const int32_t* seqlens,
                           int64_t m_begin, int64_t m_end, void* ck, int64_t nc_cap,
                           const infllmv2_params* p, void* stream);

/*
 * Block relevance scores (xugj520.cn, section 1.1: each query is scored
 * against semantic kernels, blocks are picked from them).  For query row r
 * (sequence row_seq[r], absolute position row_pos[r]) and KV head g:
 *
 *   sigma[m] = scale * sum_{h in group g} q[r][h] . ck[seq][g][m]
 *              for windows that end at or before row_pos[r]
 *   (score_mode 1: sigma[m] = sum_{h in group g} softmax over the visible
 *              windows m' of scale * q[r][h] . ck[seq][g][m'], taken at m;
 *              with one query head per group it orders the windows as mode 0
 *              does.  Mode 1 runs one workgroup per (row, KV head) and needs
 *              h_q / h_kv <= 16 and at most 16384 visible windows.)
 *   scores[r][g][b] = max of sigma[m] over the visible windows m whose token
 *              span overlaps block b, or -inf if there is none,
 *
 * written for the eligible blocks b = 0 .. floor(row_pos[r] / B); entries
 * beyond are left untouched.  Rows whose sequence is dense
 * (seqlens[seq] < dense_len) are skipped.
 *   q        [rows][h_q][d]            row_seq int32 [rows] or NULL (all 0)
 *   row_pos  int32 [rows], each < seqlens[row's sequence]; NULL means the
 *            decode position seqlens[row's sequence] - 1
 *   ck       [batch][h_kv][nc_cap][d]  holding every window visible to the rows
 *   seqlens  int32 [batch]
 *   scores   float32 [rows][h_kv][nb_cap], nb_cap >= floor(max_pos / B) + 1
 *   max_pos  host: an upper bound of row_pos (sizes the launch)
 */
int infllmv2_block_scores(int dtype, const void* q, int32_t rows,
                          const int32_t* row_seq, const int32_t* row_pos,
                          int32_t h_q, int32_t h_kv, int32_t d, const void* ck,
                          int32_t batch, int64_t nc_cap, const int32_t* seqlens,
                          float* scores, int64_t nb_cap, int32_t max_pos,
                          const infllmv2_params* p, void* stream);

/*
 * Top-k block selection (shadowrocket9.top, InfLLM v2 section: top-k blocks
 * per query; xugj520.cn, section 1.1: initial and sliding-window tokens are
 * always kept).  For row r at position pos with own block b_r = pos / B:
 *   eligible  E = {0 .. b_r}
 *   forced    F = ({0 .. init_blocks-1} U {b_r-local_blocks+1 .. b_r}) n E
 *   kept      F plus the best blocks of E \ F by (score descending, block
 *             index ascending) until min(topk, |E|) blocks are kept.
 * block_idx[r][g][:] receives the kept blocks in ascending order, padded with
 * -1.  Rows whose sequence is dense receive -1 only.  row_seq / row_pos
 * follow infllmv2_block_scores (NULL row_pos = decode positions).
 *   scores   float32 [rows][h_kv][nb_cap] as written by infllmv2_block_scores
 *   block_idx int32  [rows][h_kv][topk]
 */
int infllmv2_select_topk(const float* scores, int32_t rows, const int32_t* row_seq,
                         const int32_t* row_pos, int32_t h_kv, int64_t nb_cap,
                         const int32_t* seqlens, int32_t batch, int32_t* block_idx,
                         const infllmv2_params* p, void* stream);

/*
 * Block-sparse causal attention for a prefill chunk (xugj520.cn, section 1.1:
 * attention computed on the selected blocks only; pomoai.com, section 4:
 * chunked prefill).  One sequence; query i sits at position n_k - n_q + i and
 * attends the keys j <= its position inside its kept blocks.  If
 * n_k < dense_len the attention is dense causal and block_idx is ignored (may
 * be NULL); otherwise block_idx [n_q][h_kv][topk] is required.
 *   q    [n_q][h_q][d]          k, v [h_kv][cap][d], n_k <= cap
 *   out  [n_q][h_q][d] (dtype)  lse  float32 [n_q][h_q] natural log, or NULL
 * No workspace.
 */
int infllmv2_sparse_attn_prefill(int dtype, const void* q, int32_t n_q,
                                 const void* k, const void* v, int64_t cap,
                                 int64_t n_k, int32_t h_q, int32_t h_kv, int32_t d,
                                 const int32_t* block_idx, void* out, float* lse,
                                 const infllmv2_params* p, void* stream);

/*
 * Block-sparse decode attention, ragged batch (one new query per sequence,
 * at position seqlens[b]-1, its own K/V already in the cache).  Each sequence
 * is dense or sparse on its own length.  Split-KV: partial results go to the
 * workspace and a second kernel merges them.
 *   q    [batch][h_q][d]        k, v [batch][h_kv][cap][d]
 *   seqlens int32 [batch], 1 <= seqlens[b] <= cap
 *   max_seqlen host: upper bound of seqlens (sizes launch and workspace)
 *   block_idx int32 [batch][h_kv][topk] (may be NULL when max_seqlen <
 *            dense_len; when not NULL every row must be readable: the rows
 *            of dense sequences are read and their values ignored)
 *   out  [batch][h_q][d]        lse float32 [batch][h_q] or NULL
 *   ws   >= infllmv2_workspace_size(INFLLMV2_OP_DECODE, batch, h_q, h_kv, d,
 *            max_seqlen, p) bytes, 256-byte aligned; contents on entry do
 *            not matter.  Calls that share a workspace must not overlap.
 */
int infllmv2_sparse_attn_decode(int dtype, const void* q, int32_t batch,
                                const void* k, const void* v, int64_t cap,
                                const int32_t* seqlens, int32_t max_seqlen,
                                int32_t h_q, int32_t h_kv, int32_t d,
                                const int32_t* block_idx, void* out, float* lse,
                                void* ws, size_t ws_bytes,
                                const infllmv2_params* p, void* stream);

/*
 * Top-k selection and decode attention in one call (pomoai.com, section 4:
 * fused kernels to cut launches on the decode path).  The result equals
 * infllmv2_select_topk(scores, batch, row_seq = {0, 1, .., batch-1},
 * row_pos = NULL, h_kv, nb_cap, seqlens, batch, block_idx) followed by
 * infllmv2_sparse_attn_decode(..., block_idx, ...), bit for bit.  For bf16,
 * 16 query heads per KV head and rows of at most 4096 blocks, each split of
 * the decode kernel selects its row itself and the first split writes
 * block_idx (one launch fewer); otherwise the two kernels run in turn.
 *   scores   float32 [batch][h_kv][nb_cap] from infllmv2_block_scores,
 *            nb_cap >= ceil(max_seqlen / B)
 *   block_idx int32 [batch][h_kv][topk], output: the selection, -1 rows for
 *            dense sequences
 * Both may be NULL when max_seqlen < dense_len (every row dense; nothing is
 * selected or written).  The other arguments, the workspace and the errors
 * are those of infllmv2_sparse_attn_decode.
 */
int infllmv2_sparse_attn_decode_topk(int dtype, const void* q, int32_t batch,
                                     const void* k, const void* v, int64_t cap,
                                     const int32_t* seqlens, int32_t max_seqlen,
                                     int32_t h_q, int32_t h_kv, int32_t d,
                                     const float* scores, int64_t nb_cap,
                                     int32_t* block_idx, void* out, float* lse,
                                     void* ws, size_t ws_bytes,
                                     const infllmv2_params* p, void* stream);

/*
 * Tree speculative verification (pomoai.com, section 2: tree verification in
 * the attention kernel; xugj520.cn, section 1.1: uint64-packed mask for tree
 * speculative decoding).  n_draft draft tokens follow an n_ctx-token context.
 * Draft i keeps its own blocks (block_idx row i, selected over the context as
 * seen from position n_ctx-1) and attends, in one softmax, the context keys of
 * those blocks and every draft j whose bit j is set in tree_mask[i] (bit 0 =
 * least significant).  A draft always attends itself; bits >= n_draft are
 * ignored.  If n_ctx < dense_len the context part is dense.
 *   q          [n_draft][h_q][d]       k, v [h_kv][cap][d] (context)
 *   k_draft, v_draft [h_kv][n_draft][d] tree_mask uint64 [n_draft]
 *   block_idx  int32 [n_draft][h_kv][topk] (may be NULL when dense)
 *   out        [n_draft][h_q][d]       lse float32 [n_draft][h_q] or NULL
 *   ws >= infllmv2_workspace_size(INFLLMV2_OP_TREE, n_draft, h_q, h_kv, d,
 *         n_ctx, p) bytes, 256-byte aligned
 */
int infllmv2_tree_verify(int dtype, const void* q, int32_t n_draft, const void* k,
                         const void* v, int64_t cap, int64_t n_ctx,
                         const void* k_draft, const void* v_draft,
                         const uint64_t* tree_mask, int32_t h_q, int32_t h_kv,
                         int32_t d, const int32_t* block_idx, void* out, float* lse,
                         void* ws, size_t ws_bytes, const infllmv2_params* p,
                         void* stream);

/*
 * Top-k selection and tree verification in one call (pomoai.com, sections 2
 * and 4).  The result equals infllmv2_select_topk(scores, n_draft,
 * row_seq = NULL, row_pos = {n_ctx-1, ..}, h_kv, nb_cap, {n_ctx}, 1,
 * block_idx) followed by infllmv2_tree_verify(..., block_idx, ...), bit for
 * bit.  For bf16, 16 query heads per KV head and contexts of at most 4096
 * blocks, each split selects its draft's row itself and the first split
 * writes block_idx; otherwise the two run in turn.
 *   scores    float32 [n_draft][h_kv][nb_cap], nb_cap >= ceil(n_ctx / B)
 *   block_idx int32 [n_draft][h_kv][topk], output
 * Both may be NULL when n_ctx < dense_len.  The other arguments, the
 * workspace and the errors are those of infllmv2_tree_verify.
 */
int infllmv2_tree_verify_topk(int dtype, const void* q, int32_t n_draft, const void* k,
                              const void* v, int64_t cap, int64_t n_ctx,
                              const void* k_draft, const void* v_draft,
                              const uint64_t* tree_mask, int32_t h_q, int32_t h_kv,
                              int32_t d, const float* scores, int64_t nb_cap,
                              int32_t* block_idx, void* out, float* lse, void* ws,
                              size_t ws_bytes, const infllmv2_params* p, void* stream);

/*
 * infllmv2_sparse_attn_decode without a workspace argument, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc).  Arguments, results and errors are
 * those of infllmv2_sparse_attn_decode, which it calls with the library's own
 * fixed scratch array in place of `ws`: INFLLMV2_NOALLOC_SCRATCH_BYTES per
 * GPU, a static device array that each GPU the library runs on holds until
 * the process ends.  It allocates nothing (no hipMalloc, no hipFree); its
 * first call on a device looks up that device's copy of the array (the
 * current device, which the stream must belong to).
 *   - A call whose workspace would exceed the array
 *     (infllmv2_workspace_size(INFLLMV2_OP_DECODE, ...) >
 *     INFLLMV2_NOALLOC_SCRATCH_BYTES) returns INFLLMV2_ERR_WORKSPACE and
 *     queues nothing.
 *   - Every call on one GPU shares that GPU's array: calls that overlap on
 *     one GPU (other streams, other threads) race and may return wrong
 *     results.  Serialise them, or use infllmv2_sparse_attn_decode with
 *     workspaces of your own.
 */
#define INFLLMV2_NOALLOC_SCRATCH_BYTES (8u << 20)
int infllmv2_sparse_attn_decode_noalloc(int dtype, const void* q, int32_t batch,
                                        const void* k, const void* v, int64_t cap,
                                        const int32_t* seqlens, int32_t max_seqlen,
                                        int32_t h_q, int32_t h_kv, int32_t d,
                                        const int32_t* block_idx, void* out, float* lse,
                                        const infllmv2_params* p, void* stream);

/*
 * Gradients of infllmv2_sparse_attn_prefill with each query's kept blocks
 * held fixed (selection is a top-k and passes no gradient; the sparse
 * attention is trained through the blocks it keeps: shadowrocket9.top,
 * InfLLM v2 section, on the trainable sparse attention).  For query row i,
 * head h (KV head g) with kept keys J (those of its kept blocks at positions
 * <= its own, or all keys up to it when dense), p = softmax over j in J of
 * scale * q.k_j, and upstream gradient do = d_out[i][h]:
 *   dq[i][h]  = scale * sum_j p_j (do.v_j - do.o) k_j
 *   dk[g][j] += scale * p_j (do.v_j - do.o) q[i][h]
 *   dv[g][j] += p_j do
 * with o = out[i][h] and p recomputed from lse.
 *   q, k, v, cap, n_k, n_q, h_q, h_kv, d, block_idx: as for
 *        infllmv2_sparse_attn_prefill (block_idx may be NULL when dense; a
 *        block listed twice counts once)
 *   out  [n_q][h_q][d]  the forward output     lse float32 [n_q][h_q] its
 *        log-sum-exp (natural log), both as written by the forward call
 *   d_out [n_q][h_q][d] upstream gradient
 *   dq   [n_q][h_q][d]  written
 *   dk, dv float32 [h_kv][cap][d]: ACCUMULATED (+=) at the keys the chunk's
 *        rows attend, so the chunks of a long prompt can add into the same
 *        buffers; zero them before the first chunk.  Additions from
 *        different workgroups are float32 atomics, so the rounding of dk and
 *        dv may differ between runs.
 *   ws >= infllmv2_workspace_size(INFLLMV2_OP_PREFILL_BWD, n_q, h_q, h_kv, d,
 *        n_k, p) bytes, 256-byte aligned; contents on entry do not matter.
 *        Calls that share a workspace must not overlap.
 * bf16: matrix cores; block_size a multiple of 64, G in {1, 2, 4, 8, 16,
 * 32}, n_q < 2^24 and n_q * h_q * d * 2 < 2^32 bytes (larger calls: split
 * the chunk).  float32 (dq, like q, float32): a vector-ALU path meant for
 * small shapes, any block_size and group size the forward accepts.
 */
int infllmv2_sparse_attn_prefill_backward(int dtype, const void* q, int32_t n_q,
                                          const void* k, const void* v, int64_t cap,
                                          int64_t n_k, int32_t h_q, int32_t h_kv,
                                          int32_t d, const int32_t* block_idx,
                                          const void* out, const float* lse,
                                          const void* d_out, void* dq, float* dk,
                                          float* dv, void* ws, size_t ws_bytes,
                                          const infllmv2_params* p, void* stream);

/*
 * host: input checks of the debug build.  A library built with
 * -DINFLLMV2_DEBUG (libinfllmv2_debug.so) checks, before the attention
 * kernels of every infllmv2_sparse_attn_prefill / _decode / _tree_verify /
 * _prefill_backward call, the kept-block rows it will read (min(topk,
 * eligible) strictly ascending ids in range, the forced initial and local
 * blocks among them, then -1 padding; rows of dense sequences are skipped)
 * and the tree masks (no bit at or above n_draft, none naming a later draft).
 * The kernels never read out of bounds on such input, but their results are
 * then not those of a valid selection.  This call waits for `stream`,
 * returns in *code the first violation since the previous call (0 none;
 * 1 id out of range, 2 not ascending or duplicated, 3 padding before an id,
 * 4 forced block missing, 5 wrong count, 6 mask bit at or above n_draft,
 * 7 mask bit naming a later draft) and in *where its row * h_kv + KV head
 * (or the draft index for 6 and 7), and clears them.  Without
 * INFLLMV2_DEBUG it returns INFLLMV2_ERR_UNSUPPORTED and touches nothing.
 */
int infllmv2_debug_check(int* code, int* where, void* stream);

enum { INFLLMV2_OP_DECODE = 0, INFLLMV2_OP_TREE = 1, INFLLMV2_OP_PREFILL_BWD = 2 };

/* host: workspace bytes needed by infllmv2_sparse_attn_decode (op DECODE,
 * n = batch, max_len = max_seqlen), infllmv2_tree_verify (op TREE,
 * n = n_draft, max_len = n_ctx) or infllmv2_sparse_attn_prefill_backward
 * (op PREFILL_BWD, n = n_q, max_len = n_k).  0 on invalid arguments. */
size_t infllmv2_workspace_size(int op, int32_t n, int32_t h_q, int32_t h_kv,
                               int32_t d, int64_t max_len, const infllmv2_params* p);

#ifdef __cplusplus
}
#endif

#endif /* INFLLMV2_H */
