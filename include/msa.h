/*
 * msa.h -- C ABI of libmsa: block-sparse paged attention (MiniMax-M3 style
 * "MSA") for AMD Instinct MI355X (gfx950).
 *
 * Two operations, as the "msa" module page of the MAX Mojo docs (graph-op
 * bindings for the MiniMax-M3 MSA kernels) splits the method:
 *
 *   1. the indexer, which picks for every (new token, KV head) the KV blocks
 *      that head may read, and
 *   2. the sparse attention, which gathers only those blocks from a paged
 *      KV cache and runs a causally clipped softmax over them,
 *
 * plus the split-K combine the attention uses when it splits a row's blocks
 * over several partitions.
 *
 * Selection semantics follow the "ferrox_core::block_sparse" page (docs.rs),
 * section "Four rules": a block's score is the maximum over its positions of
 * the raw, unscaled dot product q_idx . k_idx; each KV head selects its own
 * blocks and its whole GQA group reads them; the first `init_blocks` and the
 * newest `local_blocks` blocks are always selected.  Section "The block size
 * is an ABI, not a tuning knob" of the same page fixes blocks at 128 tokens,
 * equal to the KV page size.
 *
 * Calling convention (all entry points):
 *   - Output first, then inputs, then scalars, then the stream -- the
 *     argument order of the ragged paged graph ops on the MAX pages.
 *   - Every pointer named "device" is a device (HBM) address; every struct
 *     is read on the host during the call and not kept.  The library never
 *     allocates or frees memory and keeps no pointer after returning; the
 *     caller owns every buffer and keeps it alive until the work queued on
 *     `stream` has finished.
 *   - `stream` is a hipStream_t passed as an opaque pointer (NULL: the null
 *     stream).  All work is enqueued asynchronously on it; no call
 *     synchronises with the device or copies device data to the host.
 *   - Grid sizes depend only on host scalars (batch, max_seq_length,
 *     max_cache_length, head counts, top_k, partitions), never on device
 *     data, so a call can be captured into a HIP graph and replayed.
 *   - Every argument is validated before anything is launched.  On a
 *     validation error the call returns a negative MSA_ERR_* code and
 *     enqueues nothing.  Device-data errors (a page id >= num_pages, a
 *     cache length beyond the lookup table) are not detected: their result
 *     is undefined for the rows involved.  Every kernel either skips a
 *     page id outside [0, num_pages) or reads page 0 in its place, and
 *     clips lengths to what the lookup table addresses, so such data never
 *     makes a read leave its pool or table.
 *   - Calls are stateless and may be issued from several host threads.
 *
 * Data layout:
 *   - Ragged rows: new token t of sequence b is global row
 *     r = input_row_offsets[b] + t, at logical position
 *     p = cache_lengths[b] + t (its K/V/index-K are already in the cache).
 *     It may see the nb = p / 128 + 1 blocks 0 .. p/128 and positions
 *     j <= p only ("msa" page, speculative-decode route: token position is
 *     the cache length plus the token's index; causality is per token).
 *   - Paged caches: logical position j of sequence b is slot j % 128 of page
 *     kv_lookup_table[b * lookup_stride + j / 128].  Element d of head h of
 *     that slot is at data + page*page_stride + h*head_stride
 *     + slot*token_stride + d (strides in elements; d is contiguous).
 *   - q_idx: bf16 [rows][num_kv_heads][128]; q and output: bf16
 *     [rows][num_q_heads][128]; d_indices: int32 [rows][num_kv_heads][top_k];
 *     all contiguous, 16-byte aligned.
 *   - Query head g belongs to KV head g / (num_q_heads / num_kv_heads).
 */
#ifndef MSA_H
#define MSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes returned by every entry point. */
enum msa_status {
    MSA_OK = 0,
    MSA_ERR_NULL = -1,       /* a required pointer is NULL                          */
    MSA_ERR_SHAPE = -2,      /* head_dim / page size != 128, head counts, strides,   */
                             /* alignment, or a context beyond the supported maximum */
    MSA_ERR_PARAM = -3,      /* top_k, init/local blocks, partitions, batch          */
    MSA_ERR_DTYPE = -4,      /* unsupported storage type, or K and V types differ    */
    MSA_ERR_WORKSPACE = -5,  /* workspace smaller than the *_workspace_bytes query    */
    MSA_ERR_LAUNCH = -6,     /* the HIP runtime rejected a launch                    */
    MSA_ERR_DEVICE = -7,     /* no current HIP device, or it is not gfx950           */
    MSA_ERR_SCRATCH = -8     /* msa_attention_paged_noalloc: the shape needs more    */
                             /* workspace than its fixed device array holds         */
};

/* Storage types of the paged caches.  K/V ("msa" page): BF16 or native FP8
 * e4m3 with no scales.  Index-K: BF16 ("msa" page), or FP8 e4m3 with one
 * float32 dequantization scale per token ("DeepSeekSparseAttentionConfig"
 * page, indexer_k_dtype field: 128 code bytes + a 4-byte scale per token at
 * head dim 128), k_idx(j)[d] = e4m3(code[j][d]) * scale[j]. */
enum msa_dtype {
    MSA_DTYPE_BF16 = 0,
    MSA_DTYPE_FP8_E4M3 = 1   /* OCP e4m3fn: bias 7, max 448, no inf          */
};

enum {
    MSA_BLOCK_SIZE = 128,    /* tokens per block == tokens per page */
    MSA_HEAD_DIM = 128,      /* head dim of q, k, v, q_idx, k_idx   */
    MSA_MAX_SPEC_DRAFT = 8,  /* max_seq_length 2..8 takes the speculative route */
    MSA_MAX_BLOCKS = 8192,   /* most blocks one sequence may hold (1 Mi tokens) */
    MSA_MAX_TOPK = 512,
    MSA_MAX_KV_HEADS = 256   /* most KV heads (and index heads) of one call     */
};

/* One paged cache (a page pool of one layer). */
typedef struct msa_paged_cache {
    const void* data;        /* device: page pool base, 16-byte aligned           */
    int32_t dtype;           /* enum msa_dtype                                    */
    int32_t num_pages;       /* pages in the pool                                 */
    int32_t num_heads;       /* heads stored per page                             */
    int32_t page_size;       /* must be 128 (MSA_BLOCK_SIZE)                      */
    int32_t head_dim;        /* must be 128 (MSA_HEAD_DIM)                        */
    int32_t reserved;        /* set to 0                                          */
    int64_t page_stride;     /* elements between pages                            */
    int64_t head_stride;     /* elements between heads of one page                */
    int64_t token_stride;    /* elements between slots of one head; >= 128, and   */
                             /* the 128 slots of a page span < 2 GiB              */
                             /* (token_stride * element size * 128 <= INT32_MAX)  */
    /* Per-token dequantization scales: FP8 index-K caches only (NULL for
     * BF16 caches and for K/V).  The scale of slot t of head h of page p is
     * scale[p*scale_page_stride + h*scale_head_stride + t]; the 128 slots of
     * a head are contiguous.  16-byte aligned, strides multiples of 4.  The
     * scales may sit inside the code pages (e.g. each head's 128 x 128 codes
     * followed by its 128 scales: 132 bytes per token). */
    const float* scale;
    int64_t scale_page_stride;  /* floats between pages                          */
    int64_t scale_head_stride;  /* floats between heads of one page              */
} msa_paged_cache;

/* The ragged batch: which rows are whose, and where their KV lives. */
typedef struct msa_ragged {
    const int32_t* input_row_offsets; /* device [batch+1]: prefix sums of new    */
                                      /* tokens per sequence, [0] = 0            */
    const int32_t* cache_lengths;     /* device [batch]: tokens cached before    */
                                      /* this step's new tokens                  */
    const int32_t* kv_lookup_table;   /* device [batch][lookup_stride]: page id  */
                                      /* of each logical block                   */
    int32_t lookup_stride;            /* entries per sequence in the table;      */
                                      /* blocks at or past it are never read     */
    int32_t batch;                    /* sequences                               */
    int32_t max_seq_length;           /* host bound on new tokens per sequence;  */
                                      /* picks the route: 1 decode, 2..8         */
                                      /* speculative decode, > 8 prefill         */
    int32_t max_cache_length;         /* host bound on cache_lengths[b]          */
} msa_ragged;

/* ------------------------------------------------------------------------ */
/* Bad device data                                                          */
/* ------------------------------------------------------------------------ */

/* The kernels never read outside the caller's buffers, whatever the device
 * data holds: a page id outside [0, num_pages) skips its block (or stands
 * in page 0 for it), and per-sequence new-token counts or lengths beyond
 * what max_seq_length and the lookup table allow are clipped.  The result
 * of the sequence concerned is then undefined; every other sequence's is
 * exact.  Such data also sets bits in a per-device error word: */
enum {
    MSA_DEVERR_PAGE = 1,     /* a lookup-table page id outside the pool       */
    MSA_DEVERR_LENGTH = 2    /* a new-token count above max_seq_length, or a   */
                             /* sequence longer than its lookup-table row      */
};

/*
 * Reads the current device's error word into *bits after everything
 * enqueued on `stream` so far has run, and with clear != 0 resets it to 0.
 * Synchronises the stream (a diagnostic call, not for graph capture).  The
 * word collects bits from every call on the device since the last clear.
 *
 * Errors: MSA_ERR_NULL (bits), MSA_ERR_DEVICE, MSA_ERR_LAUNCH.
 */
int msa_device_errors(uint32_t* bits, int clear, void* stream);

/* ------------------------------------------------------------------------ */
/* Indexer                                                                  */
/* ------------------------------------------------------------------------ */

/* Workspace bytes msa_indexer_paged needs for this batch shape.  Returns 0 on
 * invalid arguments (and then msa_indexer_paged reports the error). */
size_t msa_indexer_workspace_bytes(const msa_ragged* rg, int32_t num_kv_heads,
                                   int32_t top_k);

/*
 * Block selection ("ferrox_core::block_sparse", "Four rules" section and the
 * block_sparse_select function; "msa" page: the indexer emits top-k block
 * ids per (index head, token)).
 *
 * For every row r (token at position p, nb visible blocks) and KV head h:
 *   F = {0 .. min(init_blocks, nb)-1} U {max(0, nb-local_blocks) .. nb-1}.
 *   If nb <= top_k the selection is every visible block 0 .. nb-1.
 *   Otherwise every block outside F is scored with
 *     s(blk) = max over j in blk, j <= p of  sum_d q_idx[r][h][d] * k_idx(j)[d]
 *   (FP32 accumulation, no softmax scale), where k_idx(j) is head
 *   h % index_k->num_heads of position j in the index-K cache (for an FP8
 *   cache, e4m3(code) * scale of that slot: the dot product of q_idx with
 *   the codes, then times the scale), and the
 *   top_k - |F| highest scores join F; equal scores go to the lower id.
 *   d_indices[r][h][:] = the selection in ascending order, padded with -1.
 *
 * d_indices     device int32 [batch*max_seq_length rows max][num_kv_heads][top_k];
 *               rows >= input_row_offsets[batch] are not written.
 * q_idx         device bf16 [rows][num_kv_heads][128].
 * num_kv_heads  1 .. MSA_MAX_KV_HEADS.
 * index_k       BF16 cache, or FP8 e4m3 cache with per-token scales (scale
 *               non-NULL), with num_heads 1 (shared by all KV heads) or
 *               num_kv_heads.
 * top_k         1 .. MSA_MAX_TOPK; init_blocks, local_blocks >= 0 with
 *               init_blocks + local_blocks <= top_k.
 * workspace     device, >= msa_indexer_workspace_bytes(...) bytes.
 *
 * Errors: MSA_ERR_NULL, MSA_ERR_SHAPE, MSA_ERR_PARAM, MSA_ERR_DTYPE,
 * MSA_ERR_WORKSPACE, MSA_ERR_LAUNCH.  batch == 0 is a no-op.
 */
int msa_indexer_paged(int32_t* d_indices, const void* q_idx,
                      const msa_paged_cache* index_k, const msa_ragged* rg,
                      int32_t num_kv_heads, int32_t top_k, int32_t init_blocks,
                      int32_t local_blocks, void* workspace, size_t workspace_bytes,
                      void* stream);

/*
 * Reuse of a previous step's block selection across draft steps
 * ("DeepSeekSparseAttentionConfig" page, index_share_for_mtp_iteration
 * field: reuse the indexer top-k across MTP draft steps instead of
 * recomputing it).  The rows of a draft step take the selection of a row of
 * an earlier step unchanged, for every KV head:
 *   d_indices[r][h][:] = prev_indices[src_row[r]][h][:]   for r < rows;
 * a row whose src_row[r] is outside [0, prev_rows) gets -1 everywhere (no
 * block).  The attention then applies each row's own causal clip (j <= p)
 * to the reused blocks; blocks a later position could see but the source
 * row did not select are not attended.
 *
 * d_indices     device int32 [rows][num_kv_heads][top_k], written.
 * prev_indices  device int32 [prev_rows][num_kv_heads][top_k]; may not
 *               overlap d_indices.
 * src_row       device int32 [rows].
 *
 * Errors: MSA_ERR_NULL, MSA_ERR_PARAM, MSA_ERR_SHAPE, MSA_ERR_LAUNCH.  rows
 * == 0 is a no-op.
 */
int msa_indexer_reuse(int32_t* d_indices, const int32_t* prev_indices, const int32_t* src_row,
                      int32_t rows, int32_t prev_rows, int32_t num_kv_heads, int32_t top_k,
                      void* stream);

/* ------------------------------------------------------------------------ */
/* Sparse attention                                                         */
/* ------------------------------------------------------------------------ */

/* Number of split-K partitions msa_attention_paged uses for this shape when
 * called with num_partitions (0 = automatic choice that fills the GPU's
 * compute units).  Prefill (max_seq_length > 8) always uses 1.  Returns a
 * negative MSA_ERR_* code on invalid arguments. */
int msa_attention_partitions(const msa_ragged* rg, int32_t num_q_heads,
                             int32_t num_kv_heads, int32_t top_k,
                             int32_t num_partitions);

/* Workspace bytes msa_attention_paged and msa_attention_paged_shared need
 * (split-K ready flags and partials, and the union-tile plan of
 * prefill and of shared speculative steps).  Returns 0 on invalid
 * arguments.  The workspace needs no initial contents. */
size_t msa_attention_workspace_bytes(const msa_ragged* rg, int32_t num_q_heads,
                                     int32_t num_kv_heads, int32_t top_k,
                                     int32_t num_partitions);

/*
 * Sparse attention over the selected blocks ("ferrox_core::block_sparse",
 * positions_of_blocks and the masked attention pass it feeds; "msa" page,
 * routes: decode, speculative decode with per-token causality, prefill).
 *
 * For row r at position p and query head g of KV head h = g / G:
 *   P   = { j : j / 128 in d_indices[r][h][:], j <= p }   (ids < 0 ignored)
 *   out[r][g] = sum_{j in P} softmax_j(scale * q[r][g] . k(j)) v(j)
 * with FP32 accumulation, rounded to BF16 (round to nearest even).  A row
 * with no position in P gets 0.  Each row's ids must be distinct; their
 * order does not matter.
 *
 * output        device bf16 [rows][num_q_heads][128]; rows >=
 *               input_row_offsets[batch] are not written.
 * q             device bf16 [rows][num_q_heads][128].
 * d_indices     device int32 [rows][num_kv_heads][top_k] (the indexer's output).
 * k_cache, v_cache  caches with num_heads == num_kv_heads and the same dtype
 *               (BF16 or FP8 e4m3, scale-free: scale must be NULL).
 * num_kv_heads  1 .. MSA_MAX_KV_HEADS.
 * num_q_heads   a multiple of num_kv_heads with group size 1, 2, 4, 8 or 16.
 * scale         softmax scale applied to q.k (e.g. 1/sqrt(128)); positive
 *               and finite.
 * num_partitions 0 = automatic, else 1 .. 64 (decode / speculative routes).
 * workspace     device, >= msa_attention_workspace_bytes(...) bytes.
 *
 * With more than one partition, each partition stores its partial result
 * (as msa_splitk_combine takes them) and a ready flag in the workspace, and
 * the group's last partition merges them in partition order inside the
 * same launch (no separate combine launch).  Flags carry a tag of the call
 * and the merging partition clears them, so the workspace needs no initial
 * contents and no clearing between calls, and the call stays capturable in
 * a HIP graph.  Two calls that overlap on one workspace race.
 * Errors: as msa_indexer_paged.  batch == 0 is a no-op.
 */
int msa_attention_paged(void* output, const void* q, const int32_t* d_indices,
                        const msa_paged_cache* k_cache, const msa_paged_cache* v_cache,
                        const msa_ragged* rg, int32_t num_q_heads, int32_t num_kv_heads,
                        int32_t top_k, float scale, int32_t num_partitions,
                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * The same operation as msa_attention_paged, with the same arguments and
 * result, scheduled for speculative steps whose rows of one sequence share
 * one selection: draft steps that reuse a selection through
 * msa_indexer_reuse ("DeepSeekSparseAttentionConfig" page,
 * index_share_for_mtp_iteration field), with the per-token causality of the
 * "msa" page's speculative route.
 *
 * When 2 <= max_seq_length <= 8, each group of tokens of a sequence (all of
 * them, or 4 at group size 16) reads the union of its rows' blocks once,
 * and the tokens share each staged block; num_partitions is then ignored
 * and no combine runs.  Other shapes take msa_attention_paged's routes.  The
 * result is correct for any selection and equals msa_attention_paged's
 * within rounding; when the rows of a sequence select different blocks the
 * union grows and this entry point is slower, so it is a scheduling hint,
 * not a different operation.
 *
 * workspace     device, >= msa_attention_workspace_bytes(...) bytes (that
 *               size covers both entry points).
 *
 * Errors: as msa_attention_paged.
 */
int msa_attention_paged_shared(void* output, const void* q, const int32_t* d_indices,
                               const msa_paged_cache* k_cache, const msa_paged_cache* v_cache,
                               const msa_ragged* rg, int32_t num_q_heads, int32_t num_kv_heads,
                               int32_t top_k, float scale, int32_t num_partitions,
                               void* workspace, size_t workspace_bytes, void* stream);

/*
 * msa_attention_paged for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Same arguments, semantics, kernels and results as
 * msa_attention_paged, without the workspace arguments: the workspace comes
 * from one fixed device array of MSA_NOALLOC_SCRATCH_BYTES that the library
 * holds on every GPU it runs on until the process ends.  The call allocates
 * nothing (no hipMalloc, hipFree or allocating library routine).
 *
 * Limit: a shape whose msa_attention_workspace_bytes(...) exceeds
 * MSA_NOALLOC_SCRATCH_BYTES is rejected with MSA_ERR_SCRATCH before any
 * launch (64 MiB hold, e.g., a 29,696-token prefill over 8 KV heads, or
 * split-K decode partials of up to 8 partitions x 2048 rows x 64 heads).
 *
 * Sharing: every call on one GPU uses that GPU's one array, so calls that
 * overlap on one GPU (different streams, or host threads) race and must be
 * serialised by the caller; calls in order on one stream are safe.
 *
 * Errors: as msa_attention_paged, plus MSA_ERR_SCRATCH.
 */
enum { MSA_NOALLOC_SCRATCH_BYTES = 64 * 1024 * 1024 };

int msa_attention_paged_noalloc(void* output, const void* q, const int32_t* d_indices,
                                const msa_paged_cache* k_cache, const msa_paged_cache* v_cache,
                                const msa_ragged* rg, int32_t num_q_heads, int32_t num_kv_heads,
                                int32_t top_k, float scale, int32_t num_partitions,
                                void* stream);

/*
 * Split-K combine ("msa" page: partials keyed on the ragged global query
 * row; the shared combine writes the ragged output directly).  The merge
 * msa_attention_paged performs inside its kernel, as a call of its own for
 * partials computed elsewhere.
 *
 * Partition pi of row r, query head g holds its own normalised output
 * o_pi = partial_o[pi][r][g][:] and the natural log of its softmax
 * denominator lse_pi = partial_lse[pi][r][g] (-inf: no positions).  The
 * result is sum_pi exp(lse_pi - LSE) o_pi with LSE = log sum_pi exp(lse_pi),
 * rounded to BF16; 0 when every lse_pi is -inf.
 *
 * output        device bf16 [rows][num_q_heads][128].
 * partial_o     device f32 [num_partitions][batch*max_seq_length][num_q_heads][128].
 * partial_lse   device f32 [num_partitions][batch*max_seq_length][num_q_heads].
 * input_row_offsets device int32 [batch+1].
 *
 * Errors: MSA_ERR_NULL, MSA_ERR_PARAM, MSA_ERR_LAUNCH.
 */
int msa_splitk_combine(void* output, const float* partial_o, const float* partial_lse,
                       const int32_t* input_row_offsets, int32_t batch,
                       int32_t max_seq_length, int32_t num_partitions,
                       int32_t num_q_heads, void* stream);

/* ------------------------------------------------------------------------ */
/* Latent sparse attention                                                  */
/* ------------------------------------------------------------------------ */

/*
 * The second operation of the family: the mo.latent_sparse_attention.
 * ragged.paged graph op ("Struct_latent_sparse_attention_ragged_paged" page
 * of the MAX Mojo docs, struct summary and the execute argument list).  One
 * latent vector per cached entry is both key and value; entries come from
 * two paged leaves, a sliding-window leaf read by a range of positions and
 * a compressed leaf read through an explicit list of entries per query; a
 * per-head attention sink enters the softmax denominator.
 *
 * One leaf as the operation sees it: its page pool (head_dim 128, 128
 * entries per page, num_heads = latent heads, BF16 or scale-free FP8 e4m3,
 * scale NULL) and how the sequences map into it.  Entry i of sequence b is
 * slot i % 128 of page lookup_table[b * lookup_stride + i / 128]; the page's
 * layer is chosen by passing that layer's pool.
 */
typedef struct msa_latent_leaf {
    msa_paged_cache cache;
    const int32_t* cache_lengths;  /* device [batch]                              */
    const int32_t* lookup_table;   /* device [batch][lookup_stride]: page ids     */
    int32_t lookup_stride;         /* entries per sequence in the table           */
    int32_t max_cache_length;      /* host bound on cache_lengths[b]              */
} msa_latent_leaf;

enum {
    MSA_LATENT_MAX_TOPC = 16384,   /* most list slots per (row, latent head)     */
    MSA_LATENT_MAX_WINDOW = 1 << 20
};

/* Split-K partitions msa_latent_attention_paged uses for this shape when
 * called with num_partitions (0 = automatic choice that fills the GPU).
 * Returns a negative MSA_ERR_* code on invalid arguments. */
int msa_latent_partitions(int32_t batch, int32_t max_seq_length, int32_t num_heads,
                          int32_t num_latent_heads, int32_t window, int32_t top_c,
                          int32_t num_partitions);

/* Workspace bytes msa_latent_attention_paged needs (split-K partials when
 * more than one partition is used).  Returns 0 on invalid arguments. */
size_t msa_latent_workspace_bytes(int32_t batch, int32_t max_seq_length, int32_t num_heads,
                                  int32_t num_latent_heads, int32_t window, int32_t top_c,
                                  int32_t num_partitions);

/*
 * For row r = input_row_offsets[b] + t (new token t of sequence b, at
 * window-leaf position p = swa->cache_lengths[b] + t) and query head g of
 * latent head hl = g / (num_heads / num_latent_heads):
 *   W = window-leaf positions max(0, p - window + 1) .. p  (none if window 0)
 *   C = the values e of comp_indices[r][hl][0 .. top_c) with
 *       0 <= e < comp->cache_lengths[b], each occurrence counted
 *   z_j = scale * q[r][g] . x_j for every latent vector x_j of W and C
 *   out[r][g] = sum_j exp(z_j) x_j / (sum_j exp(z_j) + exp(attn_sink[g]))
 * with FP32 accumulation, rounded to BF16 (round to nearest even).  A sink
 * of -inf means no sink; a row with nothing to attend gets 0.  Sinks must be
 * finite or -inf, attended latent values finite.
 *
 * output            device bf16 [rows][num_heads][128]; rows >=
 *                   input_row_offsets[batch] are not written.
 * q                 device bf16 [rows][num_heads][128].
 * input_row_offsets device int32 [batch + 1].
 * max_seq_length    host bound on new tokens per sequence.
 * comp_indices      device int32 [rows][num_latent_heads][top_c]; may be
 *                   NULL when top_c == 0.
 * attn_sink         device float32 [num_heads].
 * swa, comp         the two leaves (num_heads == num_latent_heads in both);
 *                   swa may be NULL when window == 0, comp when top_c == 0.
 *                   Each leaf is BF16 or FP8 e4m3 (its own storage type,
 *                   as the page's swa_type / comp_type); FP8 codes are
 *                   widened to BF16 exactly.  Leaves of two types take two
 *                   launches (one per leaf) whose partials the second
 *                   launch merges, so such a call uses at least two
 *                   partitions (the workspace query reserves them).
 *                   swa->lookup_stride must cover positions up to
 *                   swa->max_cache_length + max_seq_length - 1, and
 *                   comp->lookup_stride entries up to comp->max_cache_length - 1.
 * num_heads         a multiple of num_latent_heads (any group size).
 * window            0 .. MSA_LATENT_MAX_WINDOW; top_c 0 .. MSA_LATENT_MAX_TOPC.
 * scale             positive and finite.
 * num_partitions    0 = automatic, else 1 .. 64.
 * workspace         device, >= msa_latent_workspace_bytes(...) bytes.
 *
 * Errors: MSA_ERR_NULL, MSA_ERR_SHAPE, MSA_ERR_PARAM, MSA_ERR_DTYPE,
 * MSA_ERR_WORKSPACE, MSA_ERR_LAUNCH, MSA_ERR_DEVICE.  batch == 0 is a no-op.
 * With more than one partition, the last partition of each (row, latent
 * head, group of 64 query heads) merges the partitions' results inside the
 * same launch (no combine launch); the workspace needs no initial contents.
 */
int msa_latent_attention_paged(void* output, const void* q, const int32_t* input_row_offsets,
                               int32_t batch, int32_t max_seq_length,
                               const int32_t* comp_indices, int32_t top_c,
                               const float* attn_sink, const msa_latent_leaf* swa,
                               const msa_latent_leaf* comp, int32_t num_heads,
                               int32_t num_latent_heads, int32_t window, float scale,
                               int32_t num_partitions, void* workspace, size_t workspace_bytes,
                               void* stream);

/* Human-readable name of a status code (static string). */
const char* msa_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* MSA_H */
