/*
 * swan.h -- C ABI of the SWAN hybrid-cache decode step on gfx950 (MI355X).
 *
 * SWAN ("Sparse Winnowed Attention ... via Decompression-Free KV-Cache
 * Compression", arXiv 2511.18936) keeps a small dense buffer of the R most
 * recent rotated keys/values and a large sparse history in which every older
 * rotated key and value keeps only its k largest-magnitude coordinates as
 * (8-bit index, fp16 value) pairs.  One decode step (SWAN page, hybrid-cache
 * paragraphs):
 *
 *   1. swan_project_qk    q_hat = RoPE(q) P_QK, k_hat = RoPE(k) P_QK
 *   2. swan_append_evict  put (k_hat, v_hat) in the dense buffer; the token
 *                         that leaves the buffer is pruned to its top-k
 *                         coordinates and appended to the sparse history
 *   3. swan_decode_attn   scores of q_hat against sparse + dense keys, one
 *                         softmax over both, output accumulated from sparse +
 *                         dense values, in the rotated value basis
 *
 * plus swan_prefill_convert, which turns a prefilled history into the
 * hybrid cache in one call.
 *
 * Conventions
 * -----------
 * - All array arguments are DEVICE pointers unless marked (host).  The
 *   library allocates nothing and keeps no state between calls; the caller
 *   owns every buffer.  Work is enqueued on `stream` (a hipStream_t; NULL is
 *   the null stream) and returns without synchronising.
 * - Host-side validation happens before any launch.  A failed call enqueues
 *   nothing and returns a status != SWAN_OK; swan_last_error() (host,
 *   thread-local) describes the failure.  A failed launch returns
 *   SWAN_ERR_HIP.
 * - d_h must be 128 (indices fit in 8 bits: SWAN page, memory-savings
 *   paragraphs).  The GQA group g = N_h / H_kv must be 1, 2, 4 or 8.
 *   1 <= k <= d_h.
 * - fp16 arrays hold IEEE binary16 bit patterns (uint16_t).
 * - pos[b] (int32, device) is the position (0-based) of the token appended
 *   by this step for sequence b.  After swan_append_evict the cache holds
 *   tokens 0..pos[b]: n_b = max(0, pos[b] + 1 - R) sparse rows (row t = token
 *   t) and min(pos[b] + 1, R) buffered tokens in slots t mod R (a circular
 *   buffer, "Reuse, Evict, or Limit Earlier Context" section 3.2).  A
 *   sequence with pos[b] < 0 is inactive: nothing is appended and its output
 *   rows are zero.
 * - Several layers can share one batch (dims->layers): their sequences are
 *   stacked layer-major along B in the same cache planes (contiguous) or the
 *   same pool and block table (paged), so one launch of each kernel serves
 *   every layer, e.g. the layers of micro-batches pipelined through a model.
 *   Only the projection and the prefill tell layers apart (their P_QK).
 * - max_pos (host) must be >= every pos[b]; it sizes grids and is checked
 *   against the sparse capacity.  A device pos[b] above max_pos gives
 *   undefined results for that sequence but no out-of-bounds access.
 *
 * Cache layout (all planes caller-allocated, sizes from swan_cache_bytes)
 * ------------
 * Each sparse key row stores k_stride = swan_row_stride(k) entries and each
 * value row v_stride = swan_row_stride(k_v ? k_v : k) (the count rounded up
 * to a power of two, at least 8, so a row splits evenly over lane slices);
 * entries past the kept count are padding with index 0 and value +0, which
 * contribute nothing to scores or outputs.
 *   contiguous (block_size == 0):
 *     k_idx         uint8   [B][H_kv][n_cap][k_stride]
 *     k_val         fp16 or fp8 (value_format) [B][H_kv][n_cap][k_stride]
 *     v_idx, v_val  likewise with v_stride
 *   paged (block_size > 0, "Reuse, Evict, or Limit Earlier Context" 1.2):
 *     k_idx, k_val  [num_blocks][H_kv][block_size][k_stride]
 *     v_idx, v_val  [num_blocks][H_kv][block_size][v_stride]
 *     block_table   int32   [B][max_blocks]: sparse row t of sequence b is
 *                   slot t % block_size of block block_table[b][t / block_size]
 *     Any block_size >= 1 works.  Powers of two >= 16 are the fast path:
 *     the decode reads each run of 8 or 16 rows through one block; other
 *     sizes look the block up for every row.
 *   dense buffer:
 *     k_buf, v_buf  fp16    [B][H_kv][R][128], slot = position mod R
 * Every plane must be 16-byte aligned.
 * Kept entries of a row are stored with ascending, distinct indices (as
 * swan_append_evict and swan_prefill_convert write them); swan_decode_attn
 * relies on the indices of a row being distinct.
 */
#ifndef SWAN_H
#define SWAN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum swan_status {
    SWAN_OK = 0,
    SWAN_ERR_INVALID_ARG = 1, /* null pointer, inconsistent sizes, workspace too small */
    SWAN_ERR_UNSUPPORTED = 2, /* d_h != 128, g not in {1,2,4,8} */
    SWAN_ERR_CAPACITY = 3,    /* max_pos needs more sparse rows than the cache holds */
    SWAN_ERR_HIP = 4          /* a HIP launch failed */
} swan_status;

/* Problem sizes, in the pages' notation (host struct, read during the call). */
typedef struct swan_dims {
    int32_t B;            /* sequences in the batch                               */
    int32_t N_h;          /* query heads                                          */
    int32_t H_kv;         /* kv heads; g = N_h / H_kv query heads share each one   */
    int32_t d_h;          /* head dimension, must be 128                           */
    int32_t R;            /* dense buffer capacity in tokens (0 = no buffer)       */
    int32_t k;            /* coordinates kept per pruned vector, 1..d_h            */
    int32_t n_cap;        /* contiguous layout: sparse rows per (sequence, kv head)*/
    int32_t block_size;   /* 0 = contiguous sparse rows, >0 = rows per paged block */
    int32_t max_blocks;   /* paged: block-table entries per sequence               */
    int32_t num_blocks;   /* paged: blocks in the pool                             */
    int32_t split_tokens; /* decode: work rows per wave (multiple of 64), 0 = auto */
    int32_t value_format; /* sparse values: SWAN_VALUES_FP16 (0) or SWAN_VALUES_FP8_E4M3 */
    int32_t k_v;          /* coordinates kept per pruned value vector, 0 = k (keys keep k)
                             (SWAN Appendix A.5, Table 2: keys and values may keep
                             different shares of d_h); swan_row_stride(k_v) must equal
                             swan_row_stride(k), twice it or half of it */
    int32_t layers;       /* layers whose sequences share the batch, 0 or 1 = one:
                             B counts the sequences of all layers, layer-major, so
                             sequence b belongs to layer b / (B / layers) and is
                             projected with that layer's P_QK; every decode call
                             covers all layers in one split and one reduce launch */
} swan_dims;

/* Storage of the values of sparse rows (the dense buffer is always fp16).
 * FP8_E4M3 is the 8-bit float storage the SWAN page's memory-savings
 * paragraphs allow (2k + 2 bytes a vector) in the OCP E4M3 encoding
 * (exponent bias 7, 3 fraction bits, largest finite value 448, no
 * infinities), with no scale:
 * a pruned row keeps the same coordinates as with fp16 values (chosen on the
 * fp16 magnitudes) and each kept value is rounded from fp16 to nearest even,
 * saturating at +-448. */
#define SWAN_VALUES_FP16 0
#define SWAN_VALUES_FP8_E4M3 1

/* Caller-owned cache planes (host struct holding device pointers). */
typedef struct swan_cache {
    uint8_t *k_idx;
    void *k_val; /* fp16 or fp8 E4M3 entries (dims->value_format) */
    uint8_t *v_idx;
    void *v_val;
    uint16_t *k_buf;
    uint16_t *v_buf;
    const int32_t *block_table; /* paged layout only; NULL when contiguous */
} swan_cache;

/* Human-readable name of a status (static string). */
const char *swan_status_str(swan_status s);

/* Detail of the last failed call on this host thread (static per thread). */
const char *swan_last_error(void);

/* Entries stored per sparse row: k rounded up to a power of two, >= 8. */
int32_t swan_row_stride(int32_t k);

/* Bytes of each cache plane for `dims` (host): out[0] = k_idx, out[1] =
 * k_val, out[2] = v_idx, out[3] = v_val, out[4] = k_buf (= v_buf).  Returns
 * the status of validating dims. */
swan_status swan_cache_bytes(const swan_dims *dims, size_t out[5]);

/*
 * Step 1 -- runtime projection (SWAN page, projection-absorption paragraphs:
 * RoPE cannot be absorbed into W_Q / W_K, so q -> RoPE(q) -> RoPE(q) P_QK
 * runs every step).
 *   q      float32 [B][N_h][128]   raw queries (before RoPE)
 *   k      float32 [B][H_kv][128]  raw new keys (before RoPE)
 *   pos    int32   [B]             rotation position of each sequence
 *   P_qk   float32 [layers][H_kv][128][128] row-vector convention: x_hat =
 *                                  x P, element [l][h][c][j]; query head j
 *                                  of a sequence of layer l uses P_qk[l][j / g]
 *   rope_base                      RoPE base (10000 for Llama-3)
 *   q_hat  float32 [B][N_h][128]   out: rotated queries
 *   k_hat  fp16    [B][H_kv][128]  out: rotated keys, rounded to nearest even
 * RoPE rotates pair (i, i + 64) by pos * rope_base^(-i/64).  Sequences with
 * pos < 0 are projected at position 0.
 */
swan_status swan_project_qk(const swan_dims *dims, const float *q, const float *k, const int32_t *pos,
                            const float *P_qk, float rope_base, float *q_hat, uint16_t *k_hat, void *stream);

/*
 * Step 2 -- append the new token, evict and prune (SWAN page, hybrid-cache
 * and pruning paragraphs: when the buffer exceeds its capacity the oldest
 * vectors are evicted, pruned to their top-k magnitude coordinates and
 * appended to the sparse cache).
 *   k_hat  fp16    [B][H_kv][128]  rotated new keys (from swan_project_qk)
 *   v_hat  float32 [B][H_kv][128]  new values, already in the rotated basis
 *                                  (P_VO absorbed into W_V: SWAN page,
 *                                  projection-absorption paragraphs);
 *                                  rounded to fp16 (nearest even) on store
 * For R > 0 the token at pos - R (if pos >= R) is read from slot pos mod R,
 * pruned into sparse row pos - R, and the new token takes the slot.  For
 * R == 0 the new token is pruned straight into sparse row pos.  Pruning keeps
 * the k (values: k_v) coordinates first in the order (|x| descending as fp16
 * magnitude, index ascending) and copies their values bit for bit (8-bit
 * values: rounds them to E4M3 as described above).  In the paged layout
 * the block holding the new row must be allocated and exclusively owned by
 * the sequence (copy-on-write is the caller's job).
 */
swan_status swan_append_evict(const swan_dims *dims, const swan_cache *cache, const int32_t *pos, int32_t max_pos,
                              const uint16_t *k_hat, const float *v_hat, void *stream);

/*
 * Steps 1 and 2 in one launch: swan_project_qk followed by
 * swan_append_evict, with the same arguments, layouts, results and checks
 * as the two calls (q_hat and k_hat are written as well).  Within the launch
 * each (sequence, kv head) appends as soon as its own new key is projected,
 * so the step needs one launch and no grid-wide wait between the two.
 */
swan_status swan_project_append(const swan_dims *dims, const swan_cache *cache, const float *q, const float *k,
                                const float *v_hat, const int32_t *pos, int32_t max_pos, const float *P_qk,
                                float rope_base, float *q_hat, uint16_t *k_hat, void *stream);

/* Bytes of scratch memory swan_decode_attn needs for max_pos (host); 0 if
 * dims are invalid. */
size_t swan_decode_workspace_bytes(const swan_dims *dims, int32_t max_pos);

/* Number of waves of the split pass swan_decode_attn launches for max_pos
 * (host); -1 if dims are invalid.  The batch's work rows are spread evenly
 * over them: a unit (sequence, kv head) counts its sparse rows plus its
 * buffered tokens weighted 256 / (3 swan_row_stride(k)) rows each (their
 * bytes relative to a sparse row), each part rounded up to 16; a wave takes
 * split_tokens consecutive work rows, or with split_tokens = 0 an equal share
 * (a multiple of 16, at least 64) of the batch's total.  A piece of a unit
 * takes the same fraction of its sparse rows and of its buffered tokens; a
 * wave that covers pieces of several units writes one partial per piece. */
int32_t swan_decode_num_splits(const swan_dims *dims, int32_t max_pos);

/*
 * Step 3 -- hybrid decode attention (SWAN page, hybrid-cache paragraphs and
 * Appendix A.2, steps 2-4).  For every query head of sequence b, over the n_b sparse and
 * min(pos[b] + 1, R) buffered tokens of its kv head:
 *   s_t = (sum_i q_hat[idx_t,i] val_t,i) / sqrt(128)  for sparse tokens
 *   s_t = (q_hat . k_t) / sqrt(128)                    for buffered tokens
 *   o_hat = sum_t softmax(s)_t v_t, sparse v_t scattered to its indices
 *   q_hat  float32 [B][N_h][128]
 *   o_hat  float32 [B][N_h][128]   out, in the rotated value basis
 *   workspace  device scratch of at least swan_decode_workspace_bytes()
 * Two kernels: a split kernel (wavefronts over equal shares of the batch's
 * work, each piece of a (sequence, kv head) serving the g query heads of the
 * group with an online softmax) and a reduce kernel that merges the pieces.
 * Every pos[b] must be <= max_pos: rows of a longer sequence can fall beyond
 * the last wave and are then left out (no access outside the buffers).
 */
swan_status swan_decode_attn(const swan_dims *dims, const swan_cache *cache, const int32_t *pos, int32_t max_pos,
                             const float *q_hat, float *o_hat, void *workspace, size_t workspace_bytes,
                             void *stream);

/*
 * swan_decode_attn without a workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, serving loops that must not
 * call hipMalloc, harnesses that forbid allocation).  Same arguments, checks
 * and results as swan_decode_attn, and the same two kernels; the split
 * pass's partials go to a scratch array the library holds on every GPU it
 * runs on: SWAN_NOALLOC_SCRATCH_BYTES (16 MiB) of device memory reserved
 * when the library's code is loaded on that GPU and kept until the process
 * ends.  The call allocates nothing.
 *   - SWAN_ERR_CAPACITY when the plan's partials (swan_decode_workspace_bytes
 *     for these dims and max_pos) exceed the scratch size: about 8000 pieces
 *     of work at g = 4 (the automatic plan of a batch with up to ~6000
 *     (sequence, kv head) units), half that at g = 8.
 *   - `stream` must belong to the current device (SWAN_ERR_INVALID_ARG
 *     otherwise); the scratch address of a device is looked up on the first
 *     call on it.
 *   - Every call on one GPU shares that GPU's array: calls that overlap
 *     (on different streams, or enqueued from several host threads without
 *     ordering) race and give wrong results.  Calls ordered on one stream are
 *     safe; each writes every partial it reads, so nothing carries over from
 *     the previous call.
 */
#define SWAN_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
swan_status swan_decode_attn_noalloc(const swan_dims *dims, const swan_cache *cache, const int32_t *pos,
                                     int32_t max_pos, const float *q_hat, float *o_hat, void *stream);

/* The two halves of swan_decode_attn, for callers that time or schedule them
 * separately: the split pass writes per-piece partials to the workspace, the
 * reduce pass merges them into o_hat.  Same arguments and checks; the two
 * calls must see the same pos and max_pos. */
swan_status swan_decode_split(const swan_dims *dims, const swan_cache *cache, const int32_t *pos, int32_t max_pos,
                              const float *q_hat, void *workspace, size_t workspace_bytes, void *stream);
swan_status swan_decode_reduce(const swan_dims *dims, const int32_t *pos, int32_t max_pos, const void *workspace,
                               size_t workspace_bytes, float *o_hat, void *stream);

/*
 * Prefill -> hybrid cache.  Sequence b has len[b] prefilled tokens at
 * positions 0..len[b]-1 (max_len host bound, 0 <= len[b] <= max_len); its
 * keys are projected with the P_QK of its layer ([layers][H_kv][128][128]):
 *   k_raw  float32 [B][H_kv][T_stride][128]  raw keys (before RoPE)
 *   v_hat  float32 [B][H_kv][T_stride][128]  values in the rotated basis
 * Each key gets RoPE at its own position and P_qk; keys and values are
 * rounded to fp16.  Tokens 0..len-R-1 are pruned into sparse rows, the last
 * min(len, R) go to buffer slots t mod R -- the same state as appending the
 * tokens one by one.  In the paged layout every block the rows fall in must
 * be allocated.
 */
swan_status swan_prefill_convert(const swan_dims *dims, const swan_cache *cache, const int32_t *len, int32_t max_len,
                                 int64_t T_stride, const float *k_raw, const float *v_hat, const float *P_qk,
                                 float rope_base, void *stream);

/*
 * Copy-on-write support for the paged layout ("Reuse, Evict, or Limit
 * Earlier Context" sections 1.3 and 1.4: a block referenced by more than one
 * sequence is never written; a writer first copies it to a block it owns).
 * Copies blocks src[i] -> dst[i], i < count, in all four sparse planes:
 *   src, dst   int32 [count] (device) block ids of the pool
 * Reference counts, the free list and the block tables are the caller's
 * (host) bookkeeping; this call only moves the bytes, asynchronously on
 * stream.  A pair with an id outside 0..num_blocks-1 or src == dst is
 * skipped.  The dst blocks must not be read or written by other work on
 * the stream until the copy is done (stream order guarantees this).
 * Errors: INVALID_ARG for a contiguous layout, count < 0 or > 65535, or
 * NULL arrays (count > 0); UNSUPPORTED when H_kv * block_size * k_stride is
 * not a multiple of 16 (blocks are moved in 16-byte units).
 */
swan_status swan_copy_blocks(const swan_dims *dims, const swan_cache *cache, const int32_t *src, const int32_t *dst,
                             int32_t count, void *stream);

/*
 * The host side of a paged step handed to the device by value: block-table
 * writes and copy-on-write copies (the bookkeeping of "Reuse, Evict, or
 * Limit Earlier Context" sections 1.2-1.4) carried in the arguments of the
 * launch itself, so the step enqueues no host-to-device copy.
 *   block_table  int32 [B][max_blocks] (device): must be cache->block_table
 *   entries      int32 [n_entries][2] (host): (b * max_blocks + j, id) sets
 *                block_table[b][j] = id, id in -1..num_blocks-1
 *   copies       int32 [n_copies][2] (host): (src, dst) block pairs, copied
 *                in all four sparse planes as by swan_copy_blocks
 * The host arrays are read before the call returns (any number of pairs;
 * the library splits them over launches of up to 192 entries and 32
 * copies).  Entries and copies are independent: a copy moves pool bytes, an
 * entry changes which block a sequence maps.  Later work on the stream sees
 * both.  Errors: INVALID_ARG for a contiguous layout, a table other than the
 * cache's, negative counts, NULL arrays with a positive count, an entry or a
 * pair outside the pool (nothing is launched then); UNSUPPORTED as for
 * swan_copy_blocks.
 */
swan_status swan_paged_update(const swan_dims *dims, const swan_cache *cache, int32_t *block_table,
                              const int32_t *entries, int32_t n_entries, const int32_t *copies, int32_t n_copies,
                              void *stream);

/*
 * A paged step's steps 1 and 2 and its table update in one launch (the
 * projection and append of swan_project_append with the entries and copies
 * of swan_paged_update; "Reuse, Evict, or Limit Earlier Context" sections
 * 1.2-1.4 for the table, reference counts and copy-on-write).
 *   block_table  int32 [B][max_blocks] (device): must be cache->block_table
 *   entries      int32 [n_entries][2] (host): (b * max_blocks + j, id) sets
 *                block_table[b][j] = id, id in -1..num_blocks-1; slots distinct
 *   copies       int32 [n_copies][3] (host): (src, dst, skip) copies block src
 *                to dst in all four sparse planes except row `skip` of every
 *                head (0..block_size-1, or -1 for none), which is the row this
 *                call's append writes into dst
 * Each sequence's append takes the block of its sparse row from `entries`
 * when they set that slot, else from the table, so the appends, the table
 * writes and the copies run side by side in one launch.  The results are
 * those of swan_paged_update (with full copies) followed by
 * swan_project_append, provided no copy's source block is one an append of
 * this call writes into (a caller precondition, as the exclusive ownership of
 * appended blocks is: a block is copied only when it is shared, and shared
 * blocks are not written).  Up to 192 entries and 32 copies travel in the one
 * launch; more are handed to swan_paged_update first (one launch more, same
 * results).  Errors: those of the two calls, INVALID_ARG for a skip row
 * outside [-1, block_size) or, when the entries travel in the one launch
 * (at most 192), a slot set twice.
 */
swan_status swan_project_append_paged(const swan_dims *dims, const swan_cache *cache, const float *q, const float *k,
                                      const float *v_hat, const int32_t *pos, int32_t max_pos, const float *P_qk,
                                      float rope_base, float *q_hat, uint16_t *k_hat, int32_t *block_table,
                                      const int32_t *entries, int32_t n_entries, const int32_t *copies,
                                      int32_t n_copies, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* SWAN_H */
