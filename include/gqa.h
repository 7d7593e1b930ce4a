/*
 * gqa.h - masked causal grouped-query attention over a paged KV cache, on one
 * AMD Instinct MI355X (gfx950).  Plain C ABI: device pointers, host arrays,
 * sizes and status codes; no C++ or framework types cross it.
 *
 * Sources (cited by page title and section):
 *  [P1] "Prefill：整层状态演化与 KV 建立" (glenzli.com, vol. 2 ch. 2)
 *       2.1 interface and preconditions, 2.2 mask M and the sentinel rule,
 *       2.3 g(h), S, A, O, 2.5 LayerCache and cache invariants, 2.6 prefill
 *       pseudocode (write the used K/V of the valid tokens, then attend),
 *       2.11 failure table.
 *  [P2] "模型执行：从 token 到 Prefill 与 Decode" (blog.mlxb.cc), sections on
 *       prefill/decode shapes (decode: T-1 cached + 1 new = T keys).
 *  [P3] "KV Cache 与 Prefill/Decode 推理路径" (wiki.maxwellmou.com, unit 10):
 *       prompt-edit lesson (keep [0,m), truncate, incremental prefill),
 *       PagedAttention lesson (block table, block floor(t/P), offset t mod P,
 *       any free block, results unchanged), multi-turn incremental prefill
 *       (old prefix fully visible, new block lower-triangular), RoPE paragraph
 *       of the prefix-equality proof.
 *
 * Conventions common to every call
 *  - Every function returns a gqa_status.  On any error other than
 *    GQA_ERR_HIP nothing is launched and no cache state changes ([P1] 2.1:
 *    fail before the first layer); after GQA_ERR_HIP (a failed launch or copy)
 *    the device contents are undefined.  The message is available from
 *    gqa_last_error() on the calling thread.
 *  - Calls that take `stream` (a hipStream_t, NULL = legacy default stream)
 *    only enqueue work on it and return without synchronising.  All device
 *    buffers must stay alive until that work has completed.
 *  - A cache handle is not thread-safe.  Calls on one handle must be issued
 *    from one thread and ordered on one stream.
 *  - Host arrays (masks, positions, sequence ids, lengths) are read before the
 *    call returns and may be reused immediately.
 */
#ifndef GQA_H
#define GQA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum gqa_status {
  GQA_OK = 0,
  GQA_ERR_ARG = -1,          /* null pointer, out-of-range id, repeated sequence   */
  GQA_ERR_SHAPE = -2,        /* tensor shape/stride/alignment, Hkv does not divide Hq */
  GQA_ERR_DTYPE = -3,        /* tensor dtype differs from the cache dtype          */
  GQA_ERR_MASK = -4,         /* mask entry not 0 or 1                              */
  GQA_ERR_POSITION = -5,     /* positions do not continue the cache ([P1] 2.11)    */
  GQA_ERR_CACHE = -6,        /* cache state violated (lengths, pages in use)       */
  GQA_ERR_OUT_OF_PAGES = -7, /* page pool or a sequence's block table is full      */
  GQA_ERR_UNSUPPORTED = -8,  /* configuration outside what the kernels implement   */
  GQA_ERR_HIP = -9,          /* a HIP runtime call failed                          */
  GQA_ERR_DEVICE = -10       /* a kernel reported a failure (gqa_workspace_status) */
} gqa_status;

typedef enum gqa_dtype { GQA_F32 = 0, GQA_BF16 = 1 } gqa_dtype;

/* Longest query run (rectangular rows n) that gqa_prefill / gqa_attention can
 * send to the split-T kernel: speculative verify chunks and other short runs. */
#define GQA_MAX_CHUNK_TOKENS 16

/* A strided 4-D device tensor.  stride[] is in elements; stride[3] must be 1.
 * For bf16 the data pointer and stride[0..2] must keep every row 16-byte
 * aligned.  Logical shapes used below:
 *   Q, O   [B, Hq,  n, d]     K, V  [B, Hkv, n, d]     q, o (decode) [B, Hq, 1, d] */
typedef struct gqa_tensor {
  void* data;
  int32_t dtype;     /* gqa_dtype */
  int32_t reserved;
  int64_t shape[4];
  int64_t stride[4];
} gqa_tensor;

/* Cache configuration ([P1] 2.1 cache_config, 2.5 layout_metadata).
 *  num_layers        layers; each has its own K/V and its own lengths.
 *  num_kv_heads      Hkv.   head_dim: d, 64 or 128 for bf16, 1..128 for f32.
 *  page_size         tokens per page; 16 is the only supported value.
 *  num_pages         physical pages in the pool (a page serves all layers).
 *                    For bf16 one layer of a pool (num_pages*Hkv*16*d*2
 *                    bytes) must stay below 4 GiB: the kernels address a
 *                    layer with 32-bit byte offsets (GQA_ERR_UNSUPPORTED).
 *  max_seqs          sequence ids are 0..max_seqs-1.
 *  max_pages_per_seq block-table width.
 *  dtype             storage dtype of the cache and of all Q/K/V/O tensors.
 *  rope_style        0: no position transform; 1: rotation pairing dimension
 *                    i with i + d/2 ([P3] RoPE paragraph; the pairing is this
 *                    library's convention).  Keys are cached AFTER rotation
 *                    ([P1] 2.5: the cache holds the keys used by attention).
 *  max_position      rotation table rows: positions 0..max_position-1.
 *  rope_theta        rotation base: pair i turns by p * theta^(-2i/d).
 *  window            sliding window W ([P3] sliding-window lesson: a query at
 *                    position t reads positions t-W+1..t, itself included);
 *                    0 = full causal attention.  W > 0 makes the cache a ring:
 *                    a sequence's block table holds at most max_pages_per_seq
 *                    entries and logical page L lives in entry L mod
 *                    max_pages_per_seq, so once the ring is full each new
 *                    logical page overwrites, in place, the page of the one
 *                    max_pages_per_seq before it.  max_pages_per_seq must be at
 *                    least ceil(W/16) + 1 (GQA_ERR_UNSUPPORTED).  A call that
 *                    writes positions [c, c+n) needs [max(0, c-W+1), c+n) to
 *                    fit in max_pages_per_seq consecutive logical pages
 *                    (GQA_ERR_OUT_OF_PAGES: split a long prompt into chunks).
 *                    Ring sequences are truncated only to 0 or to at least
 *                    their length, and are not forked (GQA_ERR_UNSUPPORTED);
 *                    gqa_attention queries must have their whole window still
 *                    in the ring (GQA_ERR_POSITION).                        */
typedef struct gqa_cache_config {
  int32_t num_layers;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t page_size;
  int32_t num_pages;
  int32_t max_seqs;
  int32_t max_pages_per_seq;
  int32_t dtype;
  int32_t rope_style;
  int32_t max_position;
  double rope_theta;
  int32_t window;
} gqa_cache_config;

typedef struct gqa_cache gqa_cache;

/* Bytes of the four caller-owned device buffers for a configuration.
 *  k_pool   [num_layers][num_pages][Hkv][page_size][d]   (key rows per page)
 *  v_pool   [num_layers][num_pages][Hkv][d][page_size]   (values stored d-major
 *           inside a page, so a page of one head is V^T; logical content is the
 *           same as row-major V)
 *  page_table int32 [max_seqs][max_pages_per_seq]
 *  rope_table float32: the rotation rows, pairs (cos, sin) [max_position][d/2],
 *           then the same values chunk-major, [d/4][max_position][4] (16-byte
 *           chunk j of row p at [j][p]); 2 * max_position * d * 4 bytes
 *           (0 if rope_style 0) */
gqa_status gqa_cache_buffer_sizes(const gqa_cache_config* cfg, size_t* k_pool_bytes,
                                  size_t* v_pool_bytes, size_t* page_table_bytes,
                                  size_t* rope_table_bytes);

/* Create the host-side state of a cache over caller-owned device buffers
 * ([P1] 2.5 LayerCache: per layer the used K and V with the lengths and
 * layout metadata that locate each sequence's slots; [P3] PagedAttention
 * lesson: a pool of fixed-size blocks, a per-request block table and free
 * blocks handed out on demand).  free_list_order: NULL for 0..num_pages-1, else a permutation of the pool that
 * fixes the order in which free pages are handed out.  Page contents are not
 * touched (fresh pages may hold anything; nothing beyond a sequence's length
 * is ever used).  The rotation table is computed on the host here and copied to
 * rope_table on the stream of the first call that launches work.
 * No HIP call is made by this function. */
gqa_status gqa_cache_create(const gqa_cache_config* cfg, void* k_pool, void* v_pool,
                            int32_t* page_table, void* rope_table,
                            const int32_t* free_list_order, gqa_cache** out);
/* Release the host-side state ([P1] 2.5 LayerCache).  The device buffers stay
 * the caller's; no HIP call is made.  NULL is accepted. */
gqa_status gqa_cache_destroy(gqa_cache* cache);

/* Append the valid tokens of K and V to layer `layer` of sequences seq_ids[0..B)
 * ([P1] 2.6 cache.write_sequence; [P3] decode append, one K/V per token).
 *  valid_mask  host uint8 [B][n], 1 = valid token, 0 = padding ([P1] 2.2:
 *              G in {0,1}); padding may sit before, after or between the valid
 *              tokens of a row.  GQA_ERR_MASK for any other value.
 *  positions   host int32 [B][n]; for the valid tokens, in row order, they
 *              must be c_b, c_b+1, ... where c_b is the layer's current length
 *              for that sequence (slot = position).  Padding entries are ignored.
 * Keys are rotated (rope_style 1) in float32 and rounded to the cache dtype,
 * values are copied bit-exactly.  Pages are taken from the free list when a
 * layer first needs them: in batch order, then logical page order.
 * B == 0 or n == 0 is a no-op. */
gqa_status kv_cache_append(gqa_cache* cache, int32_t layer, int32_t B, const int32_t* seq_ids,
                           const gqa_tensor* K, const gqa_tensor* V, const uint8_t* valid_mask,
                           const int32_t* positions, void* stream);

/* Prefill attention ([P1] 2.2-2.3, 2.6): kv_cache_append of K and V, then for
 * every valid query token at position p and head h, with g = floor(h*Hkv/Hq),
 *   O[b,h,i] = sum_{j<=p} softmax_j( <rot(q), k_used[g,j]> / sqrt(d) ) v[g,j]
 * over the cache slots of the sequence.  With a non-empty cache this is the
 * incremental (suffix) prefill of [P3]: the old prefix is fully visible.
 * Rows of O for padding tokens are written as 0.  Q and O are [B,Hq,n,d] in the
 * cache dtype; accumulation is float32.
 * workspace may be NULL (ws_bytes 0): the query tiles then run on the tiled
 * kernel.  For a bf16 cache and 1 <= n <= GQA_MAX_CHUNK_TOKENS, a non-NULL
 * workspace sends the attention to the split-T kernel instead, unless a row's
 * valid tokens have padding between them (the decode
 * kernel with one matrix column per (query token, head), split over the cached
 * keys, which suits short chunks on long caches); it must then follow the
 * gqa_decode workspace rule with gqa_attention_workspace_size(cache, B, Hq, n)
 * bytes.  Both kernels meet the same accuracy; their roundings differ. */
gqa_status gqa_prefill(gqa_cache* cache, int32_t layer, int32_t B, const int32_t* seq_ids,
                       const gqa_tensor* Q, const gqa_tensor* K, const gqa_tensor* V,
                       const uint8_t* valid_mask, const int32_t* positions, const gqa_tensor* O,
                       void* workspace, size_t ws_bytes, void* stream);

/* The attention half of gqa_prefill ([P1] 2.6 separates cache.write_sequence
 * from causal_attention): for every valid query token, whose K/V must already
 * be in the cache, at position p, O[b,h,i] attends to slots 0..p of layer
 * `layer`.  The valid tokens of a row (padding may sit between them) must
 * carry consecutive positions p0, p0+1, ... in row order that end at or before
 * the layer's current length; rows of O for padding tokens are written as 0.  gqa_prefill is kv_cache_append
 * followed by this call with p0 = the length before the append.  Same
 * workspace rule as gqa_prefill. */
gqa_status gqa_attention(gqa_cache* cache, int32_t layer, int32_t B, const int32_t* seq_ids,
                         const gqa_tensor* Q, const uint8_t* valid_mask, const int32_t* positions,
                         const gqa_tensor* O, void* workspace, size_t ws_bytes, void* stream);

/* Decode attention ([P2] decode shapes; [P3] single-token decode needs no mask):
 * one query per sequence at position T_b - 1 against all T_b cached slots of
 * layer `layer`.  valid_lengths (host int32 [B]) must equal each sequence's
 * current length in that layer (append the new token's K/V first) and be >= 1.
 * q and o are [B,Hq,1,d].  workspace: device scratch for split partials and
 * ready flags, at least gqa_workspace_size(cache, B, Hq) bytes, 256-byte
 * aligned and ZERO-FILLED before its first use (every call leaves its flags at
 * zero again, so one zeroed workspace serves any number of ordered calls of any
 * B, Hq or chunk length, provided every call passes the same ws_bytes: its
 * layout depends only on ws_bytes and d).  Calls that share a workspace must
 * not overlap in time.  It may be NULL when every sequence fits one split
 * (short caches).  GQA_ERR_ARG if it is needed and missing, misaligned or too
 * small.  The splits of a sequence are combined inside the launch; a combine
 * that waits too long for a split (it never should) writes NaN to its outputs
 * and sets the workspace's sticky status word, which gqa_workspace_status
 * turns into GQA_ERR_DEVICE. */
gqa_status gqa_decode(gqa_cache* cache, int32_t layer, int32_t B, const int32_t* seq_ids,
                      const gqa_tensor* q, const int32_t* valid_lengths, const gqa_tensor* o,
                      void* workspace, size_t ws_bytes, void* stream);

/* One decode step in one launch: kv_cache_append of the new token (k_new,
 * v_new [B,Hkv,1,d], position = the layer's current length c_b, rotated with
 * that position) followed by gqa_decode with T_b = c_b + 1 ([P3] decode
 * lessons: each step appends one K/V per layer, then the new query reads all T
 * entries).  Same results, cache contents and page assignment as the two calls;
 * bf16 caches do both in a single kernel.  Same workspace rule as gqa_decode. */
gqa_status gqa_decode_step(gqa_cache* cache, int32_t layer, int32_t B, const int32_t* seq_ids,
                           const gqa_tensor* q, const gqa_tensor* k_new, const gqa_tensor* v_new,
                           const gqa_tensor* o, void* workspace, size_t ws_bytes, void* stream);

/* gqa_decode_step without a workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  Same arguments, results, cache contents and page
 * assignment as gqa_decode_step; the split partials, ready flags and status
 * word live in the library's static scratch instead: a 48 MiB device array
 * that each GPU the library runs on holds until the process ends, set up on
 * the first call on each device (with that device current) and reused by
 * every later call there.  No device memory is allocated and no memset is
 * recorded (the first call zero-fills the flags with a kernel on `stream`).
 * Calls on one device share the scratch: calls that overlap in time (two
 * streams, two threads) race and must be ordered by the caller.  A call whose
 * split records would not fit (GQA_ERR_UNSUPPORTED, nothing changed) needs
 * gqa_decode_step with a workspace; at Hkv = 8 and d = 128 every call of up to
 * 64 sequences fits.  gqa_workspace_status(cache, NULL, 0, ...) reads and
 * clears the scratch's status word on the current device. */
gqa_status gqa_decode_step_noalloc(gqa_cache* cache, int32_t layer, int32_t B, const int32_t* seq_ids,
                                   const gqa_tensor* q, const gqa_tensor* k_new, const gqa_tensor* v_new,
                                   const gqa_tensor* o, void* stream);

/* Prompt edit at position m ([P3] prompt-edit lesson): keep positions [0,m) in
 * every layer of seq_id, drop the rest and give up the sequence's references to
 * the pages no layer still uses; a page whose last reference goes returns to
 * the back of the free list (ascending logical order).  Host only; no launch.
 * m beyond a layer's length leaves that layer unchanged.  m == 0 releases the
 * sequence. */
gqa_status kv_cache_truncate(gqa_cache* cache, int32_t seq_id, int32_t m);

/* Prefix sharing ([P3] prefix-sharing lesson: requests whose first m tokens
 * agree have the same per-layer K/V there, so a second request references the
 * cached blocks instead of prefilling them again).  Sequence dst, which must
 * be empty (length 0 in every layer), takes src's positions [0, m) in every
 * layer: its first ceil(m/16) block-table entries become src's pages, each
 * counting one more reference.  Nothing is copied.  Later, a write into a page
 * that more than one table references (the page holding slot m when m is not a
 * multiple of 16, or any page after a truncate inside it) first copies that
 * page, every layer, to a page from the front of the free list, and the
 * writer's entry points at the copy (copy-on-write for a fork inside a block);
 * the copy runs on the stream of the writing call.  A shared page returns to
 * the free list only when its last reference goes (truncate).  Host only; no
 * launch.  Errors: GQA_ERR_ARG (ids out of range, src == dst, m < 0),
 * GQA_ERR_CACHE (dst not empty), GQA_ERR_POSITION (m beyond src's length in
 * some layer). */
gqa_status kv_cache_fork(gqa_cache* cache, int32_t src_seq, int32_t dst_seq, int32_t m);

/* Prefix index ([P3] prefix-sharing lesson: a cached prefix is reusable only
 * on an exact token-id match, and two requests that first differ at index m
 * share positions 0..m-1; a prefix tree over the requests answers which prefix
 * is reusable, the block tables where it lives).  A host-only radix tree over
 * the token ids the caller records per request; it never touches the cache:
 * the caller keeps it in step with the cache (insert after a prefill, remove
 * or re-insert after a truncate) and shares the match with kv_cache_fork.
 * Not thread-safe; no HIP call. */
typedef struct gqa_prefix_index gqa_prefix_index;
gqa_status gqa_prefix_index_create(gqa_prefix_index** out);
gqa_status gqa_prefix_index_destroy(gqa_prefix_index* index);
/* Record that request seq (>= 0) holds the cache of tokens[0..n) (host int32),
 * replacing what seq held before.  GQA_ERR_ARG on a null index or tokens,
 * seq < 0 or n < 0. */
gqa_status gqa_prefix_index_insert(gqa_prefix_index* index, int32_t seq, const int32_t* tokens, int32_t n);
/* Forget request seq (no-op if it is not recorded). */
gqa_status gqa_prefix_index_remove(gqa_prefix_index* index, int32_t seq);
/* Longest common prefix of tokens[0..n) with any recorded request: *m_out its
 * length and *seq_out the smallest request id that reaches it, or -1 (and
 * *m_out 0) when no recorded request shares even the first token. */
gqa_status gqa_prefix_index_match(const gqa_prefix_index* index, const int32_t* tokens, int32_t n,
                                  int32_t* seq_out, int32_t* m_out);

/* Move n physical pages ([P1] 2.2: the manager may move physical pages but not
 * change which tokens they hold).  src_pages (host) must be in use, dst_pages
 * (host) free and all distinct.  Copies every layer's K and V of each page on
 * `stream`, rewrites every block-table entry that references a moved page (a
 * shared page has several) and returns the source pages to the back of the
 * free list in the order given. */
gqa_status kv_cache_remap(gqa_cache* cache, int32_t n, const int32_t* src_pages,
                          const int32_t* dst_pages, void* stream);

/* Host-side queries, no HIP call.
 * gqa_cache_length: the written length of (seq_id, layer), i.e. the number of
 *   slots [0, length) holding that layer's used K/V ([P1] 2.5: the cache
 *   length equals the next position to write).  GQA_ERR_ARG for a null
 *   argument or an id out of range.
 * gqa_cache_page_table: the sequence's block table ([P3] PagedAttention
 *   lesson: logical block t/16 of the sequence lives in physical page out[t/16];
 *   in a ring, logical page L in entry L mod max_pages_per_seq).  *n_out gets
 *   the number of entries; they are copied to the host array out[0..cap) when
 *   they fit (GQA_ERR_ARG otherwise, with *n_out still set; out may be NULL
 *   when the table is empty).
 * gqa_cache_free_pages: pages on the free list. */
gqa_status gqa_cache_length(const gqa_cache* cache, int32_t seq_id, int32_t layer, int32_t* out);
gqa_status gqa_cache_page_table(const gqa_cache* cache, int32_t seq_id, int32_t* out, int32_t cap,
                                int32_t* n_out);
gqa_status gqa_cache_free_pages(const gqa_cache* cache, int32_t* out);
/* Cache invariants ([P1] 2.5, invariants 2.2): every layer of a sequence has the
 * same length, a sequence's table holds exactly ceil(length/page_size) distinct
 * pages, every page's reference count equals the table entries that name it,
 * and every page is either referenced or listed once in the free list.
 * GQA_ERR_CACHE if not. */
gqa_status gqa_cache_check(const gqa_cache* cache);

/* Device workspace bytes that suffice for gqa_decode / gqa_decode_step with up
 * to B sequences and Hq query heads, whatever their lengths (zero-fill it once
 * before first use).  0 for a null cache, B < 0 or Hq < 1. */
size_t gqa_workspace_size(const gqa_cache* cache, int32_t B, int32_t Hq);

/* Device workspace bytes that suffice for a split-T gqa_prefill / gqa_attention
 * call with up to B sequences, Hq query heads and n rectangular rows, whatever
 * the lengths.  0 when that call would not take the split-T kernel (f32 cache,
 * n < 1 or n > GQA_MAX_CHUNK_TOKENS) or for invalid arguments.  A workspace of
 * this size also serves gqa_decode for the same B and Hq. */
size_t gqa_attention_workspace_size(const gqa_cache* cache, int32_t B, int32_t Hq, int32_t n);

/* Sticky failure status of a split-T workspace.  Waits for the work queued on
 * `stream`, then reads the status word that a split combine sets when it gives
 * up waiting for a split (its outputs then hold NaN instead of a result).
 * Returns GQA_OK if no combine has given up since the word was last cleared,
 * GQA_ERR_DEVICE if one has.  With clear != 0 the word and every ready flag
 * are zeroed afterwards (on `stream`, waited for), which makes the workspace
 * as good as freshly zero-filled: do this after GQA_ERR_DEVICE before reusing
 * it.  workspace NULL with ws_bytes 0 means the static scratch of
 * gqa_decode_step_noalloc on the current device.  GQA_ERR_ARG for a null
 * cache or a workspace too small for one slot; GQA_ERR_HIP if the read fails.
 * Synchronises: not for use under capture. */
gqa_status gqa_workspace_status(const gqa_cache* cache, void* workspace, size_t ws_bytes, int32_t clear,
                                void* stream);

/* Test control of the split combine's bounded wait (process-wide, for tests of
 * the failure report above).  polls: how many times a combine polls one ready
 * flag before it gives up (default 262144, about 0.1 s); unreachable != 0
 * makes combines wait for a flag value no split writes, so every split-T
 * launch that needs a combine gives up after `polls` polls and reports it,
 * while every workgroup still exits.  gqa_set_merge_wait(262144, 0) restores
 * the default.  GQA_ERR_ARG if polls < 0.  Host only. */
gqa_status gqa_set_merge_wait(int32_t polls, int32_t unreachable);

/* Message of the last failed call on this thread ("" if none). */
const char* gqa_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* GQA_H */
