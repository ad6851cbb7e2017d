/*
 * inferscale.h -- C ABI of the retrieve-and-inject hot path on MI355X (gfx950).
 *
 * The operations follow "InferScale: GPU-Native KV Injection for
 * Personalized LLM Serving" (gist.science explainer pages, technical
 * summary):
 *   - the fact store holds, per fact, the keys captured before RoPE and the
 *     raw values ("Online phase", pre-RoPE storage), here laid out
 *     [fact][layer][kv_head][token][head_dim];
 *   - retrieval runs over a GPU-resident index ("Contributions", GPU-native
 *     system design); here an exact inner-product top-k over fp16 fact
 *     embeddings stands in for the pages' index;
 *   - the selected facts are composed into one contiguous segment, each
 *     stored key is re-rotated to its new serving position ("Online phase",
 *     dynamic rotation, Theorem 6) and the K/V are scatter-copied into the
 *     serving engine's paged KV cache ("Online phase", injection);
 *   - a store larger than GPU memory keeps part of its facts in host memory
 *     ("Results", scalability: offload of the KV store to host DRAM).
 * Readings where the pages are silent: textbook RoPE with frequencies
 * theta^(-2i/d), rotate-half pairing (i, i + d/2), optional Llama-3.1
 * frequency scaling; facts back to back in the caller's order right after
 * the request's prefix; RoPE uses the logical position, not the slot.
 *
 * Conventions for every call:
 *   - returns IS_OK (0) or a negative is_status; is_last_error() describes
 *     the last failure of the calling thread;
 *   - "host" pointers are read during the call only; "device" pointers must
 *     stay valid until the work enqueued on `stream` has completed;
 *   - `stream` is a hipStream_t (NULL = the default stream);
 *   - validation completes before anything is enqueued: on error nothing
 *     is written anywhere (all or nothing);
 *   - thread safety: each store has a lock that every call taking the
 *     store holds while it reads or changes the store's tables, so calls
 *     from several host threads are safe; the device work of a call is
 *     ordered only on its own stream, so work that changes a store
 *     (append, update) must be ordered by the caller against work on other
 *     streams that reads the same facts.
 */
#ifndef INFERSCALE_H
#define INFERSCALE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  IS_OK = 0,
  IS_ERR_INVALID_ARG = -1,  /* null pointer, bad size or count           */
  IS_ERR_FACT_ID = -2,      /* fact id outside [0, n_facts)              */
  IS_ERR_BLOCK_TABLE = -3,  /* block table too short or entry out of range */
  IS_ERR_SLOT_OVERLAP = -4, /* two injected tokens map to one cache slot */
  IS_ERR_DTYPE = -5,        /* cache dtype differs from the store's      */
  IS_ERR_ALIGN = -6,        /* pointer or stride breaks 16-byte rows     */
  IS_ERR_OOM = -7,          /* device or pinned-host allocation failed   */
  IS_ERR_HIP = -8,          /* a HIP runtime call failed                 */
  IS_ERR_UNSUPPORTED = -9   /* valid, but outside what the kernels cover */
} is_status;

typedef enum { IS_DTYPE_F32 = 0, IS_DTYPE_BF16 = 1 } is_dtype;

typedef enum { IS_ROPE_NONE = 0, IS_ROPE_LLAMA3 = 1 } is_rope_scaling;

typedef struct is_store is_store;

/*
 * Store description (all host memory, read during is_store_create only).
 *   n_layers, n_kv_heads, head_dim   K/V geometry; head_dim * element size
 *                                    must be a multiple of 32 bytes (two
 *                                    16-byte halves); head_dim/2 split into
 *                                    16-byte chunks of 2, 4, 8, 16 or 32
 *                                    lanes (bf16: head_dim 32..512, fp32:
 *                                    16..256, powers of two)
 *   kv_dtype                         is_dtype of stored K/V (and the cache)
 *   n_facts, fact_len[n_facts]       number of facts and their token counts
 *                                    (each >= 1)
 *   emb_dim                          fp16 embedding width (multiple of 32),
 *                                    0 = the store has no index (no top-k)
 *   hbm_budget_bytes                 device bytes allowed for K+V; facts are
 *                                    placed in id order in HBM while they
 *                                    fit, the rest in pinned host memory;
 *                                    < 0 means no limit
 *   k_src, v_src                     optional host sources, every fact's
 *                                    [layer][kv_head][token][head_dim] block
 *                                    back to back in id order (NULL: leave
 *                                    uninitialised, fill with is_store_load)
 *   emb_src                          optional host [n_facts][emb_dim] fp16
 *   spare_facts, spare_tokens        room kept in HBM for facts added later
 *                                    by is_store_append (0: none); a store
 *                                    with a host tier takes no spare room
 */
typedef struct {
  int32_t n_layers;
  int32_t n_kv_heads;
  int32_t head_dim;
  int32_t kv_dtype;
  int64_t n_facts;
  const int32_t* fact_len;
  int32_t emb_dim;
  int32_t reserved0;
  int64_t hbm_budget_bytes;
  const void* k_src;
  const void* v_src;
  const uint16_t* emb_src;
  int64_t spare_facts;
  int64_t spare_tokens;
} is_store_desc;

/*
 * Paged KV cache owned by the caller (the serving engine), in device
 * memory.  Element (layer l, block b, slot s, kv_head h, dim i) of the K
 * cache is k_base[l*stride_layer + b*stride_block + s*stride_slot +
 * h*stride_head + i]; the same strides apply to v_base.  head_dim is
 * contiguous.  Strides are in elements; every row start must be 16-byte
 * aligned.  NHD layout [layer][block][slot][head][dim] and HND layout
 * [layer][block][head][slot][dim] are both expressible.
 */
typedef struct {
  void* k_base;
  void* v_base;
  int64_t stride_layer;
  int64_t stride_block;
  int64_t stride_slot;
  int64_t stride_head;
  int32_t block_size;
  int32_t dtype;
  int64_t n_blocks;
} is_cache;

/*
 * RoPE parameters: frequencies theta^(-2i/head_dim), i < head_dim/2, and,
 * for IS_ROPE_LLAMA3, the Llama-3.1 rule: wavelengths below
 * orig_max_pos/high_freq_factor are kept, above orig_max_pos/low_freq_factor
 * divided by `factor`, blended linearly in between.
 */
typedef struct {
  double theta;
  int32_t scaling;
  int32_t reserved0;
  double factor;
  double low_freq_factor;
  double high_freq_factor;
  double orig_max_pos;
} is_rope;

/* Placement summary of a store. */
typedef struct {
  int64_t n_facts;
  int64_t n_hbm_facts;       /* facts [0, n_hbm_facts) live in HBM         */
  int64_t hbm_kv_bytes;      /* device bytes of K+V                        */
  int64_t host_kv_bytes;     /* pinned host bytes of K+V                   */
  int64_t total_tokens;
  int64_t emb_bytes;
} is_store_info;

/*
 * (Online phase, pre-RoPE storage: every fact's keys captured before RoPE
 * and its raw values, held on the GPU; Results, scalability: the part that
 * does not fit in HBM is offloaded to host DRAM.)
 * Creates a store: allocates device memory for the facts that fit the HBM
 * budget (and pinned host memory for the rest) plus the fp16 embedding
 * matrix, and copies the optional sources.  The library owns the memory;
 * the caller may free its sources when the call returns.  Synchronous.
 * Errors: IS_ERR_INVALID_ARG (geometry, lengths), IS_ERR_UNSUPPORTED
 * (head_dim or emb_dim outside the kernels' shapes), IS_ERR_OOM.  Nothing
 * stays allocated on error; *out is set only on success.
 */
int is_store_create(const is_store_desc* desc, is_store** out);

/*
 * (Offline phase: the facts' encodings are computed ahead of serving and
 * written into the store.)
 * Fills facts [first_fact, first_fact + n_facts) from K/V sources laid out
 * like the store (those facts' blocks back to back) and, when emb is not
 * NULL, their embedding rows.  src_on_device = 1 means the sources are
 * device pointers.  Synchronous.  For stores larger than host memory the
 * caller loads in chunks.  k or v may be NULL to skip that tensor.
 * Errors: IS_ERR_INVALID_ARG (range), IS_ERR_HIP.
 */
int is_store_load(is_store* s, int64_t first_fact, int64_t n_facts,
                  const void* k, const void* v, const uint16_t* emb,
                  int src_on_device);

/* Placement summary (Results, scalability: HBM and host-DRAM tiers).
 * Errors: IS_ERR_INVALID_ARG. */
int is_store_get_info(const is_store* s, is_store_info* out);

/*
 * (Contributions, GPU-native system design: retrieval over an index that
 * stays on the GPU; the pages do not describe the index, and this exact
 * search stands in for it.)
 * Exact top-k inner-product search: for each query q (device
 * q_f16[n_q][emb_dim], fp16 bits) the k facts with the largest
 * <q, E[f]> (fp16 products, fp32 accumulation on the matrix cores), written
 * to device ids[n_q][k] (int32) and scores[n_q][k] (fp32) in order of score
 * descending, ties to the lower id.  Requires 1 <= k <= min(64, n_facts)
 * and an embedding index.  Asynchronous on `stream`.
 * Errors: IS_ERR_INVALID_ARG, IS_ERR_UNSUPPORTED (k > 64, no index),
 * IS_ERR_OOM, IS_ERR_HIP.
 */
int is_topk(const is_store* s, const uint16_t* q_f16, int32_t n_q, int32_t k,
            int32_t* ids, float* scores, void* stream);

/*
 * is_topk for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments, results (bit for bit) and errors as is_topk, but the
 * call allocates nothing: its scratch is one fixed 80 MiB array in device
 * memory per GPU, held from the first call on that GPU until the process
 * ends, instead of the store's scratch ring.  Limit: stores of at most
 * 65,536 facts (larger stores: IS_ERR_UNSUPPORTED, nothing enqueued).
 * Every call on one GPU uses the same array, whatever its store, so calls
 * that overlap on a GPU (other streams, other host threads) race: order
 * them.  No part of the array needs clearing between calls (each call
 * writes every element it reads before reading it).
 */
int is_topk_noalloc(const is_store* s, const uint16_t* q_f16, int32_t n_q, int32_t k,
                    int32_t* ids, float* scores, void* stream);

/*
 * (Online phase: the retrieved facts are composed into one contiguous
 * segment, every stored key gets the RoPE rotation of its new serving
 * position -- dynamic rotation, exact by Theorem 6 -- and the K/V are
 * scatter-copied into the engine's paged KV cache.)
 * Retrieve-and-inject for a batch of requests.
 *   req_off[n_req+1]   host; request r uses fact_ids[req_off[r]..req_off[r+1])
 *   fact_ids[]         host; facts in segment order (a repeat is allowed and
 *                      is injected twice)
 *   prefix_len[n_req]  host; tokens already in the cache before the segment
 *   block_tables       host [n_req][max_blocks]; physical block ids
 * Request r's facts occupy serving positions prefix_len[r] .. prefix_len[r]
 * + T_r - 1 back to back; the token at position p goes to slot
 * block_tables[r][p / block_size] * block_size + p % block_size.  Its
 * stored pre-RoPE key is rotated to position p (fp32 arithmetic, one
 * rounding to the cache dtype) and written with its raw value to that slot;
 * no other cache element is written.
 * Validation (all before any work is enqueued): ids in range, every block
 * table entry used in [0, n_blocks), block tables long enough, no two
 * injected tokens of the call share a slot, cache dtype equals the store's,
 * 16-byte row alignment, positions below 2^24.  Host arrays are copied
 * before return; the kernels run asynchronously on `stream`.
 * Errors: IS_ERR_INVALID_ARG, IS_ERR_FACT_ID, IS_ERR_BLOCK_TABLE,
 * IS_ERR_SLOT_OVERLAP, IS_ERR_DTYPE, IS_ERR_ALIGN, IS_ERR_OOM, IS_ERR_HIP.
 */
int is_inject(const is_store* s, int32_t n_req, const int32_t* req_off,
              const int32_t* fact_ids, const int32_t* prefix_len,
              const int32_t* block_tables, int32_t max_blocks,
              const is_cache* cache, const is_rope* rope, void* stream);

/*
 * Retrieve-and-inject without a host round trip: for each request r, the
 * top-k facts of its query (as is_topk), laid out in rank order as one
 * contiguous segment from serving position prefix_len[r] on and injected
 * as by is_inject -- composition, validation and injection all run on the
 * device, on `stream`, so the ids never travel to the host.  (Online phase:
 * retrieved facts composed into one segment and injected into the paged
 * cache.)
 *   q_f16[n_req][emb_dim]        device, fp16 bits, 16-byte aligned
 *   prefix_len[n_req]            device
 *   block_tables[n_req][max_blocks]  device; read by the kernels, so it must
 *                                stay valid until the stream has completed
 *   ids_out[n_req][k]            device, optional (NULL): the selected ids
 *   status                       device int32, written on the stream:
 *                                IS_OK, or the smallest (most negative) code
 *                                among the failed checks -- IS_ERR_FACT_ID,
 *                                IS_ERR_BLOCK_TABLE (table too short or an
 *                                entry outside [0, n_blocks)),
 *                                IS_ERR_SLOT_OVERLAP (two injected tokens of
 *                                the call share a slot), IS_ERR_INVALID_ARG
 *                                (negative prefix, positions reaching 2^24).
 *                                When it is not IS_OK no cache element is
 *                                written.
 * Returns before the work completes; host-side checks (store, k, cache
 * geometry and alignment, rope, pointers) fail with the return code and
 * enqueue nothing.  Requires 1 <= k <= min(64, n_facts), an embedding
 * index, and a cache of at most 2^32 slots (the slot check keeps a
 * bitmap of slots / 8 bytes).
 * HIP graph capture: the call only launches kernels, so it may be captured
 * on `stream` and the graph replayed (new query contents in the same
 * buffers give new retrievals).  Captured calls use one scratch workspace
 * per store, sized by the eager calls until the first capture and fixed
 * from then on: capture after an eager call of at least the same n_req, k
 * and cache (else IS_ERR_UNSUPPORTED, nothing captured).  Replays of
 * graphs captured on one store share that workspace, so they must be
 * ordered among themselves (one stream, or synchronized); eager calls use
 * other scratch and may interleave.  A graph searches the facts the store
 * held at capture (facts appended later are not searched; facts updated
 * in place are read as updated); once a graph has been captured,
 * is_store_remove refuses (it would free the index the graph reads).
 * Errors: IS_ERR_INVALID_ARG, IS_ERR_UNSUPPORTED, IS_ERR_DTYPE,
 * IS_ERR_ALIGN, IS_ERR_OOM, IS_ERR_HIP.
 */
int is_retrieve_inject(const is_store* s, const uint16_t* q_f16, int32_t n_req, int32_t k,
                       const int32_t* prefix_len, const int32_t* block_tables,
                       int32_t max_blocks, const is_cache* cache, const is_rope* rope,
                       int32_t* ids_out, int32_t* status, void* stream);

/*
 * Adds n facts from their context-window encodings (Offline phase: a fact
 * is encoded behind a window of preceding tokens, and only the fact's own
 * tokens' pre-RoPE keys and raw values are stored).
 *   fact_len[n]        host, each >= 1
 *   window             tokens encoded before each fact (>= 0)
 *   k_enc, v_enc       device, the n encodings back to back, fact i as
 *                      [layer][kv_head][window + fact_len[i]][head_dim]
 *                      (16-byte aligned); only rows window .. window +
 *                      fact_len[i] - 1 of each (layer, kv_head) are stored,
 *                      bit for bit
 *   emb                device [n][emb_dim] fp16 (required when the store
 *                      has an index, else NULL)
 *   first_id           host out: the id of the first new fact (ids are
 *                      consecutive)
 * The new facts go to HBM, into the spare room reserved at creation or the
 * room that removed facts left (first fit).  Asynchronous on `stream`: calls that use the new facts must be ordered
 * after it on the device (same stream, or synchronized).  The sources must
 * stay valid until the stream has completed.
 * Errors: IS_ERR_INVALID_ARG, IS_ERR_ALIGN, IS_ERR_OOM (no spare room),
 * IS_ERR_UNSUPPORTED (the store has a host tier), IS_ERR_HIP.
 */
int is_store_append(is_store* s, int32_t n, const int32_t* fact_len, int32_t window,
                    const void* k_enc, const void* v_enc, const uint16_t* emb,
                    int64_t* first_id, void* stream);

/*
 * Replaces the stored K/V (and, when emb is not NULL, the embedding row) of
 * fact `fact_id` from a new window encoding of the same length
 * ([layer][kv_head][window + len][head_dim], device, 16-byte aligned) --
 * a fact update; host-tier facts are rewritten in place over PCIe.
 * Asynchronous on `stream`; the caller orders it against calls that read
 * the fact.  Errors: IS_ERR_INVALID_ARG, IS_ERR_FACT_ID, IS_ERR_ALIGN,
 * IS_ERR_HIP.
 */
int is_store_update(is_store* s, int64_t fact_id, int32_t window, const void* k_enc,
                    const void* v_enc, const uint16_t* emb, void* stream);

/*
 * Evicts facts from the store.  A personal memory store drops facts as
 * well as gaining them; the pages define the store only by what it holds
 * (Offline phase), so removal is the plain one: the listed facts leave the
 * store, the others keep their order and are renumbered densely -- a
 * fact's new id is its old id minus the number of removed ids below it.
 *   ids[n]   host int32, distinct, each in [0, n_facts); n = 0 is a no-op
 * The surviving facts' K/V stay where they are (their addresses move in the
 * fact tables only); the removed facts' HBM spans are reused by later
 * appends; the embedding index is compacted into a fresh arena.
 * Synchronous: returns when the work queued on `stream` has completed.
 * Must not overlap any other call that uses the store.
 * Errors: IS_ERR_INVALID_ARG (null, an id listed twice), IS_ERR_FACT_ID,
 * IS_ERR_UNSUPPORTED (the store has a host tier, or a HIP graph was
 * captured on it), IS_ERR_OOM, IS_ERR_HIP;
 * nothing changes on error.
 */
int is_store_remove(is_store* s, int64_t n, const int32_t* ids, void* stream);

/*
 * Query-only attention over the paged cache, the step that follows the
 * injection (Online phase: the engine prefills only the query over the
 * cache holding the injected facts; Theorem 6).  For every layer l of the
 * store's geometry, request r, query token t at position q_pos[r] + t and
 * query head hq (kv head hq / g, g = n_q_heads / n_kv_heads):
 *   out = sum_p softmax_p(<R(q_pos[r] + t) q, K_l[slot_r(p)][hq / g]> / sqrt(d))
 *               * V_l[slot_r(p)][hq / g],  p in [ctx_begin[r], ctx_end[r])
 * with slot_r(p) = block_tables[r][p / block_size] * block_size
 * + p % block_size; an empty context gives zeros.
 *   q     device [n_layers][n_req][n_qtok][n_q_heads][head_dim] in the store's
 *         dtype (bf16 bits or fp32), before RoPE (rotated here in fp32),
 *         16-byte aligned
 *   out   device fp32, same shape, 16-byte aligned
 *   q_pos, ctx_begin, ctx_end   host [n_req]
 *   block_tables                host [n_req][max_blocks]
 * bf16 stores with head_dim 128 run on the matrix cores, the fp32 operands
 * (rotated query, probabilities) split into two bf16 parts, accumulation in
 * fp32; other head dims (even, at most 256) and fp32 stores run a plain
 * fp32 kernel (one wave per query row), a parity path for small shapes.
 * Validation before any work: positions in [0, 2^24), 0 <= begin <= end,
 * block tables cover every context position with entries in [0, n_blocks).
 * Host arrays are copied before return; the kernel runs on `stream`.
 * Errors: IS_ERR_INVALID_ARG, IS_ERR_BLOCK_TABLE, IS_ERR_DTYPE, IS_ERR_ALIGN,
 * IS_ERR_UNSUPPORTED (head_dim above 256), IS_ERR_OOM, IS_ERR_HIP.
 */
int is_attend(const is_store* s, const is_cache* cache, const is_rope* rope, int32_t n_req,
              int32_t n_qtok, int32_t n_q_heads, const void* q, const int32_t* q_pos,
              const int32_t* ctx_begin, const int32_t* ctx_end, const int32_t* block_tables,
              int32_t max_blocks, float* out, void* stream);

/*
 * (Online phase: composition of the retrieved facts into one segment after
 * the prefix, as for is_inject.)
 * The host half of is_inject on its own: validation and composition
 * against a store description (no store, no GPU).  Returns the status
 * is_inject would return for the same arguments before any device work,
 * and the number of tokens that would be injected in *n_tokens (may be
 * NULL).  The cache pointers are checked for alignment only.
 */
int is_inject_check(const is_store_desc* desc, int32_t n_req,
                    const int32_t* req_off, const int32_t* fact_ids,
                    const int32_t* prefix_len, const int32_t* block_tables,
                    int32_t max_blocks, const is_cache* cache,
                    const is_rope* rope, int64_t* n_tokens);

/*
 * (Offline phase: the store lives across serving; this ends its life.)
 * Frees the store's device and host memory.  The caller must have
 * completed all streams that use it.  NULL is a no-op.
 */
int is_store_destroy(is_store* s);

/* Description of the calling thread's last error (empty if none); a
 * library convention, no passage of the pages. */
const char* is_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* INFERSCALE_H */
