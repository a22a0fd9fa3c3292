/*
 * verify_step -- one batched, paged decode / speculative-verify step of a
 * Llama-style decoder on an AMD Instinct MI355X (gfx950).
 *
 * C ABI. Plain pointers and sizes only. Device pointers are HIP device
 * addresses on the current device; host pointers are ordinary process memory.
 * Every call returns a vs_status; on failure vs_last_error() gives a message
 * (thread-local, valid until the next call on the same thread). No C++
 * exception crosses this interface.
 *
 * Sources (page titles; section numbers as printed on each page):
 *   [Serving Efficiency] "Chapter 31 Serving Efficiency: Reuse, Kernels,
 *                        Speculation, and Batching"
 *   [Spending the Idle]  "Spending the Idle"
 *   [Serving]            "Serving"
 *   [KV Cache]           "Inference at Scale: KV Cache, Prefill, and Decode"
 *
 * Ownership. The caller owns every device buffer: the KV pool's memory, the
 * weights, the batch arrays, the outputs and the workspace. The library owns
 * only host-side pool metadata. Nothing on the step path allocates device
 * memory, synchronises the device, or issues a memset, so decode_step,
 * verify_accept and verify_sample may be captured into a HIP graph.
 *
 * Asynchrony. decode_step, verify_accept, verify_sample and the copy that kv_append may
 * enqueue are asynchronous on the stream passed in; their inputs must stay
 * valid until the stream reaches them. Argument errors are reported before
 * anything is enqueued. A device fault surfaces as VS_ERR_HIP at a later
 * checked call. The pool calls are not thread-safe (one scheduler thread).
 */
#ifndef VERIFY_STEP_H
#define VERIFY_STEP_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t vs_status;
#define VS_OK 0
#define VS_ERR_INVALID (-1) /* bad argument, or a pool operation that would break its invariants */
#define VS_ERR_OOM (-2)     /* the pool has too few free pages; state unchanged */
#define VS_ERR_SHAPE (-3)   /* sizes the kernels do not support, or a workspace that is too small */
#define VS_ERR_HIP (-4)     /* a HIP runtime call failed */

/* Message for the last failing call on this thread ("" if none). */
const char* vs_last_error(void);

/* Storage type of weights and KV cache. Arithmetic is fp32 throughout. */
#define VS_F32 0
#define VS_F16 1
#define VS_BF16 2
/* KV cache only: OCP 8-bit floats, one byte per value ([KV Cache] section 03:
 * an FP8 cache in the e4m3 or e5m2 format halves the K/V bytes). K and V are
 * rounded once from their rotated fp32 values, to nearest with ties to even,
 * saturating at the largest finite magnitude (448 for e4m3, 57344 for e5m2). */
#define VS_FP8_E4M3 3
#define VS_FP8_E5M2 4

/* ------------------------------------------------------------------ model */

/* A pre-norm decoder layer stack ([KV Cache] section 03: the 7B shape is
 * Llama 2 7B's, multi-head attention with as many KV heads as query heads):
 * RMSNorm, rotary q/k, causal softmax attention scaled by 1/sqrt(head_dim),
 * output projection + residual, RMSNorm, SwiGLU MLP + residual; final RMSNorm
 * and an untied LM head. */
typedef struct vs_model_desc {
    int32_t d_model;    /* = n_heads * head_dim */
    int32_t n_heads;
    int32_t n_kv_heads; /* divides n_heads (equal for multi-head attention) */
    int32_t head_dim;   /* 64 or 128 */
    int32_t ffn;        /* MLP hidden width */
    int32_t vocab;
    int32_t n_layers;
    int32_t dtype;      /* VS_F32, VS_F16 or VS_BF16 */
    float rope_theta;   /* rotary base, e.g. 10000 */
    float eps;          /* RMSNorm epsilon, e.g. 1e-5 */
} vs_model_desc;

/* Device pointers to one layer's weights, all in the model dtype. Matrices are
 * row-major [out][in] (a product reads row n to make output feature n). */
typedef struct vs_layer_weights {
    const void* attn_norm; /* [d_model] */
    const void* wq;        /* [n_heads*head_dim][d_model] */
    const void* wk;        /* [n_kv_heads*head_dim][d_model] */
    const void* wv;        /* [n_kv_heads*head_dim][d_model] */
    const void* wo;        /* [d_model][n_heads*head_dim] */
    const void* ffn_norm;  /* [d_model] */
    const void* wg;        /* [ffn][d_model] gate */
    const void* wu;        /* [ffn][d_model] up */
    const void* wd;        /* [d_model][ffn] down */
} vs_layer_weights;

typedef struct vs_weights {
    vs_model_desc dims;
    const void* embed;              /* device [vocab][d_model] */
    const void* final_norm;         /* device [d_model] */
    const void* lm_head;            /* device [vocab][d_model] */
    const vs_layer_weights* layers; /* HOST array of n_layers entries (device pointers inside) */
} vs_weights;

/* ------------------------------------------------------------------ KV pool */

/* Paged KV cache ([KV Cache] section 05 "The block table"): fixed blocks of
 * page_tokens token slots; a per-sequence block table maps logical block i
 * (positions [16i, 16i+16)) to a physical page anywhere in the pool.
 *
 * Page layout in device memory (one page holds every layer):
 *   page p, layer l, K (0) or V (1), KV head h, slot s, dim e at element
 *   ((((p*n_layers + l)*2 + kv)*n_kv_heads + h)*page_tokens + s)*head_dim + e
 * so one (page, layer, K|V, head) block of page_tokens*head_dim values is
 * contiguous (4 KiB for 16 x 128 fp16, 2 KiB in an 8-bit cache). */
typedef struct vs_pool_desc {
    int32_t num_pages;
    int32_t page_tokens; /* 16 */
    int32_t n_layers;
    int32_t n_kv_heads;
    int32_t head_dim;
    int32_t dtype; /* VS_F32, VS_F16, VS_BF16: the model's dtype; or VS_FP8_E4M3 / VS_FP8_E5M2 with
                      an fp16 or bf16 model whose head_dim is 128 */
} vs_pool_desc;

typedef struct vs_pool vs_pool;

/* Bytes of one page for this geometry. */
size_t kv_page_bytes(const vs_pool_desc* desc);

/* Create a pool over caller-owned device memory of at least
 * num_pages * kv_page_bytes bytes (the region left after the weights,
 * [KV Cache] section 03 "The memory budget of a GPU"). Every page starts free.
 * kv_pool_destroy frees the host metadata only. */
vs_status kv_pool_create(const vs_pool_desc* desc, void* dev_base, size_t dev_bytes, vs_pool** out);
void kv_pool_destroy(vs_pool* pool);

/* Take n free pages, all or nothing; each gets reference count 1. Writes the
 * page ids to out_ids (host, n entries). VS_ERR_OOM leaves the pool unchanged. */
vs_status kv_alloc(vs_pool* pool, int32_t n, int32_t* out_ids);

/* Add one reference to each listed page (a fork, or a prefix shared between
 * requests: [KV Cache] section 05 "Block sharing and copy-on-write").
 * Every page must be in use; otherwise VS_ERR_INVALID and nothing changes. */
vs_status kv_share(vs_pool* pool, const int32_t* ids, int32_t n);

/* Drop one reference from each listed page (a page listed twice loses two);
 * a page returns to the free list at zero. Dropping a reference that does not
 * exist is VS_ERR_INVALID and nothing changes. */
vs_status kv_free(vs_pool* pool, const int32_t* ids, int32_t n);

/* Make room for positions [cur_len, cur_len + n_new) of one sequence.
 * bt_row (host, capacity max_blocks) holds *n_blocks page ids, which must equal
 * ceil(cur_len / page_tokens). A new page is taken only when the last one is
 * full ([KV Cache] section 05). If the last page is partly filled and shared
 * (reference count > 1), the sequence first gets a private copy of it:
 * a fresh page is taken, one page-sized device copy is enqueued on `stream`,
 * the shared page loses this sequence's reference and bt_row is rewritten
 * (copy-on-write at block granularity, [KV Cache] section 05; [Serving
 * Efficiency] section 31.3). All or nothing: VS_ERR_OOM leaves everything
 * unchanged. *n_blocks is updated on success. */
vs_status kv_append(vs_pool* pool, int32_t* bt_row, int32_t* n_blocks, int32_t max_blocks, int32_t cur_len,
                    int32_t n_new, hipStream_t stream);

int32_t kv_num_free(const vs_pool* pool);
int32_t kv_refcount(const vs_pool* pool, int32_t page); /* -1 for an out-of-range id */
/* Device address of the pool memory and the page geometry, for filling pages. */
void* kv_pool_base(const vs_pool* pool);

/* ------------------------------------------------------------------ prefix cache */

/* Prefix caching ([KV Cache] section 05 "Prefix caching"; [Serving Efficiency]
 * section 31.3): a full block is named by a hash of its own tokens and of the
 * block before it, so the name covers the whole prefix up to it; a new
 * sequence that finds the names of its leading blocks takes those pages
 * instead of recomputing their K/V. The chain starts at a root that names the
 * computation version (model and weights, adapters, positional conventions)
 * and the access scope allowed to share, so different versions or scopes never
 * match. Only full blocks are named.
 *
 * Hash: 64-bit FNV-1a (offset basis 0xcbf29ce484222325, prime 0x100000001b3).
 * root = FNV-1a over the caller's key bytes; block i's hash = FNV-1a over the
 * 8 little-endian bytes of the previous hash (the root for block 0) followed
 * by the block's page_tokens token ids as 4 little-endian bytes each.
 *
 * The index lives with the pool (host memory) and holds one reference on each
 * indexed page, so an indexed page stays allocated after every sequence has
 * freed it, until kv_prefix_evict drops it. Not thread-safe, like the pool. */
vs_status kv_prefix_root(const void* key, size_t len, uint64_t* root);
/* hashes[i] for the floor(n_tokens / page_tokens) full blocks of tokens[0 .. n_tokens). */
vs_status kv_prefix_chain(uint64_t root, const int32_t* tokens, int32_t n_tokens, int32_t page_tokens,
                          uint64_t* hashes);
/* Index the n_blocks leading full blocks of a sequence whose K/V are in pages[0 .. n_blocks) (call it
 * once the step that wrote them has completed). hashes must be the chain of tokens under root
 * (checked); a block already indexed keeps its page (the caller's copy is left alone). Each new entry
 * takes one reference on its page. *n_added (may be NULL) = entries added. */
vs_status kv_prefix_insert(vs_pool* pool, uint64_t root, const uint64_t* hashes, const int32_t* tokens,
                           const int32_t* pages, int32_t n_blocks, int32_t* n_added);
/* The longest run of leading blocks indexed under these hashes whose stored tokens (and parent
 * hash) also match, *n_hit of them; pages_out[0 .. *n_hit) receive their pages, each with one
 * reference taken for the caller (released with kv_free like any other page). Marks them used. */
vs_status kv_prefix_lookup(vs_pool* pool, uint64_t root, const uint64_t* hashes, const int32_t* tokens,
                           int32_t n_blocks, int32_t* pages_out, int32_t* n_hit);
/* Drop up to n_pages entries whose page only the index still holds, least recently used first
 * (deeper blocks of a chain first among equals), returning their pages to the free list.
 * *n_freed (may be NULL) = pages freed. */
vs_status kv_prefix_evict(vs_pool* pool, int32_t n_pages, int32_t* n_freed);
int32_t kv_prefix_entries(const vs_pool* pool);

/* ------------------------------------------------------------------ step */

/* One step's batch ([Serving] "Continuous batching"; [KV Cache] section 06:
 * the batch is re-formed every iteration). Sequence b brings rows
 * q_start[b] .. q_start[b+1]-1; row i of sequence b sits at position
 * ctx_len[b] + i, where ctx_len[b] counts positions already in its cache.
 * The step writes K/V of every row into the pages through the block table,
 * and each row attends to positions 0 .. its own position of its own
 * sequence ([KV Cache] sections 02 and 07). */
typedef struct vs_batch_desc {
    int32_t B;          /* sequences, >= 1 */
    int32_t M;          /* rows = q_start[B] */
    int32_t M_log;      /* rows that produce logits (length of logit_rows) */
    int32_t max_rows;   /* >= rows of any one sequence */
    int32_t max_ctx;    /* >= ctx_len[b] + rows of b, for every b */
    int32_t max_blocks; /* row stride of block_tables; >= ceil(max_ctx / page_tokens) */
    const vs_pool* pool;
    const int32_t* q_start;    /* device [B+1], q_start[0] = 0, non-decreasing */
    const int32_t* ctx_len;    /* device [B] */
    const int32_t* tokens;     /* device [M] token ids (the draft tokens of a verify pass). May be the
                                  same array as out->argmax when acceptance is not fused: every
                                  token is read before any argmax is written, so a replayed
                                  greedy loop feeds each step's tokens to the next. */
    const int32_t* logit_rows; /* device [M_log], ascending row indices; NULL if M_log = 0 */
    int32_t* ctx_advance;      /* device [B] or NULL. If set, the step's last kernel adds each
                                  sequence's row count to ctx_advance[b] after every other use of
                                  ctx_len; it may be ctx_len itself (a replayed decode loop then
                                  needs no host update of the context lengths). */
    int32_t* error_flags;      /* device int32 or NULL: input validation. The device arrays are not
                                  read on the host, so their contents cannot be checked before the
                                  launch. Without this word, out-of-range values are clamped
                                  silently (a token id into [0, vocab), a page id into
                                  [0, num_pages)), so no access leaves its buffer but the result is
                                  that of other inputs. With it, the step's first kernel also ORs in
                                  VS_STEP_BAD_TOKEN for a token id outside [0, vocab),
                                  VS_STEP_BAD_PAGE for a block-table entry outside [0, num_pages)
                                  among the pages a row reads or writes, and VS_STEP_BAD_BATCH for a
                                  decreasing q_start or a negative ctx_len; the step still completes
                                  with the clamped values. The caller zeroes the word beforehand and
                                  reads it after the stream reaches the step; any bit set means
                                  the step's outputs are not valid (treat as VS_ERR_INVALID). */
    /* Shared-prefix groups, a hint (n_prefix_groups = 0: none). Group g is the sequences
       group_seq0[g] .. group_seq0[g] + group_n[g] - 1, each bringing exactly one row, whose block
       tables hold the same first group_pages[g] page ids (a prefix found with kv_prefix_lookup or
       shared with kv_share: [KV Cache] section 05, "Prefix caching", the shared blocks stored
       once) and whose contexts cover those pages (ctx_len >= 16 * group_pages[g]). The step then
       reads those pages once per group for all of the group's rows, and each sequence's own pages
       after them, the two parts merged as key splits are ([KV Cache] section 07). The groups are
       used for fp16 / bf16 models with head_dim 128 and ignored otherwise; with error_flags set,
       a group whose rows or block tables break these conditions raises VS_STEP_BAD_BATCH (the
       results of its rows are then not valid). Groups are disjoint. */
    int32_t n_prefix_groups;    /* >= 0 (host) */
    int32_t max_group_size;     /* >= every group_n[g] (host) */
    int32_t max_group_pages;    /* >= every group_pages[g] (host) */
    const int32_t* group_seq0;  /* device [n_prefix_groups], or NULL when there are none */
    const int32_t* group_n;     /* device [n_prefix_groups], each >= 1 */
    const int32_t* group_pages; /* device [n_prefix_groups], each >= 1 */
} vs_batch_desc;

#define VS_STEP_BAD_TOKEN 1
#define VS_STEP_BAD_PAGE 2
#define VS_STEP_BAD_BATCH 4

typedef struct vs_step_out {
    float* logits;     /* device [M_log][vocab] fp32, or NULL */
    int32_t* argmax;   /* device [M]: greedy token of each logit row (lowest index on exact
                          ties), -1 for rows without logits; may be NULL if M_log = 0 */
    float* top2_gap;   /* device [M]: top-1 minus top-2 logit (0 on a tie), or NULL */
    /* Fused greedy acceptance (see verify_accept); all three NULL to skip it. */
    const int32_t* g0; /* device [B] */
    int32_t* accept_len; /* device [B] */
    int32_t* bonus;      /* device [B] */
} vs_step_out;

/* Workspace bytes decode_step needs for this batch shape and model. */
vs_status decode_step_workspace_bytes(const vs_batch_desc* desc, const vs_model_desc* dims, size_t* bytes);

/* One forward step of every row of every sequence. The weights are streamed
 * once for all rows ([Spending the Idle] section 12.2; [KV Cache] section 02):
 * embedding gather, then per layer RMSNorm, QKV product with rotary q/k and
 * the K/V write into the pages, paged split-KV attention with an online-softmax
 * merge ([KV Cache] section 07, Flash-Decoding), output product + residual,
 * RMSNorm, gate/up product with SwiGLU, down product + residual; final RMSNorm
 * and LM head on the logit rows, with the per-row argmax and top-2 gap.
 * block_tables: device [B][max_blocks] int32 page ids. ws: device workspace of
 * at least decode_step_workspace_bytes. Work is queued on `stream` in order; in
 * a step that mixes one-row sequences with longer ones, or has prefix groups,
 * one attention kernel per layer runs on a second stream the library keeps per
 * device (default priority), forked from `stream` and joined back into it by
 * events before the next work on `stream`, so the step still completes in
 * `stream`'s order and may be captured into a graph. The second stream is
 * made by the first such step on a device whose stream is not being captured;
 * until then the kernels run one after the other on `stream`. */
vs_status decode_step(const vs_batch_desc* desc, const int32_t* block_tables, const vs_weights* weights,
                      const vs_step_out* out, void* ws, size_t ws_bytes, hipStream_t stream);

/* decode_step for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same step and the same kernels, with the workspace taken from a scratch
 * array the library holds in device memory, VS_NOALLOC_SCRATCH_BYTES per GPU,
 * from the first call on that GPU until the process ends. The caller still
 * owns every input and output. Allocates nothing: no hipMalloc, hipFree or
 * allocating library routine. Returns VS_ERR_SHAPE, before enqueueing
 * anything, when decode_step_workspace_bytes for this batch exceeds the array
 * (every batch of up to 64 rows of the 7B shape fits; a large-vocabulary model
 * at 64 rows does not). Every call on one GPU shares that GPU's array:
 * calls that overlap on one GPU (two streams, two threads) race and give
 * undefined results; calls serialised on one stream are safe. Nothing in the
 * array needs to start at zero. The current device must be the stream's.
 * Every kernel runs on `stream` (no second stream is made or used). */
#define VS_NOALLOC_SCRATCH_BYTES (96u << 20)
vs_status decode_step_noalloc(const vs_batch_desc* desc, const int32_t* block_tables, const vs_weights* weights,
                              const vs_step_out* out, hipStream_t stream);

/* Greedy acceptance of a verify pass ([Serving Efficiency] section 31.5;
 * [Spending the Idle] section 12.4; [KV Cache] section 08). For sequence b
 * with rows r0 = q_start[b] .. r0+K-1 holding drafts d_1..d_K (the row
 * tokens), g0[b] the target's greedy token for the first draft's position
 * (known from the previous pass) and g_j = argmax[r0+j-1] the target's greedy
 * token after row j-1: accept_len[b] = the largest n with d_j == g_{j-1} for
 * every j <= n, and bonus[b] = g_n (the target's own token at the first
 * mismatch, or after the last draft). A plain decode step is the K = 1 case
 * with d_1 = g0. All arrays are on the device. */
vs_status verify_accept(int32_t B, const int32_t* q_start, const int32_t* drafts, const int32_t* g0,
                        const int32_t* argmax, int32_t* accept_len, int32_t* bonus, hipStream_t stream);

/* Stochastic acceptance of a verify pass by modified rejection sampling
 * ([Serving Efficiency] section 31.5, Example 31.3; [Spending the Idle]
 * section 12.4; [Serving] "Lossless"; [KV Cache] section 08). The output
 * tokens follow the target distribution exactly, whatever the draft
 * distribution was.
 *
 * Sequence b has rows r0 = q_start[b] .. r0+K-1 carrying drafts d_1..d_K
 * (drafts[r0+j-1]), drawn by the draft model from q_j = q_probs[r0+j-1][.].
 * Target distributions, softmax(z / temperature) in fp32: p_0 from
 * p0_logits[b][.] (the previous pass's logits for the position of d_1), p_j
 * from logits[r0+j-1][.] (this pass's row j-1). In draft order, d_j is kept
 * when u[r0+j-1] < min(1, p_{j-1}(d_j) / q_j(d_j)); a draft with q_j(d_j) = 0
 * or an id outside [0, V) is rejected. At the first rejection (n = j-1 kept)
 * token[b] is drawn from norm(max(0, p_n - q_{n+1})) -- from p_n itself if
 * that is all zero -- and if every draft is kept (n = K), from p_K. The draw
 * is the inverse CDF in token-id order: the smallest x whose cumulative weight
 * exceeds v[b] times the total. accept_len[b] = n.
 *
 * Layouts (all device, fp32 row-major, row stride V): p0_logits [B][V],
 * logits [M][V] indexed by batch row (decode_step's logits when every row
 * produces logits, M_log = M), q_probs [M][V] (each row a distribution),
 * u [M] and v [B] uniforms in [0, 1) that the caller draws. Rows must have a
 * finite maximum; -inf entries are allowed. temperature > 0 and finite.
 * ws: device workspace of at least verify_sample_workspace_bytes(B, M, V)
 * bytes, 8-byte aligned, holding per-row softmax maxima and normalisers of
 * 2048-token segments between the two kernels. Rows past M named by q_start
 * are not read. Draws are deterministic: the same inputs give the same
 * outputs. 16-byte aligned logit rows (V a multiple of 4) take the vector
 * path; any V works. */
vs_status verify_sample_workspace_bytes(int32_t B, int32_t M, int32_t V, size_t* bytes);
vs_status verify_sample(int32_t B, int32_t M, int32_t V, const int32_t* q_start, const int32_t* drafts,
                        const float* p0_logits, const float* logits, const float* q_probs, const float* u,
                        const float* v, float temperature, int32_t* accept_len, int32_t* token, void* ws,
                        size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------ instrumentation */

/* Kernel kinds of one step, for timing. Where a product runs as split-K
 * partial sums, the kernel that adds the slices and runs the product's
 * epilogue is timed with the product's kind. */
#define VS_KERNEL_NONE 0
#define VS_KERNEL_QKV 1       /* QKV product + rotary + K/V page write */
#define VS_KERNEL_ATTN 2      /* paged split-KV attention */
#define VS_KERNEL_MERGE 3     /* split merge */
#define VS_KERNEL_OPROJ 4     /* output product + residual */
#define VS_KERNEL_GATEUP 5    /* gate/up product + SwiGLU */
#define VS_KERNEL_DOWN 6      /* down product + residual */
#define VS_KERNEL_LMHEAD 7    /* LM head + argmax partials */
#define VS_KERNEL_SMSTATS 8   /* verify_sample: per-row softmax maximum and normaliser */
#define VS_KERNEL_SAMPLE 9    /* verify_sample: accept tests and the draw */

/* Measurement aid, not part of the step's function. While armed, every
 * launch of kernel kind `kind` in decode_step or verify_sample is dispatched with
 * hipExtLaunchKernel so that start_events[i] and stop_events[i] take the
 * dispatch's own start and end times, i = 0, 1, ... up to `capacity` launches
 * (later launches are not timed). The events are caller-created hipEvent_t
 * handles. kind = VS_KERNEL_NONE disarms.
 * vs_timed_launches returns how many launches were bracketed since arming.
 * Process-wide state; not for use while another thread runs decode_step. */
vs_status vs_time_kernel(int32_t kind, void* const* start_events, void* const* stop_events, int32_t capacity);
int32_t vs_timed_launches(void);

/* Measurement aid: the streaming-read ceiling of the device. Reads `bytes` (a
 * multiple of 8192) of device memory at `buf` once, in the GEMV's load shape
 * (1 KB wave-wide nontemporal loads, rows of 8 KB spread over 512 workgroups
 * of 8 waves), and computes nothing else; sink: device array of 512 uint32
 * that is written only in a practically impossible case (it keeps the loads).
 * Asynchronous on the stream. */
vs_status vs_stream_read(const void* buf, size_t bytes, uint32_t* sink, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* VERIFY_STEP_H */
