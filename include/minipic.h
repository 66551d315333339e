/*
 * minipic.h - C ABI of libminipic.so: position-free paged prefill attention
 * for AMD Instinct MI355X (gfx950).
 *
 * The method is the one of "MiniPIC: Flexible Position-Independent Caching in
 * <100LOC" (Ordonez, Parnell):
 *   - §3.2.1 (score equation): score(t, j) = (R_t q_t)^T (R_pi(j) k~_j) / sqrt(d).
 *     The KV cache holds unrotated keys k~_j; pi(j) is the per-request logical
 *     position of key j, so one physical block can serve many requests at
 *     different offsets (§3.3.1, last paragraph).
 *   - §3.2.2 (kernel modification): each gathered K tile is rotated inside the
 *     attention kernel after a cos/sin table lookup at pi(j); V is unchanged.
 *   - §3.1.1 (three user-facing primitives): padding, SSep and PDep shape the
 *     block-level attention structure. This library takes that structure as
 *     per-block descriptors (span id and PDEP / GLOBAL bits).
 *
 * Conventions shared by every entry point:
 *   - Tensor pointers are DEVICE pointers owned by the caller, unless a comment
 *     says "host". The library never allocates or frees device memory, never
 *     synchronises, and enqueues all work on `stream` (a hipStream_t passed as
 *     void*; NULL means the default stream), so calls can be captured in a
 *     HIP graph.
 *   - Every argument check runs before the first HIP call: an invalid call
 *     returns an error code without touching the GPU. Checks cover host
 *     scalars and pointer presence only; device arrays are read only by the
 *     kernels, which clamp out-of-range indices into bounds and then record
 *     the violation in the workspace error word (see minipic_prefill_attn).
 *   - On failure, minipic_last_error() returns a thread-local description.
 */
#ifndef MINIPIC_H
#define MINIPIC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes returned by every entry point. */
#define MINIPIC_OK               0
#define MINIPIC_ERR_INVALID_ARG  (-1)  /* null pointer, negative or inconsistent size */
#define MINIPIC_ERR_UNSUPPORTED  (-2)  /* dtype, head_dim, block_size or GQA ratio not built */
#define MINIPIC_ERR_WORKSPACE    (-3)  /* workspace smaller than minipic_workspace_size() */
#define MINIPIC_ERR_HIP          (-4)  /* a HIP call or launch failed; see minipic_last_error() */

/* Element types of q, k, v, out and the caches. */
#define MINIPIC_F32   0
#define MINIPIC_BF16  1

/* Per-block descriptor bits (blk_flags). */
#define MINIPIC_BLK_PDEP    1u  /* block belongs to a PDep segment: its tokens see every earlier token */
#define MINIPIC_BLK_GLOBAL  2u  /* shared-prefix block: visible to every later token of the request */

/* Call flags (minipic_prefill_attn / minipic_reference_prerotated). */
#define MINIPIC_FLAG_ROTATE_Q  1u  /* q is unrotated; rotate each row by pi(its context index) */

/* Bits of the workspace error word (first uint32_t of the workspace). */
#define MINIPIC_EW_BLOCK   1u  /* a block_table entry was outside [0, num_blocks) */
#define MINIPIC_EW_POS     2u  /* a logical position was outside [0, max_pos) */
#define MINIPIC_EW_QCTX    4u  /* a q_ctx_idx entry was outside [0, ctx_len) */
#define MINIPIC_EW_CTX     8u  /* ctx_len exceeded max_blocks_per_req * block_size */
#define MINIPIC_EW_SPAN   16u  /* a query's span id also names a block before its own run
                                  (the span-id contract of minipic_batch is broken) */
#define MINIPIC_EW_PLAN   32u  /* minipic_prefill_run found no plan of its configuration
                                  in the workspace (nothing was computed) */

/*
 * One batch of prefill requests. Host scalars plus device arrays.
 *
 * Request r owns context tokens 0 .. ctx_len[r]-1 (its context index order)
 * laid out in logical blocks of `block_size` tokens; logical block b lives in
 * physical cache block block_table[r][b]. Its query rows are rows
 * q_indptr[r] .. q_indptr[r+1]-1 of q / out; row i is the token at context
 * index q_ctx_idx[i]. Query rows need not be a contiguous suffix (a prompt can
 * interleave cached and freshly computed spans).
 *
 * Visibility (the block structure of "MiniPIC ...", §3.1.1 and §3.3.1), for a
 * query at context index c and a key at context index j, with bc = c / 16 and
 * bj = j / 16:
 *     j <= c  and  ( PDEP(bc)  or  GLOBAL(bj)  or  span_id[bj] == span_id[bc] )
 * Contract: a span_id value names ONE contiguous run of blocks of a request.
 * The span test is evaluated on runs (found by scanning neighbours): a block
 * that carries a query's span id but lies before the start of the query's own
 * run is a different span and is not attended; when such a block exists (the
 * contract is broken) the attention calls also set MINIPIC_EW_SPAN in the
 * workspace error word. Causality is by context index, not by logical
 * position. Pad tokens are ordinary tokens.
 * Cache slots past ctx_len[r] in request r's last block hold no token: their
 * K/V may be anything (unwritten memory, NaN); they never reach a result, and
 * logical_pos entries past ctx_len[r] are not read for a result either (no
 * MINIPIC_EW_POS for them).
 */
typedef struct minipic_batch {
  int32_t num_reqs;            /* number of requests, >= 0 */
  int32_t num_q_heads;         /* Hq */
  int32_t num_kv_heads;        /* Hkv, at most 255; Hq / Hkv must be 1, 2, 4 or 8 */
  int32_t head_dim;            /* d: 64 or 128 */
  int32_t block_size;          /* tokens per cache block: must be 16 */
  int32_t max_blocks_per_req;  /* row stride of block_table / span_id / blk_flags */
  int64_t total_q;             /* q_indptr[num_reqs] (host copy) */
  int32_t max_q_len;           /* >= max_r (q_indptr[r+1] - q_indptr[r]) (host) */
  int32_t max_ctx_len;         /* >= max_r ctx_len[r] (host); sizes the split-KV plan */
  const int32_t* q_indptr;     /* [num_reqs + 1], ascending, q_indptr[0] = 0 */
  const int32_t* q_ctx_idx;    /* [total_q] context index of each query row, ascending per request */
  const int32_t* ctx_len;      /* [num_reqs] */
  const int32_t* block_table;  /* [num_reqs][max_blocks_per_req] physical block ids */
  const int32_t* logical_pos;  /* [num_reqs][max_blocks_per_req * block_size] pi per context token;
                                  16-byte aligned */
  const int32_t* span_id;      /* [num_reqs][max_blocks_per_req] */
  const uint8_t* blk_flags;    /* [num_reqs][max_blocks_per_req] MINIPIC_BLK_* bits */
} minipic_batch;

/* Launch geometry chosen for a batch (host-side planning, no GPU work). */
typedef struct minipic_launch_info {
  int32_t rows_per_tile;       /* query rows (token x head) per work item */
  int32_t tokens_per_tile;     /* query tokens per q tile */
  int32_t num_q_tiles;         /* q tiles per request (upper bound from max_q_len) */
  int32_t num_splits;          /* most pieces one tile's key-block list may be cut into */
  int32_t split_blocks;        /* shortest piece, in key blocks (longer pieces are chosen on the GPU) */
  int32_t threads;             /* threads per attention work-group */
  int64_t num_workgroups;      /* persistent attention work-groups on the current device (0: no device) */
  int64_t num_tiles;           /* num_reqs * num_q_tiles */
  int32_t partial_slots;       /* partial-result slots in the workspace (pieces of split tiles) */
  int32_t reserved;
} minipic_launch_info;

const char* minipic_version(void);
const char* minipic_status_string(int status);
/* Thread-local text of the last failure on this thread ("" if none). */
const char* minipic_last_error(void);

/*
 * Fill the cos/sin lookup table used by the in-kernel rotation ("MiniPIC ...",
 * §3.2.2: a cos/sin table lookup per K element).
 *   cos_sin : device float32 [max_pos][head_dim]; row p holds cos(p * theta_i)
 *             in columns [0, d/2) and sin(p * theta_i) in columns [d/2, d),
 *             with theta_i = base^(-2i/d) (rotate-half pairing i <-> i + d/2).
 *             Angles and sin/cos are evaluated in float64 on the GPU and
 *             rounded once to float32.
 *   max_pos > 0, head_dim even (64 or 128 for the attention kernels), base > 0.
 */
int minipic_rope_table(float* cos_sin, int32_t max_pos, int32_t head_dim, double base,
                       void* stream);

/*
 * Scatter the UNROTATED keys k~ and the values of new tokens into the paged
 * cache by slot mapping ("MiniPIC ...", abstract and §3.2: the cache stores
 * unrotated K vectors; V is stored as is).
 *   k, v         : [num_tokens][num_kv_heads][head_dim], element type `dtype`
 *   slot_mapping : int64 [num_tokens]; slot = physical_block * block_size + offset;
 *                  a negative slot skips the token; a slot beyond the cache is
 *                  skipped as well.
 *   k_cache      : [num_blocks][num_kv_heads][block_size][head_dim]
 *   v_cache      : [num_blocks][num_kv_heads][head_dim][block_size]  (V transposed
 *                  inside each block, so attention reads key-contiguous V rows)
 * Bits are copied exactly; no arithmetic is applied.
 */
int minipic_write_kv(const void* k, const void* v, const int64_t* slot_mapping, int64_t num_tokens,
                     int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                     void* k_cache, void* v_cache, int64_t num_blocks, int32_t dtype,
                     void* stream);

/* Bytes of device workspace minipic_prefill_attn needs for `batch` (host scalars only). */
int minipic_workspace_size(const minipic_batch* batch, int32_t dtype, size_t* bytes);

/* Launch geometry for `batch` (host scalars only; for tests and reporting). */
int minipic_get_launch_info(const minipic_batch* batch, int32_t dtype, minipic_launch_info* info);

/*
 * Position-free paged prefill attention ("MiniPIC ...", §3.2.1 and §3.2.2).
 *   q        : [total_q][num_q_heads][head_dim]; R_t q_t (already rotated by the
 *              query's own logical position t = pi(c)) unless MINIPIC_FLAG_ROTATE_Q.
 *   k_cache, v_cache : layouts of minipic_write_kv, holding UNROTATED keys.
 *   num_blocks : physical blocks in each cache.
 *   cos_sin  : float32 [max_pos][head_dim] as filled by minipic_rope_table;
 *              max_pos * head_dim * 4 must stay below 2^31 bytes (the kernels
 *              address the table through a 32-bit buffer range), else
 *              MINIPIC_ERR_INVALID_ARG.
 *   softmax_scale : <= 0 means 1/sqrt(head_dim).
 *   out      : [total_q][num_q_heads][head_dim], element type `dtype`.
 *   workspace: device scratch of minipic_workspace_size() bytes (256-byte
 *              aligned). Its first uint32_t is the error word: kernels OR in
 *              MINIPIC_EW_* bits when they meet out-of-range metadata (after
 *              clamping it); the caller may read it after its own sync and
 *              should zero it to reset it. The library never reads it back.
 *              Bytes 128..159 (measurement only) hold four uint64_t stamps of
 *              the attention kernel's first work-group: the shader clock
 *              counter and the 100 MHz real-time counter when it starts, then
 *              both again when it has no work left; the shader clock in MHz is
 *              100 * (clock difference) / (real-time difference).
 * Query head h reads KV head h / (num_q_heads / num_kv_heads).
 */
int minipic_prefill_attn(const void* q, const void* k_cache, const void* v_cache, int64_t num_blocks,
                         const minipic_batch* batch, const float* cos_sin, int32_t max_pos,
                         float softmax_scale, void* out, void* workspace, size_t workspace_bytes,
                         uint32_t flags, int32_t dtype, void* stream);

/*
 * minipic_prefill_attn without a caller workspace and without any allocation:
 * for callers that cannot allocate device memory (code under HIP stream
 * capture, tight serving loops, harnesses that forbid hipMalloc).
 *   The workspace is the library's own device array of
 *   MINIPIC_STATIC_WORKSPACE_BYTES bytes (one per GPU, kept until the process
 *   ends; its address is looked up on the first call on each device). A batch
 *   whose minipic_workspace_size() exceeds it is rejected with
 *   MINIPIC_ERR_WORKSPACE before any HIP call. The call allocates nothing
 *   (no hipMalloc, hipFree or allocating library routine) and records no
 *   kernel-timing events.
 *   err_word : NULL, or a 4-byte aligned device uint32_t of the caller's that
 *              receives the MINIPIC_EW_* bits (the role of the workspace's
 *              first word in minipic_prefill_attn); the caller zeroes it and
 *              reads it after its own sync. With NULL the bits are dropped.
 *   Every other argument, the result and the kernels are those of
 *   minipic_prefill_attn, bit for bit.
 * Every call on one GPU shares that GPU's array, which keeps the last call's
 * contents (each call rebuilds what it reads): calls that can overlap on one
 * GPU (different streams, or host threads without ordering) race and must not
 * be made; calls in order on one stream are safe.
 */
#define MINIPIC_STATIC_WORKSPACE_BYTES (128u * 1024u * 1024u)
int minipic_prefill_attn_static(const void* q, const void* k_cache, const void* v_cache, int64_t num_blocks,
                                const minipic_batch* batch, const float* cos_sin, int32_t max_pos,
                                float softmax_scale, void* out, uint32_t* err_word, uint32_t flags,
                                int32_t dtype, void* stream);

/*
 * The same kernel without the in-kernel key rotation: k_cache holds keys that
 * are ALREADY rotated (R_pi(j) k~_j), as in the baseline FlashAttention of
 * "MiniPIC ...", §3.2.2. Used to measure the cost of the rotation. cos_sin /
 * max_pos are needed only with MINIPIC_FLAG_ROTATE_Q (may be NULL / 0 otherwise).
 */
int minipic_reference_prerotated(const void* q, const void* k_cache, const void* v_cache,
                                 int64_t num_blocks, const minipic_batch* batch,
                                 const float* cos_sin, int32_t max_pos, float softmax_scale,
                                 void* out, void* workspace, size_t workspace_bytes,
                                 uint32_t flags, int32_t dtype, void* stream);

/*
 * minipic_prefill_attn in two parts, for a model that runs the same batch
 * through many layers: the work decomposition of the position-free paged
 * attention ("MiniPIC ...", §3.2.1 and §3.2.2: which key blocks each query
 * tile sees, the pieces long key lists are cut into, their queues and the
 * split groups to merge) depends only on the batch's descriptors, not on q or
 * the caches, so it can be built once and used by every layer.
 *   minipic_prefill_plan : launches the planning kernels only. Arguments as
 *              for minipic_prefill_attn (q, the caches and out are not taken;
 *              num_blocks, cos_sin / max_pos and flags are, since the plan
 *              checks block numbers and key positions against them).
 *   minipic_prefill_run  : launches the attention and merge kernels on a
 *              workspace that holds a plan of the same batch, made by
 *              minipic_prefill_plan with the same num_blocks, cos_sin,
 *              max_pos, flags and dtype on the same device (the caller
 *              keeps the batch's device arrays unchanged in between). Its
 *              results are those of minipic_prefill_attn, bit for bit. The
 *              run leaves the plan ready for the next run (the merge kernel
 *              re-arms the scheduler's counters), so one plan serves any
 *              number of runs in order on one stream.
 * The plan records a key of its configuration in the workspace (the scalars
 * above, the batch's scalars and array addresses, the launch size); a run
 * whose key differs computes nothing, leaves out untouched and sets
 * MINIPIC_EW_PLAN in the error word. Host-side errors are returned as by
 * minipic_prefill_attn. Runs and plans on one workspace must not overlap.
 */
int minipic_prefill_plan(int64_t num_blocks, const minipic_batch* batch, const float* cos_sin, int32_t max_pos,
                         void* workspace, size_t workspace_bytes, uint32_t flags, int32_t dtype, void* stream);
int minipic_prefill_run(const void* q, const void* k_cache, const void* v_cache, int64_t num_blocks,
                        const minipic_batch* batch, const float* cos_sin, int32_t max_pos,
                        float softmax_scale, void* out, void* workspace, size_t workspace_bytes,
                        uint32_t flags, int32_t dtype, void* stream);

/*
 * Decode-phase position-free paged attention: one query row per request
 * ("MiniPIC ...", §3.2.1 score equation, §3.2.2 rotation of each K tile at
 * pi(j); visibility rule of §3.1.1 / §3.3.1 as for prefill). Memory bound:
 * each visible K/V block is read once per KV head.
 *   q        : [num_reqs][num_q_heads][head_dim] bf16; row r is request r's
 *              query, already rotated by its own logical position.
 *   batch    : as for minipic_prefill_attn, with total_q == num_reqs;
 *              q_ctx_idx[r] is the context index of request r's query (usually
 *              ctx_len[r] - 1). q_indptr is not read.
 *   k_cache, v_cache, num_blocks, cos_sin, max_pos, softmax_scale : as for
 *              minipic_prefill_attn (k_cache holds UNROTATED keys).
 *   out      : [num_reqs][num_q_heads][head_dim] bf16.
 *   workspace: minipic_decode_workspace_size() bytes, 256-byte aligned; its
 *              first uint32_t is the error word, as for prefill.
 * dtype must be MINIPIC_BF16 (else MINIPIC_ERR_UNSUPPORTED); flags must be 0.
 * Two kernels run on `stream`: the split attention and the merge of splits.
 */
int minipic_decode_workspace_size(const minipic_batch* batch, int32_t dtype, size_t* bytes);
int minipic_decode_attn(const void* q, const void* k_cache, const void* v_cache, int64_t num_blocks,
                        const minipic_batch* batch, const float* cos_sin, int32_t max_pos,
                        float softmax_scale, void* out, void* workspace, size_t workspace_bytes,
                        uint32_t flags, int32_t dtype, void* stream);

/*
 * Decode without the in-kernel key rotation: k_cache holds keys ALREADY
 * rotated by their positions (the pre-rotated baseline of "MiniPIC ...",
 * §3.2.2), for the cost of the rotation in decode.
 */
int minipic_decode_prerotated(const void* q, const void* k_cache, const void* v_cache,
                              int64_t num_blocks, const minipic_batch* batch, float softmax_scale,
                              void* out, void* workspace, size_t workspace_bytes, uint32_t flags,
                              int32_t dtype, void* stream);

/*
 * Kernel timing, for measurement (not part of the method). With timing on,
 * every attention call (prefill, decode, and their pre-rotated variants) of
 * the calling host thread also records four HIP events on its stream, around
 * the planning kernels (none for decode), the attention kernel and the merge
 * kernel.
 * Switching timing on (or off) forgets the calls timed before.
 * minipic_kernel_times waits for the most recent such call of the thread to
 * finish and writes the three durations in milliseconds to ms[0..2] (plan,
 * attention, merge).
 * minipic_kernel_times_all waits for the most recent call and writes the
 * three durations of every call timed since timing was switched on, oldest
 * first, to ms[3 c .. 3 c + 2] for call c < *num_calls; *num_calls is at most
 * max_calls and at most 4096 (only the latest 4096 calls are kept). It lets a
 * caller time a run of calls without waiting after each one.
 * Both return MINIPIC_ERR_INVALID_ARG when timing is off, no call was timed
 * yet or a pointer is NULL, MINIPIC_ERR_HIP when the events fail. The events
 * belong to the library (one set of four per kept call and host thread, kept
 * until the process ends).
 */
int minipic_set_kernel_timing(int enable);
int minipic_kernel_times(float* ms);
int minipic_kernel_times_all(float* ms, int32_t max_calls, int32_t* num_calls);

#ifdef __cplusplus
}
#endif
#endif /* MINIPIC_H */
