/*
 * pakv.h - C ABI of libpakv: decode-step paged attention over a shared pool
 * of BF16 KV pages, for AMD Instinct MI355X (gfx950).
 *
 * The operation (sources cited by page title and section):
 *
 *  - "Curso gratuito recorre la inferencia de LLM con videos, notas y un motor
 *    funcional en C++" (news-factory.app), section "¿Cómo administra el motor
 *    la memoria de la caché KV?": one shared pool of BF16 pages, each physical
 *    page holding keys and values for 16 tokens; one block table per sequence
 *    and layer; decode attention reads each sequence's cached pages in place,
 *    with an FP32 online softmax, instead of gathering a contiguous prefix. A
 *    request that cannot be served is rejected with an error, not a crash.
 *  - comrad404.com review of the samir-vllm README, section "Что README
 *    говорит о KV-кэше и пакетном декодировании": decode adds the new token's
 *    keys and values to the request's pages.
 *  - "Construye tu propio motor de inferencia LLM de alto rendimiento en C++ y
 *    CUDA" (aibit.im), section "Atención de Consulta Agrupada (GQA)": several
 *    query heads share one KV head, grouped contiguously (query head h reads
 *    KV head h / (Hq / Hkv)); section "El truco de transposición de cuBLAS":
 *    the K/V projection yields one row of Hkv * head_dim BF16 values per
 *    sequence, which is the append input.
 *
 * For sequence b with n = context_lens[b] cached tokens and query head h,
 * g = h / (Hq / Hkv):
 *     s_t      = scale * sum_i q[b][h][i] * K(b, t)[g][i]      t = 0 .. n-1
 *     out[b][h] = sum_t softmax(s)_t * V(b, t)[g]
 * where token t of sequence b is slot t % 16 of physical page
 * block_tables[b][t / 16]. n == 0 gives an all-zero output row.
 *
 * Memory layout (all device memory is owned by the caller; the library never
 * allocates, frees or synchronises, and queues all work on the caller's
 * stream):
 *  - K pool: BF16 [num_pages][num_kv_heads][head_dim / 32][16][32]
 *            element (p, g, slot, i) at
 *            ((p * Hkv + g) * 16 * d) + (i / 32) * 512 + slot * 32 + i % 32
 *  - V pool: BF16 [num_pages][num_kv_heads][head_dim][16]
 *            element (p, g, slot, i) at ((p * Hkv + g) * d + i) * 16 + slot
 *    One physical page id indexes both pools, and each (page, KV head) tile is
 *    16 * d contiguous elements in both. Inside a K tile the dimensions come
 *    in slabs of 32: a slab holds 64 bytes of every slot, so the 16-byte
 *    operand pieces one matrix-core K-step needs from 16 tokens fill whole
 *    128-byte cache lines. The V pool keeps the 16 slots of each dimension
 *    together so that a decode lane's 16-byte load is exactly one
 *    matrix-core operand (8 consecutive tokens of one dimension).
 *  - q: BF16 [num_seqs][num_q_heads][head_dim]
 *  - out: FP32 [num_seqs][num_q_heads][head_dim]
 *  - k_new, v_new: BF16 [num_seqs][num_kv_heads][head_dim]
 *  - block_tables: int32 [num_seqs][max_pages_per_seq] (one layer's table)
 *  - context_lens, positions: int32 [num_seqs]
 * Alignment: the pools, q, out, k_new, v_new and the workspace must be
 * 16-byte aligned (they are accessed with 16-byte loads and stores); the
 * int32 arrays need 4-byte alignment.
 *
 * Device-resident data is not read by the host. Preconditions on it: page ids
 * in [0, num_pages); context_lens[b] in [0, max_pages_per_seq * 16]; the
 * tokens a sequence attends over hold finite values. The kernels clamp page
 * ids and context lengths into range so that a violation cannot read or write
 * outside the pool, but the result for that sequence is then meaningless.
 * Slots past context_lens[b] and pages no block table names may hold any bits
 * (NaN included): they never contribute.
 *
 * Errors: every entry point returns a pa_status and never aborts; arguments
 * are validated on the host before any work is queued. A launch failure
 * reported by the HIP runtime gives PA_ERR_LAUNCH.
 */
#ifndef PAKV_H
#define PAKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. Compiled as C++ the enum is given int as its underlying
 * type, so that any int a C caller passes (pa_status_str of an unknown
 * code, say) is a valid value on both sides; the size and the calling
 * convention are those of an int either way. */
typedef enum pa_status
#ifdef __cplusplus
    : int
#endif
{
  PA_OK = 0,
  PA_ERR_NULL = 1,        /* a required pointer is NULL */
  PA_ERR_INVALID = 2,     /* a count or size is out of range (also: the host could not
                             allocate the memory a descriptor or a plan needs) */
  PA_ERR_UNSUPPORTED = 3, /* valid in principle, not built: head_dim, page size, group size */
  PA_ERR_ALIGN = 4,       /* a device pointer is not aligned as documented below */
  PA_ERR_WORKSPACE = 5,   /* workspace missing or smaller than pa_decode_workspace_bytes */
  PA_ERR_LAUNCH = 6,      /* the HIP runtime reported an error when queueing a kernel */
  PA_ERR_CAPACITY = 7,    /* a request larger than the whole pool: rejected (pakv_sched.h) */
  PA_ERR_STATE = 8        /* a request is not in a state that allows the call (pakv_sched.h) */
} pa_status;

/* Opaque host-side description of one K/V page pool (no device memory). */
typedef struct pa_pool pa_pool;

/*
 * Describe a caller-owned pool. k_pages / v_pages: device pointers laid out as
 * above. page_size must be 16 (the page of the samir-vllm pool);
 * head_dim must be 64 or 128; num_kv_heads >= 1; num_pages >= 1.
 * On success *out receives a descriptor to release with pa_pool_destroy.
 * No device work is queued.
 */
pa_status pa_pool_create(pa_pool** out, void* k_pages, void* v_pages,
                         int32_t num_pages, int32_t page_size,
                         int32_t num_kv_heads, int32_t head_dim);

/* Release a descriptor (not the pool memory). NULL is ignored. */
void pa_pool_destroy(pa_pool* pool);

/*
 * Paged write of each sequence's new token (decode adds the new token's K/V,
 * samir-vllm README review): for every b with 0 <= positions[b] <
 * max_pages_per_seq * 16, copies k_new[b] / v_new[b] bit for bit into slot
 * positions[b] % 16 of page block_tables[b][positions[b] / 16] in the K and V
 * pools. A negative position skips the sequence; so does a page id outside
 * the pool. No other pool byte changes. Queued on `stream` (a hipStream_t;
 * NULL is the default stream); a pa_decode queued after it on the same
 * stream sees the new token. num_seqs == 0 queues nothing.
 */
pa_status pa_kv_append(const pa_pool* pool, const void* k_new, const void* v_new,
                       int32_t num_seqs, const int32_t* block_tables,
                       int32_t max_pages_per_seq, const int32_t* positions,
                       void* stream);

/*
 * Bytes of workspace pa_decode needs for these sizes: 0 when no context can
 * have more splits than one workgroup finishes itself (4 splits, or 2 when
 * more than 8 query heads share a KV head). Contexts are cut into splits of
 * a fixed number of tokens per head_dim (pa_split_tokens); the split
 * partials of longer contexts are kept in the workspace and merged by
 * log-sum-exp. Returns 0 for a NULL pool, non-positive sizes, or a query-head
 * count that is not a multiple of the pool's KV heads.
 */
size_t pa_decode_workspace_bytes(const pa_pool* pool, int32_t num_seqs,
                                 int32_t num_q_heads, int32_t max_pages_per_seq);

/* Tokens per split for a head_dim: 2048 at 64, 1024 at 128; 0 for others.
 * Fixed per head_dim, so a sequence's result never depends on the rest of
 * the batch. */
int32_t pa_split_tokens(int32_t head_dim);

/*
 * Decode-step paged attention for one layer: out[b][h] as defined above,
 * FP32 accumulation and FP32 online softmax. q: BF16 queries; num_q_heads a
 * multiple of the pool's num_kv_heads with at most 16 query heads per KV
 * head; block_tables / context_lens: this layer's table and lengths;
 * scale: softmax scale; scale and scale * log2(e) must be finite in FP32
 * (else PA_ERR_INVALID), and scale * <q, k> * log2(e) must stay finite in
 * FP32 for every attended key (a precondition on device data). workspace:
 * device memory of at least
 * pa_decode_workspace_bytes(...) bytes (may be NULL when that is 0); its
 * contents need no initialisation and are overwritten. Queued on `stream`.
 * num_seqs == 0 queues nothing.
 *
 * How the result is reduced (fixed per head_dim and group size, never by
 * the batch): splits of pa_split_tokens tokens; inside a split, W logical
 * waves (16 at head_dim 64, 8 at 128) each take every W-th pair of pages
 * with their own online-softmax state, merged in logical-wave order; the
 * splits of a sequence merged by log-sum-exp in split order. Without a plan
 * one workgroup takes the splits of a sequence in groups of 4 (2 when more
 * than 8 query heads share a KV head); a sequence with at most that many
 * splits is finished inside its workgroup, a longer one by a second, merge
 * kernel.
 */
pa_status pa_decode(const pa_pool* pool, const void* q, int32_t num_seqs,
                    int32_t num_q_heads, const int32_t* block_tables,
                    int32_t max_pages_per_seq, const int32_t* context_lens,
                    float scale, float* out, void* workspace,
                    size_t workspace_bytes, void* stream);

/*
 * pa_kv_append followed by pa_decode, in one call: decode adds the new token
 * to the cache and then attends over it (samir-vllm README review;
 * news-factory.app course article, KV-cache section). Arguments are those of
 * the two calls; k_new / v_new / positions as in pa_kv_append; every
 * argument of both is checked before either is queued. Queues the append
 * kernel, then the decode, so the pool after the call and `out` are
 * bit-identical to those of the two separate calls, and context_lens[b] may
 * include the new token (the usual case: positions[b] == context_lens[b] - 1).
 */
pa_status pa_decode_append(const pa_pool* pool, const void* q, const void* k_new,
                           const void* v_new, const int32_t* positions, int32_t num_seqs,
                           int32_t num_q_heads, const int32_t* block_tables,
                           int32_t max_pages_per_seq, const int32_t* context_lens,
                           float scale, float* out, void* workspace,
                           size_t workspace_bytes, void* stream);

/*
 * Launch plan (host side, optional). Without one, pa_decode runs one
 * workgroup per sequence and group of splits, however uneven the contexts.
 * A plan packs the batch's units (one split of one sequence each) into work
 * items of up to 4 units (2 when more than 8 query heads share a KV head)
 * and the items into bins, one persistent workgroup per bin and KV head
 * that runs its bin's items in turn:
 *  - a sequence with at most that many splits is one group, kept whole in
 *    one item (finished inside its workgroup, as without a plan); a longer
 *    one gives one group per split (its split partials merged by the merge
 *    kernel);
 *  - a group costs its page pairs plus 2 per unit (the fixed work of an
 *    item's start and merge); groups, costliest first, go each to the bin
 *    of least cost so far (ties: the lower bin), over as many bins as the
 *    device holds decode workgroups at once divided by the KV heads (or one
 *    per group when there are fewer groups), so that the bins end together;
 *  - in each bin, its groups in that order go to the first of its items
 *    with room (a new item when none has);
 *  - item b (b < bins) is bin b's first item; every item names the bin's
 *    next one, and those are listed after all the first items, bin by bin.
 * Each item also carries, per unit, the count of pairs before it in the
 * item (mod the waves per workgroup), so the workgroup's waves deal all of
 * the item's pairs round-robin. Serving code knows its context lengths on
 * the host, and one plan serves every layer of a step.
 *
 * pa_decode_plan_capacity: int32 words a plan may need for these sizes
 * (8 per possible unit: num_seqs * splits per sequence * 8), or -1 when the
 * sizes are out of range (num_seqs above 2^20, or more than 2^11 splits per
 * sequence).
 * pa_decode_plan: writes the plan for the host array context_lens_host
 * [num_seqs] (values clamped into [0, max_pages_per_seq * 16], as the
 * kernel does) and num_q_heads into plan[capacity] (host memory) and its
 * length in int32 words into *num_ints. Item encoding, 8 words: units
 * b | (split << 20), or -1 for none, in words 0..3; the units' rotations,
 * 4 bits each, in word 4; the index of the bin's next item in word 5 (0 for
 * none; the kernel ends a chain at any index that is not above the
 * current one or not among the items after the first ones); words 6..7
 * zero. Pure host code; queues nothing. PA_ERR_INVALID when the plan would
 * not fit `capacity` or host memory runs out.
 */
int64_t pa_decode_plan_capacity(const pa_pool* pool, int32_t num_seqs,
                                int32_t max_pages_per_seq);
pa_status pa_decode_plan(const pa_pool* pool, const int32_t* context_lens_host,
                         int32_t num_seqs, int32_t num_q_heads, int32_t max_pages_per_seq,
                         int32_t* plan, int64_t capacity, int32_t* num_ints);

/*
 * pa_decode driven by a plan: the same arguments, plus plan (device memory,
 * int32 [num_ints], a copy of what pa_decode_plan wrote for the same context
 * lengths and num_q_heads) and num_ints (a multiple of 8). The output is
 * bit-identical to pa_decode's: the splits, the logical waves and the merge
 * order do not depend on which workgroup runs a unit. A plan made from other
 * lengths leaves the output of the sequences it misses unwritten; units
 * naming a sequence or split out of range are skipped on the device.
 */
pa_status pa_decode_planned(const pa_pool* pool, const void* q, int32_t num_seqs,
                            int32_t num_q_heads, const int32_t* block_tables,
                            int32_t max_pages_per_seq, const int32_t* context_lens,
                            float scale, float* out, void* workspace,
                            size_t workspace_bytes, const int32_t* plan,
                            int32_t num_ints, void* stream);

/*
 * pa_decode_planned with the plan in host memory (plan_host: what
 * pa_decode_plan wrote, num_ints <= 2048 words, i.e. at most 256 items). The
 * plan travels by value in the decode kernel's arguments, which the HIP
 * runtime copies when the launch is queued: nothing is copied to device
 * memory beforehand, no device plan buffer is needed, and plan_host may be
 * reused or freed as soon as the call returns. Larger plans give
 * PA_ERR_INVALID (use pa_decode_planned). Same results, bit for bit. The
 * argument block grows with the plan (1 KiB up to 256 words, 8 KiB above):
 * measured on MI355X, queueing an 8 KiB block costs the host ~60 us per
 * launch against ~4 us for pa_decode_planned, whose plan is one copy to the
 * device per step instead; the device time is the same either way.
 */
pa_status pa_decode_planned_host(const pa_pool* pool, const void* q, int32_t num_seqs,
                                 int32_t num_q_heads, const int32_t* block_tables,
                                 int32_t max_pages_per_seq, const int32_t* context_lens,
                                 float scale, float* out, void* workspace,
                                 size_t workspace_bytes, const int32_t* plan_host,
                                 int32_t num_ints, void* stream);

/*
 * pa_decode for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same arguments without the workspace, the same output bit for bit. The
 * split partials go to the library's own scratch, a static device array of
 * 32 MiB per device (held until the process ends; its address is looked up
 * on the device's first call). Calls that would need more give
 * PA_ERR_WORKSPACE (the need is pa_decode_workspace_bytes of the same
 * sizes). Nothing is allocated or freed; the scratch needs no clearing
 * (a launch reads only what it wrote). All calls on one GPU share that GPU's
 * scratch: calls that overlap on one GPU (on different streams) race.
 */
pa_status pa_decode_static(const pa_pool* pool, const void* q, int32_t num_seqs,
                           int32_t num_q_heads, const int32_t* block_tables,
                           int32_t max_pages_per_seq, const int32_t* context_lens,
                           float scale, float* out, void* stream);

/*
 * Paged prefill. A chunk of new tokens per sequence: prefill fills a
 * request's pages (samir-vllm README review, KV-cache section) and processes
 * all of its tokens at once ("Construye tu propio motor de inferencia LLM
 * ..." (aibit.im), section "Prefill vs. Decode").
 *
 * Rows: sequence b owns rows query_start[b] .. query_start[b+1]-1 of the row
 * arrays (q: BF16 [num_rows][num_q_heads][head_dim]; k_rows, v_rows: BF16
 * [num_rows][num_kv_heads][head_dim]; out: FP32 [num_rows][num_q_heads]
 * [head_dim]). Its row i is the token at position context_lens[b] + i:
 * context_lens gives the tokens already in the cache before the chunk (0 for
 * a new request; the shared prefix, or earlier chunks, otherwise).
 * query_start: int32 [num_seqs + 1], nondecreasing, device memory.
 * max_chunk: a host-side bound on every chunk's length (the grid is sized
 * from it; longer chunks are cut to it).
 *
 * pa_kv_write: writes every chunk token's K/V into its page slot (slot
 * pos % 16 of page block_tables[b][pos / 16]), bit for bit, nothing else.
 *
 * pa_prefill: pa_kv_write, then causal grouped-query attention: the token at
 * position p of sequence b attends over positions 0 .. p of that sequence
 * (its own chunk and the cache before it), read in place from the pages;
 * FP32 accumulation and online softmax as in pa_decode. out[row][h] is
 * written for every chunk row. Both calls queue their kernels on `stream`.
 *
 * Preconditions as for pa_decode (page ids in the pool; positions within the
 * block-table row). Row offsets and lengths are clamped on the device so a
 * violation cannot touch memory outside the row arrays, the pool or the
 * block-table row. Alignment: q, k_rows, v_rows, out 16 bytes; int32 arrays
 * 4 bytes. num_seqs, num_rows or max_chunk == 0 queues nothing.
 */
pa_status pa_kv_write(const pa_pool* pool, const void* k_rows, const void* v_rows,
                      int32_t num_seqs, int32_t num_rows, int32_t max_chunk,
                      const int32_t* query_start, const int32_t* block_tables,
                      int32_t max_pages_per_seq, const int32_t* context_lens, void* stream);
pa_status pa_prefill(const pa_pool* pool, const void* q, const void* k_rows, const void* v_rows,
                     int32_t num_seqs, int32_t num_q_heads, int32_t num_rows, int32_t max_chunk,
                     const int32_t* query_start, const int32_t* block_tables,
                     int32_t max_pages_per_seq, const int32_t* context_lens, float scale,
                     float* out, void* stream);

/*
 * Launch plan for pa_prefill (optional; the same results bit for bit).
 * pa_prefill's grid visits every (sequence, row block of 128 query rows) in
 * a fixed order; the attention of a row block costs in proportion to the
 * keys its last row can see, which depends on the cache and chunk lengths
 * the device holds. A host that knows those lengths (the scheduler does)
 * can order the row blocks by that cost instead, largest first, leaving out
 * the blocks past each chunk's end: when the whole grid fits the device at
 * once (row blocks x num_kv_heads <= 256 CUs x the prefill workgroups a CU
 * holds: 4 at head_dim 64, 2 at 128), every other tier of row blocks that
 * the CUs of one XCD take in turn is reversed, pairing large blocks with
 * small ones on each CU, as pa_decode_plan does for splits.
 *
 * pa_prefill_plan_capacity: items a plan may need (num_seqs x row blocks
 * per sequence), or -1 when the sizes are out of range (num_seqs above
 * 2^20, more than 2^11 row blocks, or a query-head count pa_prefill
 * refuses).
 * pa_prefill_plan: writes the plan for the host arrays context_lens_host and
 * chunk_lens_host ([num_seqs]; the tokens cached before the chunk and the
 * chunk's length, clamped as the kernels clamp them) into plan[capacity]
 * (host memory) and its length into *num_items. Item encoding:
 * b | (row_block << 20). Pure host code; queues nothing.
 * pa_prefill_planned: pa_prefill's arguments plus plan (device memory, int32
 * [num_items], a copy of what pa_prefill_plan wrote) and num_items. Items
 * naming a sequence or row block out of range are skipped on the device; a
 * plan made from other lengths leaves the rows it misses unwritten.
 */
int64_t pa_prefill_plan_capacity(const pa_pool* pool, int32_t num_seqs, int32_t num_q_heads,
                                 int32_t max_chunk);
pa_status pa_prefill_plan(const pa_pool* pool, const int32_t* context_lens_host,
                          const int32_t* chunk_lens_host, int32_t num_seqs, int32_t num_q_heads,
                          int32_t max_pages_per_seq, int32_t max_chunk, int32_t* plan,
                          int64_t capacity, int32_t* num_items);
pa_status pa_prefill_planned(const pa_pool* pool, const void* q, const void* k_rows,
                             const void* v_rows, int32_t num_seqs, int32_t num_q_heads,
                             int32_t num_rows, int32_t max_chunk, const int32_t* query_start,
                             const int32_t* block_tables, int32_t max_pages_per_seq,
                             const int32_t* context_lens, float scale, float* out,
                             const int32_t* plan, int32_t num_items, void* stream);

/* Human-readable text for a status code (static storage). */
const char* pa_status_str(pa_status status);

/*
 * Measurement helpers (not part of the attention path).
 *
 * pa_profile_start: from now on, bracket every kernel the library queues
 * with a pair of HIP events on the same stream. pa_profile_stop waits for
 * those events, returns the summed milliseconds and launch counts per kernel
 * kind (index 0: decode split kernel, 1: split merge kernel, 2: append
 * kernel, 3: chunk write kernel, 4: prefill attention kernel) in ms[5] /
 * launches[5], and stops recording. Not thread-safe.
 */
pa_status pa_profile_start(void);
pa_status pa_profile_stop(double* ms, int64_t* launches);

/*
 * Streaming-read ceiling: reads `bytes` (a multiple of 16) from src with
 * 16-byte loads and writes nothing visible except, improbably, one word of
 * `sink`. Used to measure the achievable HBM read bandwidth of the device.
 */
pa_status pa_stream_read(const void* src, size_t bytes, void* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PAKV_H */
