/*
 * mac.h -- C ABI of the MAC-Attention decode library for MI355X (gfx950).
 *
 * The operation is the decode step of MAC-Attention (arXiv 2604.00235; paper
 * card at thelatestinai.com, abstract and Figure 2): for every (request,
 * query head) the pre-RoPE query is matched by L2 distance against a short
 * ring of recent pre-RoPE queries (match, Figure 2 (a)); on a hit only the
 * band+tail of the KV cache is attended and merged in the log domain with the
 * matched entry's cached prefix summary (complete, Figure 2 (b)); off the
 * critical path the last r keys are removed from the new summary and the pair
 * (pre-RoPE query, summary) enters the ring (amend, Figure 2 (c)).  A miss is
 * full attention over the whole context.  mac_prefill applies the same policy
 * to a prompt with an unbounded window (the pages' Table 8 ablation).
 *
 * Conventions for every call:
 *  - Pointers are device pointers unless marked "host".  The key/value
 *    caches, k_new, v_new, the queries (q_pre_rope, q_pre) and out must be
 *    16-byte aligned (the kernels move rows as 16-byte vectors); a misaligned
 *    one is MAC_EINVAL.
 *  - Positions are 0-based.  For request b the query position is
 *    m = seq_lens[b] - 1; its own K/V row must already be in the cache.
 *  - A summary (o, M, l) is the normalised attention output o[d], a reference
 *    max M of the scaled logits and the normaliser l = sum exp(logit - M).
 *  - Calls are asynchronous on the stream they receive (NULL: the handle's main
 *    stream) unless stated.  A handle is one attention layer and is not
 *    thread-safe.  Its calls may use different streams: a decode, prefill or
 *    reset call on another stream than the handle's previous one waits for
 *    that call's work (an event recorded at the end of each call; none is
 *    recorded on a stream being captured into a graph, and calls that follow
 *    a captured one on another stream must be ordered by the caller).
 *  - A HIP failure part-way through mac_decode_step or mac_prefill can leave
 *    the device state out of step with the host's; both calls then return
 *    MAC_ESTATE until mac_reset succeeds.
 *  - No C++ exception crosses this boundary.  Every call returns mac_status;
 *    mac_last_error() gives the handle's last message.  Shape and pointer
 *    errors are caught on the host before any launch.  Device faults surface
 *    as MAC_EHIP at the next synchronising call.  Data values are not
 *    validated (NaN propagates); indices read from device memory are
 *    bounds-checked on the device and never dereferenced out of range: a
 *    sequence length past the cache idles its request, an append position
 *    past it skips its row, and a page id outside the pool is read as page 0
 *    (that request's output is then meaningless).  Each is counted in
 *    mac_stats_t.bad_input.
 */
#ifndef MAC_H
#define MAC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct mac_ctx *mac_handle;

typedef enum {
    MAC_OK = 0,
    MAC_EINVAL = 1,          /* bad argument or configuration */
    MAC_ENOMEM = 2,          /* device allocation failed */
    MAC_EHIP = 3,            /* a HIP runtime call failed */
    MAC_ESTATE = 4,          /* call not valid in the handle's state */
    MAC_EUNSUPPORTED = 5     /* valid request this build does not implement */
} mac_status;

typedef enum { MAC_KV_CONTIGUOUS = 0, MAC_KV_PAGED = 1 } mac_kv_layout;
typedef enum { MAC_BF16 = 0, MAC_FP32 = 1 } mac_dtype;

enum {
    MAC_F_DISABLE_REUSE = 1u,  /* every head misses: plain full attention, no ring upkeep */
    MAC_F_SYNC_AMEND = 2u,     /* run amend on the decode stream instead of the amend stream */
    MAC_F_TIMING = 4u,         /* time each kernel with HIP events (read via mac_stats) */
    MAC_F_RECORD_DEBUG = 8u,   /* keep per-head decisions for mac_debug_last */
    /* Fused amend (a variant of Figure 2 (c)): complete cuts every span before
     * the band [m-r+1, m], and the reduce forms AS_{1:m-r} as the stored
     * prefix merged with the part before the band and writes the ring entry
     * itself: no band re-read, no log-domain removal, no amend stream work.
     * Same results up to rounding.  Where a step is short (a small batch) it
     * is the fast form: the default hands each call's amend to the second
     * stream through a cross-queue event wait, which costs 11-16 us of host
     * time per call on this runtime (spent by the handle's own thread when it
     * created the amend stream) and runs amend after the reduce. */
    MAC_F_FUSED_AMEND = 16u,
    /* Keep the ring's pre-RoPE queries as bfloat16 (rounded to nearest, ties
     * to even) and match against those: half the match traffic, ~6x a token's
     * K/V bytes per ring entry as in the pages' Table 7.  Decisions can differ
     * from the fp32 ring where the nearest entries are within rounding. */
    MAC_F_RING_BF16 = 32u,
    /* Stale-by-one ring (the asynchronous cache update of Figure 2 (c) with
     * one call of lag): the match of call t ignores the entry call t-1
     * inserts, so it need not wait for that call's amend, which then runs
     * beside call t's match (and, on a stream the handle owns, its complete).
     * Call t's match and overrides see the entries of calls t-W .. t-2; the
     * first two calls after init or reset miss, and W = 1 never hits.  Not
     * combinable with MAC_F_FUSED_AMEND (MAC_EINVAL). */
    MAC_F_STALE_RING = 64u,
    /* Measurement baseline for Figure 8 (b): replace the balanced plan (the
     * step's pages split evenly over the waves of the complete grid, Figure
     * 3 (b)) with an unbalanced one that gives every (request, KV group) the
     * same number of waves, so the longest span sets the step's time.  Same
     * results up to rounding.  MAC_EUNSUPPORTED at mac_init when the grid has
     * fewer waves than batch * num_kv_heads (x2 with MAC_F_FUSED_AMEND). */
    MAC_F_UNBALANCED_PLAN = 128u
};

/* Layer configuration (host struct).  head_dim must be 128; Hq % Hkv == 0;
 * 1 <= ring_size <= 2048; band >= 1; page_size must be 16.  tau < 0 disables
 * every hit.  sm_scale == 0 selects 1/sqrt(head_dim). */
typedef struct {
    int32_t batch;          /* B: requests decoded together */
    int32_t num_q_heads;    /* Hq */
    int32_t num_kv_heads;   /* Hkv; query head h reads KV head h / (Hq/Hkv) */
    int32_t head_dim;       /* d */
    int32_t ring_size;      /* W: recent queries kept per (request, query head) */
    int32_t band;           /* r: band width removed by amend */
    float tau;              /* relative-L2 threshold: hit iff ||q~ - q~_p|| <= tau ||q~|| */
    float rope_theta;       /* RoPE base (rotate-half), e.g. 500000 */
    float sm_scale;         /* softmax scale on <q, k>; 0 -> 1/sqrt(d) */
    int32_t layout;         /* mac_kv_layout */
    int32_t kv_dtype;       /* mac_dtype of the cache */
    int32_t page_size;      /* tokens per page (16) */
    int32_t max_seq_len;    /* token capacity per request (multiple of page_size) */
    uint32_t flags;         /* MAC_F_* */
    /* NULL, or host array [num_q_heads] of per-head bands r_h >= 1 (Figure
     * 3 (b): the band size varies by head); query head h of every request
     * then uses r_h for its hit span [p - r_h + 1, m] and its amend band, and
     * `band` is ignored.  Read by mac_init, mac_config_validate and
     * mac_aux_bytes only (copied; the caller may free it afterwards).  With
     * MAC_F_FUSED_AMEND the heads of one KV group must share a band
     * (MAC_EUNSUPPORTED otherwise). */
    const int32_t *band_per_head;
} mac_config;

/* Borrowed view of one layer's KV cache (host struct; pointed-to memory is
 * device memory owned by the caller).
 *  contiguous: k, v are [B][Hkv][max_seq_len][d]
 *  paged:      k, v are [num_pages][Hkv][page_size][d]; request b's token t
 *              lives in page page_table[b*max_pages_per_req + t/page_size],
 *              row t%page_size.  Keys are stored post-RoPE. */
typedef struct {
    void *k;
    void *v;
    const int32_t *page_table;   /* paged only: [B][max_pages_per_req] */
    int32_t max_pages_per_req;   /* paged only */
    int32_t num_pages;           /* paged only */
    const int32_t *seq_lens;     /* [B]; <= 0 marks an idle request */
} mac_kv_view;

/* Counters since mac_init / mac_reset.  Byte counts are the algorithmic bytes
 * of key/value rows streamed (each key row and value row counted once). */
typedef struct {
    uint64_t steps;              /* decode steps run (counted on the device: graph replays included) */
    uint64_t decisions;          /* (request, head) decisions taken by match */
    uint64_t hits;
    uint64_t misses;
    uint64_t near_tau;           /* decisions whose relative distance lies within 1e-4 of tau */
    uint64_t override_invalid;   /* forced hits naming no stored position (taken as misses) */
    uint64_t kv_tokens_critical; /* keys streamed by complete, summed over KV groups */
    uint64_t kv_tokens_amend;    /* keys re-read by amend */
    uint64_t kv_bytes_critical;
    uint64_t kv_bytes_amend;
    uint64_t aux_bytes;          /* device memory owned by the handle */
    uint64_t bad_input;          /* device-side index checks that idled a request or row */
    float last_us_match;         /* MAC_F_TIMING: last step, microseconds */
    float last_us_complete;
    float last_us_reduce;        /* combine of the partial summaries + merge with the stored one */
    float last_us_amend;
    float last_us_attention;     /* match + complete + reduce, one event pair */
    uint64_t prefill_tokens;     /* prompt tokens taken by mac_prefill */
    uint64_t prefill_decisions;  /* their (token, query head) decisions */
    uint64_t prefill_hits;
    uint64_t prefill_kv_tokens;  /* keys attended, per KV group and prompt token */
    uint64_t prefill_override_invalid;
    uint64_t complete_waves;     /* waves of the complete kernel's persistent grid (the plan's workers) */
} mac_stats_t;

/* Check a configuration without touching the GPU (host only). */
mac_status mac_config_validate(const mac_config *cfg /* host */);

/* An upper bound of the device bytes mac_init allocates for cfg on a device
 * with num_cu compute units: it counts 8 resident blocks of the complete
 * kernel per CU, where mac_init sizes the per-wave partials for the blocks
 * that actually fit (2 or 3).  Host only; 0 for an invalid cfg. */
size_t mac_aux_bytes(const mac_config *cfg /* host */, int32_t num_cu);

/* Create a handle: validate cfg, allocate the rings, summaries and work
 * buffers on the current device, and take main_stream as the default stream.
 * amend_stream NULL creates a stream of default priority owned by the handle.
 * Rings start empty (the first decode call misses everywhere). */
mac_status mac_init(const mac_config *cfg /* host */, void *main_stream, void *amend_stream,
                    mac_handle *out /* host */);

/* Free everything mac_init allocated.  Synchronises the handle's streams and
 * waits for the last call's work on the stream it ran on (unless that stream
 * was being captured). */
mac_status mac_destroy(mac_handle h);

/* Empty every ring and zero the counters (asynchronous on the main stream,
 * ordered after pending amend work). */
mac_status mac_reset(mac_handle h);

/* Write this step's post-RoPE key and value rows into the cache: k_new and
 * v_new are [B][Hkv][d] in the cache dtype; request b's rows go to position
 * positions[b] (< 0: skipped).  The KV manager's job; the pages say the method
 * composes with paged KV managers (abstract). */
mac_status mac_append_kv(mac_handle h, const mac_kv_view *kv /* host */, const void *k_new,
                         const void *v_new, const int32_t *positions, void *stream);

/* One MAC decode step (Figure 2): q_pre_rope is [B][Hq][d] fp32 pre-RoPE
 * queries, out receives [B][Hq][d] fp32 attention outputs.  override_pos is
 * NULL or [B][Hq] int32: -2 no override, -1 force a miss, p >= 0 force a hit
 * on the ring entry stored at position p (a counted miss when absent).
 * Waits on the previous step's amend (with MAC_F_STALE_RING, on the amend of
 * the step before it); enqueues match, complete and the
 * reduce/merge on `stream`, then amend on the amend stream (or on `stream`
 * with MAC_F_SYNC_AMEND; with MAC_F_FUSED_AMEND the reduce does the ring
 * update and no amend is enqueued).  On an amend stream the handle created
 * (amend_stream NULL at mac_init), a thread of the handle launches that amend
 * once it sees (blocking on the host) that the call's reduce has run, so the
 * call returns once the reduce is enqueued; the handle's next call (and
 * mac_stats, mac_reset, mac_debug_last, mac_prefill, mac_destroy) first waits
 * until that thread has launched it, and reports a HIP error it met there.
 * When a call finds that thread still waiting (the GPU is behind the host,
 * calls of one handle back to back), the following calls enqueue their amend
 * on `stream` after the reduce, until a call finds the GPU caught up with the
 * previous one; the results are the same bits either way.
 * When the amend stream was supplied to
 * mac_init (layers may share it), the complete kernel also waits for all work
 * queued on it before it: complete gives every wave of a full-occupancy grid
 * an equal share, and a kernel still resident when it starts would delay some
 * of its waves.  The library copies what amend needs, so the caller
 * may reuse q_pre_rope, out and seq_lens as soon as the step's work on
 * `stream` has run.  The ring slot a call writes comes from a call counter
 * kept on the device (mac_stats' steps), so with MAC_F_FUSED_AMEND or
 * MAC_F_SYNC_AMEND (and without MAC_F_STALE_RING or MAC_F_TIMING) a call
 * enqueues only kernels whose arguments do not change from call to call: the
 * caller may capture append + decode on one stream into a HIP graph and
 * replay it, updating the positions, seq_lens and query buffers in place
 * between replays (warm up and capture on the same stream).  The default
 * form orders the amend stream with events chosen per call on the host, the
 * stale-by-one ring alternates its buffers per call on the host, and
 * MAC_F_TIMING records events per kernel: on a stream being captured these
 * return MAC_EUNSUPPORTED before enqueuing anything, and the handle stays
 * usable.  The handle's amend thread makes no call on a captured stream; it
 * runs in the relaxed capture mode, so a capture elsewhere in the process
 * does not stop it. */
mac_status mac_decode_step(mac_handle h, const mac_kv_view *kv /* host */,
                           const float *q_pre_rope, float *out, const int32_t *override_pos,
                           void *stream);

/* MAC-Attention over the prompt, the pages' Table 8 ablation (reuse in
 * prefill as well as decode, window unbounded).  Request b's prompt tokens
 * t = 0 .. seq_lens[b]-1, whose post-RoPE keys and values are already in the
 * cache, are taken as decode steps in order: token t matches the pre-RoPE
 * queries of every earlier prompt token of its (request, query head), with
 * the handle's tau, bands and scale, and on a hit at p attends only
 * [p - r_h + 1, t] merged with the summary token p stored.  The decode rings
 * are neither read nor written, and ring_size does not apply.
 *   q_pre:        [B][num_tokens][Hq][d] fp32 pre-RoPE queries (16-byte aligned)
 *   out:          [B][num_tokens][Hq][d] fp32 outputs; rows t >= seq_lens[b] get zeros
 *   override_pos: NULL or [B][num_tokens][Hq] int32 (-2 none, -1 miss, p >= 0 hit
 *                 on earlier token p; p >= t is a counted miss)
 *   p_out:        NULL or [B][num_tokens][Hq] int32 device: matched position or -1
 * 1 <= num_tokens <= 32768; a seq_lens[b] beyond num_tokens or the cache idles
 * request b (counted in bad_input).  Honours MAC_F_DISABLE_REUSE (plain
 * causal attention) and MAC_F_RING_BF16 (earlier queries rounded to bf16
 * for the match); the other flags do not apply.  Enqueued on `stream` (NULL:
 * the main stream); its scratch ((5 d + 20) * 4 = 2640 bytes per (request,
 * token, query head)) is allocated and released stream-ordered on that stream (MAC_ENOMEM
 * if that fails).  Counters: mac_stats' prefill_* fields. */
mac_status mac_prefill(mac_handle h, const mac_kv_view *kv /* host */, int32_t num_tokens,
                       const float *q_pre, float *out, const int32_t *override_pos,
                       int32_t *p_out, void *stream);

/* mac_prefill for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation): the
 * same operation, arguments, results and counters, but the scratch lives in
 * a static device array of 64 MiB per GPU, held by the library until the
 * process ends, and the call allocates and frees nothing.  The scratch takes
 * (5 d + 20) * 4 = 2640 bytes per (request, token, query head): calls whose
 * batch * num_tokens * num_q_heads rows need more than 64 MiB (25,420 rows,
 * e.g. 1 x 780 x 32) return MAC_EINVAL before any GPU work.  Every call on a
 * GPU, from any handle, shares that GPU's array: calls that may overlap on
 * one GPU (other streams, other host threads) race and must be ordered by
 * the caller. */
mac_status mac_prefill_noalloc(mac_handle h, const mac_kv_view *kv /* host */, int32_t num_tokens,
                               const float *q_pre, float *out, const int32_t *override_pos,
                               int32_t *p_out, void *stream);

/* Synchronise the handle's streams and copy the counters (host). */
mac_status mac_stats(mac_handle h, mac_stats_t *out /* host */);

/* MAC_F_RECORD_DEBUG only: synchronise and copy the last step's per-head
 * matched position (-1 on a miss), hit flag and relative distance of the
 * nearest entry (NaN when the ring held none); each [B][Hq] host arrays, any
 * may be NULL. */
mac_status mac_debug_last(mac_handle h, int32_t *p /* host */, uint8_t *hit /* host */,
                          float *rel /* host */);

/* Message for the handle's last failed call ("" if none); h NULL gives the
 * message of the last failed mac_init or validation on this thread. */
const char *mac_last_error(mac_handle h);

const char *mac_status_string(mac_status s);

#ifdef __cplusplus
}
#endif

#endif /* MAC_H */
