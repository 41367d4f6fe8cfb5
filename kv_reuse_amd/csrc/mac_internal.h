// mac_internal.h -- state layout and kernel launch interface shared by the
// host runtime (mac_runtime.cpp) and the gfx950 kernels (match.hip,
// complete.hip, reduce.hip, amend.hip, prefill.hip).
//
// Device memory owned by a handle (fp32 unless noted):
//   ring_q     [B][Hq][W][D]        pre-RoPE queries of recent steps (fp32, or
//                                   bf16 bit patterns with MAC_F_RING_BF16)
//   ring_s     [B][Hq][W][SUMM]     summaries AS_{1:pos-r}: o[D], M, l, pad
//   ring_pos   [B][W]  int32        position stored in each slot (-1 empty)
//   q_copy     [B][Hq][D]           this step's pre-RoPE queries (for amend)
//   q_rot      [B][Hq][D]           this step's post-RoPE queries
//   m_buf      [B]     int32        this step's query position (-1 idle)
//   step_slot  [1]     int32        the ring slot this step writes (set by match)
//   dec_slot   [B][Hq] int32        matched slot (-1 miss)
//   dec_p      [B][Hq] int32        matched position (-1 miss)
//   dec_start  [B][Hq] int32        first key of the head's span
//   dec_rel    [B][Hq]              relative distance of the nearest entry
//   tile_best  [B][Hq][W/64][3]     W > 64, few heads: nearest entry of each 64-slot tile
//   grp_parts  [B][Hkv][nseg][2] int32  first and last worker whose partial covers a segment
//   partials   [NW + B*Hkv*nseg][G][SUMM] per-(worker, segment) unnormalised summaries
//   as_full    [B][Hq][SUMM]        AS_{1:m} of this step, input of amend
//   band       [Hq]    int32        band r_h of each query head
//   stats      [MAC_NSTAT] + [B*Hq][HEAD_NSTAT] + [B*Hkv][GRP_NSTAT] uint64 counters
// With the stale-by-one ring (MAC_F_STALE_RING) q_copy, q_rot, m_buf,
// step_slot and as_full are held twice and calls alternate between the copies, so that the
// amend of call t-1, still running, reads its own while call t writes the
// other.
// A group's union span (the keys complete streams for it) starts at the
// smallest first key of its heads' spans; the plan derives it from dec_start.
// The work list is cut into segments: one per group, or with fused amend two
// (the span up to m - r, then the band [m - r + 1, m]).
// M values inside the library are in log2 units of the scaled logit
// (s * log2 e); every summary the library stores uses the same units.
#pragma once
#include <cstdint>
#include <hip/hip_runtime.h>

namespace mac {

constexpr int D = 128;          // head_dim supported by the kernels
constexpr int SUMM = D + 4;     // o[D], M, l, 2 pad floats (16-byte rows)
constexpr int PAGE = 16;        // tokens per page
constexpr int BLOCK = 256;      // threads per workgroup (4 waves of 64)
constexpr int WAVES = BLOCK / 64;
constexpr int MAX_W = 2048;     // ring slots per (request, head)
constexpr int TILE_W = 64;      // longest ring one match wave holds whole (longer: several waves)
constexpr int MAX_GROUPS = 4096;  // B * Hkv
constexpr int MIN_PAGES_PER_WORKER = 1;

// Counters, one uint64 block: MAC_NSTAT device-wide ones (by atomics: bad
// input on error paths, the prefill's counts once per block), then
// HEAD_NSTAT per (request, query head), written without atomics by the match
// wave that owns the head, then GRP_NSTAT per (request, KV group): keys
// streamed by complete (written by block 0 of the complete grid) and re-read
// by amend (written by the amend block of the group).  The host sums them.
enum GlobalStat {
    ST_BAD_INPUT = 0,
    ST_PF_TOKENS,        // prompt tokens taken by the prefill
    ST_PF_DECISIONS,     // their (token, head) decisions
    ST_PF_HITS,
    ST_PF_KV,            // keys attended per (KV group, token)
    ST_PF_OVR_INVALID,   // prefill overrides naming no earlier token
    ST_STEPS,            // decode calls: match takes the ring slot (ST_STEPS mod W) and advances it
    MAC_NSTAT = 8
};
enum HeadStat { HS_HITS = 0, HS_MISSES, HS_NEAR_TAU, HS_OVR_INVALID, HEAD_NSTAT };
enum GroupStat { GS_TOK_CRIT = 0, GS_TOK_AMEND, GRP_NSTAT };
inline long stats_count(long n_heads, long n_groups)
{
    return MAC_NSTAT + n_heads * HEAD_NSTAT + n_groups * GRP_NSTAT;
}

struct KvView {
    void *k;
    void *v;
    const int32_t *page_table;
    int32_t max_pages;      // pages per request (paged) -- bound of page_table rows
    int32_t num_pages;      // paged: pages in the pool
    int32_t max_seq_len;    // contiguous: row stride in tokens; both: token bound
    int32_t paged;
};

struct Shape {
    int32_t B, Hq, Hkv, G, W;
    float tau, scale_log2;  // scale_log2 = sm_scale * log2(e)
    int32_t reuse;          // 0: every head misses
    int32_t nseg;           // work-list segments per group: 1, or 2 when amend is fused
    int32_t ring_bf16;      // ring queries stored as bf16 (rounded to nearest, ties to even)
    int32_t unbalanced;     // plan: the same number of waves per segment (measurement baseline)
    int32_t plan_bounds;    // the complete kernel's LDS plan also keeps each segment's first
                            // key and each request's position (small work lists)
};

struct State {
    void *ring_q;             // float, or uint16_t (bf16) when Shape::ring_bf16
    float *ring_s, *q_copy, *q_rot, *partials, *as_full, *dec_rel;
    int32_t *ring_pos, *m_buf, *dec_slot, *dec_p, *dec_start;
    int32_t *step_slot;       // [1] ring slot of this step (match -> reduce, amend)
    int32_t *grp_parts;       // [B*Hkv*nseg][2] worker range of each segment's partials (complete -> reduce)
    unsigned long long *stats;        // [MAC_NSTAT], then the two blocks below
    unsigned long long *head_stats;   // [B*Hq][HEAD_NSTAT]
    unsigned long long *grp_stats;    // [B*Hkv][GRP_NSTAT]
    const double *inv_freq;   // [D/2] theta^(-2i/D), fp64
    const int32_t *band;      // [Hq] band r_h of each query head
    float *tile_best;         // W > TILE_W: [B*Hq][ceil(W/TILE_W)][3] per-tile nearest (D, pos, slot)
    int32_t n_workers;        // waves in the complete grid
    int32_t slots;            // blocks of the complete grid per CU (dispatch rounds)
};

// Launchers (enqueue only; return the launch status).
// `hidden` is a ring slot this call's match and override ignore (-1: none).
hipError_t launch_match(const Shape &s, const State &st, const KvView &kv, const int32_t *seq_lens,
                        const float *q_pre, const int32_t *override_pos, float *out, int hidden,
                        hipStream_t stream);
hipError_t launch_complete(const Shape &s, const State &st, const KvView &kv, bool kv_fp32,
                           int n_blocks, hipStream_t stream);
// reduce (fused amend) and amend write the ring slot match chose (step_slot).
hipError_t launch_reduce(const Shape &s, const State &st, float *out, hipStream_t stream);
hipError_t launch_amend(const Shape &s, const State &st, const KvView &kv, bool kv_fp32,
                        hipStream_t stream);
hipError_t launch_append(const Shape &s, const State &st, const KvView &kv, bool kv_fp32,
                         const void *k_new, const void *v_new, const int32_t *positions,
                         hipStream_t stream);
hipError_t launch_reset(const Shape &s, const State &st, hipStream_t stream);
// MAC over the prompt (seq_lens[b] tokens of request b, N rows each) with an
// unbounded window; scratch holds prefill_scratch_bytes(s, N) bytes.
size_t prefill_scratch_bytes(const Shape &s, int N);
hipError_t launch_prefill(const Shape &s, const State &st, const KvView &kv, bool kv_fp32,
                          const int32_t *seq_lens, int N, const float *q_pre, float *out,
                          const int32_t *override_pos, int32_t *p_out, void *scratch,
                          hipStream_t stream);
// Allocation-free prefill: a static device array of PREFILL_STATIC_BYTES per
// GPU.  prefill_static_scratch_init takes its address on `device` (which must
// be current), once; prefill_static_scratch returns it (null before init).
constexpr size_t PREFILL_STATIC_BYTES = size_t(64) << 20;
hipError_t prefill_static_scratch_init(int device);
void *prefill_static_scratch(int device);
// Workgroups of the complete kernel resident per CU (occupancy query).
int complete_blocks_per_cu(bool kv_fp32, int G, size_t plan_lds_bytes);
bool supported_group(int G);

}  // namespace mac
