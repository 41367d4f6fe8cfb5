// match.hip -- match step of the MAC-Attention decode (Figure 2 (a)): pre-RoPE
// L2 nearest neighbour over each (request, query head) ring, relative-L2
// threshold, RoPE of the query, and each head's key span.
#include "mac_device.h"

namespace mac {
namespace {

// Sum over each 32-lane half of the wave (DPP inside rows, ds_swizzle across
// the two rows of a half).
__device__ __forceinline__ float half_sum(float v)
{
    v = row16_sum(v);
    v += xor_lanes<16>(v);
    return v;
}

// Nearest-entry order: smaller distance, then newer position, then larger slot.
__device__ __forceinline__ bool nearer(float d2, int p2, int j2, float d, int p, int j)
{
    return d2 < d || (d2 == d && (p2 > p || (p2 == p && j2 > j)));
}

// Valid entry stamps are positions 0 <= pos <= m (the ring holds only earlier
// steps of this request); m = seq_len - 1, or -1 for an idle or bad request.
__device__ __forceinline__ int query_position(const KvView &kv, int seq, bool &bad)
{
    int m = seq - 1;
    bad = m >= 0 && (m >= kv.max_seq_len || (kv.paged && m / PAGE >= kv.max_pages));
    return bad ? -1 : m;
}

// One wave holds up to SLOTS (16, 32 or 64) ring slots of one head in
// registers, loaded in a single round: with fp32 queries each 1 KB wave load
// covers two slots (lanes 0-31 and 32-63, four columns each), with bf16
// queries four (lanes 16j .. 16j+15 hold one slot, eight columns each).  Slots
// past nslot are not loaded (zero).  The loads do not depend on the query position,
// so the match kernel issues them with its other loads.
template <int SLOTS, bool BF16>
struct RingTile {
    static constexpr int PER = BF16 ? 4 : 2;   // slots per wave load
    static constexpr int NL = SLOTS / PER;
    using Vec = typename std::conditional<BF16, uint4, float4>::type;
    Vec v[NL];

    // slots [base, base + nslot) of head idx.  ALL: every load is issued, a
    // slot past nslot re-reading the last valid slot's row (scan ignores it):
    // for loads kept in flight across later work, since loads under a branch
    // leave the compiler unable to count a wave's loads in flight, and every
    // later wait is then for all of them.  Otherwise such slots are zero.
    template <bool ALL = false>
    __device__ __forceinline__ void load(const Shape &s, const State &st, long idx, int base,
                                         int nslot)
    {
        const int lane = lane_id();
        const long row = (idx * s.W + base) * D;
        const int sub = lane / (64 / PER), c = lane % (64 / PER);
        const Vec *rq = BF16 ? reinterpret_cast<const Vec *>(
                                   static_cast<const uint16_t *>(st.ring_q) + row)
                             : reinterpret_cast<const Vec *>(
                                   static_cast<const float *>(st.ring_q) + row);
        constexpr int VPR = BF16 ? D / 8 : D / 4;   // vectors per slot
#pragma unroll
        for (int u = 0; u < NL; ++u) {
            const int sl = PER * u + sub;
            if (ALL || sl < nslot) {
                // read once per step: streaming hint
                const uint4 t = load_stream(rq + (long)(ALL ? min(sl, nslot - 1) : sl) * VPR + c);
                v[u] = *reinterpret_cast<const Vec *>(&t);
            } else {
                v[u] = Vec{};
            }
        }
    }

    // Nearest valid entry of the loaded slots (wave-uniform result): squared
    // L2 distance to the pre-RoPE query qsrc, summed over each slot's lanes;
    // pos_l is the stamp of slot base + lane; valid stamps are 0 .. m.
    // The query columns this lane compares (4 for fp32 slots, 8 for bf16).
    __device__ __forceinline__ static void load_query(const float *qsrc, float (&q)[8])
    {
        const int c = lane_id() % (64 / PER);
        if constexpr (BF16) {
            const float4 a = reinterpret_cast<const float4 *>(qsrc)[2 * c];
            const float4 b = reinterpret_cast<const float4 *>(qsrc)[2 * c + 1];
            q[0] = a.x, q[1] = a.y, q[2] = a.z, q[3] = a.w;
            q[4] = b.x, q[5] = b.y, q[6] = b.z, q[7] = b.w;
        } else {
            const float4 a = reinterpret_cast<const float4 *>(qsrc)[c];
            q[0] = a.x, q[1] = a.y, q[2] = a.z, q[3] = a.w;
            q[4] = q[5] = q[6] = q[7] = 0.f;
        }
    }

    __device__ __forceinline__ void scan(const float *qsrc, int base, int nslot, int pos_l, int m,
                                         float &kd, int &kp, int &kj) const
    {
        float q[8];
        load_query(qsrc, q);
        scan(q, base, nslot, pos_l, m, kd, kp, kj);
    }

    // The same with the lane's query columns already in registers (q).
    __device__ __forceinline__ void scan(const float (&q)[8], int base, int nslot, int pos_l,
                                         int m, float &kd, int &kp, int &kj) const
    {
        const int lane = lane_id();
        const int sub = lane / (64 / PER);
        kd = INFINITY;
        kp = INT_MIN;
        kj = -1;
#pragma unroll
        for (int u = 0; u < NL; ++u) {
            const int sl = PER * u + sub;
            float d = 0.f;
            if constexpr (BF16) {
                float f[8];
                to_f32(v[u], f);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float t = q[e] - f[e];
                    d = fmaf(t, t, d);
                }
                d = row16_sum(d);
            } else {
                const float t0 = q[0] - v[u].x, t1 = q[1] - v[u].y, t2 = q[2] - v[u].z,
                            t3 = q[3] - v[u].w;
                d = t0 * t0;
                d = fmaf(t1, t1, d);
                d = fmaf(t2, t2, d);
                d = fmaf(t3, t3, d);
                d = half_sum(d);
            }
            // the slots' stamps by wave-uniform lane reads (no LDS round trip),
            // then each lane group takes its own slot's
            int pos = __builtin_amdgcn_readlane(pos_l, PER * u);
#pragma unroll
            for (int g = 1; g < PER; ++g) {
                const int pg = __builtin_amdgcn_readlane(pos_l, PER * u + g);
                pos = sub == g ? pg : pos;
            }
            const bool valid = sl < nslot && pos >= 0 && pos <= m;
            if (valid && nearer(d, pos, base + sl, kd, kp, kj)) {
                kd = d;
                kp = pos;
                kj = base + sl;
            }
        }
        // the lane groups saw different slots
        if constexpr (BF16) {
            const float d2 = xor_lanes<16>(kd);
            const int p2 = xor_lanes_i<16>(kp);
            const int j2 = xor_lanes_i<16>(kj);
            if (nearer(d2, p2, j2, kd, kp, kj)) {
                kd = d2;
                kp = p2;
                kj = j2;
            }
        }
        const float d2 = xor_lanes<32>(kd);
        const int p2 = xor_lanes_i<32>(kp);
        const int j2 = xor_lanes_i<32>(kj);
        if (nearer(d2, p2, j2, kd, kp, kj)) {
            kd = d2;
            kp = p2;
            kj = j2;
        }
    }
};

// ================================================================== match
// The head's decision is taken by one wave once the nearest valid ring entry
// is known; the kernels below differ in how they find it.  The match step is
// latency-bound, so the one-wave kernel issues every load that does not depend
// on the query position (query, angles, ring, stamps, override, the head's
// counters) before it waits on any of them.  The head then takes its decision (hit iff the relative L2 distance of the nearest valid entry is
// within tau, compared squared), applies an override, rotates its query
// (rotate-half RoPE, angle in fp64) and records its key span:
// [max(p - r + 1, 0), m] on a hit, [0, m] on a miss.

// The head's inputs other than the ring, loaded by the deciding wave.
struct HeadIn {
    float qa, qb;      // pre-RoPE query, elements lane and lane + 64
    float q2;          // |q|^2 (head_norm2), read by decide
    double inv;        // inverse frequency of the lane's rotation pair
    int ov, band, pos_l;
    unsigned long long old[HEAD_NSTAT];
};

__device__ __forceinline__ void load_head(const Shape &s, const State &st, const float *q_pre,
                                          const int32_t *ovr, int b, int h, int hidden,
                                          HeadIn &in)
{
    const long idx = (long)b * s.Hq + h;
    const int lane = lane_id();
    in.qa = q_pre[idx * D + lane];
    in.qb = q_pre[idx * D + lane + 64];
    in.inv = st.inv_freq[lane];
    in.ov = ovr ? ovr[idx] : -2;
    in.band = st.band[h];
    in.pos_l = (s.reuse && lane < s.W && lane != hidden) ? st.ring_pos[(long)b * s.W + lane] : -1;
#pragma unroll
    for (int k = 0; k < HEAD_NSTAT; ++k)
        in.old[k] = 0;
    if (lane == 0) {
        const unsigned long long *hstat = st.head_stats + idx * HEAD_NSTAT;
#pragma unroll
        for (int k = 0; k < HEAD_NSTAT; ++k)
            in.old[k] = hstat[k];
    }
}

// |q|^2 of the pre-RoPE query, wave-uniform.
__device__ __forceinline__ void head_norm2(HeadIn &in)
{
    in.q2 = wave_sum(in.qa * in.qa + in.qb * in.qb);
}

// This step's query copies: pre-RoPE (for amend) and rotated (for complete);
// an idle request's output is zero (no group of it gets work).
__device__ __forceinline__ void store_queries(const State &st, long idx, int m, const HeadIn &in,
                                              float *out)
{
    const int lane = lane_id();
    if (m >= 0) {
        st.q_copy[idx * D + lane] = in.qa;
        st.q_copy[idx * D + lane + 64] = in.qb;
        float ra, rb;
        rope_pair(in.qa, in.qb, m, in.inv, ra, rb);
        st.q_rot[idx * D + lane] = ra;
        st.q_rot[idx * D + lane + 64] = rb;
    } else {
        out[idx * D + lane] = 0.f;
        out[idx * D + lane + 64] = 0.f;
    }
}

// The decision from the nearest valid entry (kd, kp, kj; kp < 0: none), the
// override, the span and the counters; one wave.
__device__ __forceinline__ void decide(const Shape &s, const State &st, int b, int h, int m,
                                       bool bad, const HeadIn &in, float kd, int kp, int kj,
                                       int hidden)
{
    const long idx = (long)b * s.Hq + h;
    const int lane = lane_id();
    int slot = -1, p = -1, start = 0;
    float rel = NAN;
    int cnt[HEAD_NSTAT] = {0, 0, 0, 0};
    const bool act = m >= 0;
    if (act && s.reuse) {
        const float q2 = in.q2;
        if (kp >= 0) {
            rel = q2 > 0.f ? sqrtf(kd / q2) : (kd == 0.f ? 0.f : INFINITY);
            // relative-L2 test compared squared: D <= tau^2 |q~|^2
            if (s.tau >= 0.f && kd <= s.tau * s.tau * q2) {
                slot = kj;
                p = kp;
            }
            if (fabsf(rel - s.tau) < 1e-4f)
                cnt[HS_NEAR_TAU] = 1;
        }
        if (in.ov != -2) {
            slot = -1;
            p = -1;
            if (in.ov >= 0) {
                // the largest slot holding position ov, 64 slots at a time
                for (int c0 = 0; c0 < s.W; c0 += 64) {
                    const int sl = c0 + lane;
                    const int ps = c0 == 0 ? in.pos_l
                                           : (sl < s.W ? st.ring_pos[(long)b * s.W + sl] : -1);
                    const bool mine = sl < s.W && sl != hidden && in.ov <= m && ps == in.ov;
                    const unsigned long long bal = __ballot(mine);
                    if (bal) {
                        slot = c0 + 63 - __clzll(bal);
                        p = in.ov;
                    }
                }
                if (slot < 0)
                    cnt[HS_OVR_INVALID] = 1;
            }
        }
        if (slot >= 0)
            start = max(p - in.band + 1, 0);
    }
    if (lane == 0) {
        st.dec_slot[idx] = slot;
        st.dec_p[idx] = p;
        st.dec_start[idx] = start;
        st.dec_rel[idx] = rel;
        if (act) {
            // this wave owns the head's counters: no atomics
            cnt[slot >= 0 ? HS_HITS : HS_MISSES] = 1;
            unsigned long long *hstat = st.head_stats + idx * HEAD_NSTAT;
#pragma unroll
            for (int k = 0; k < HEAD_NSTAT; ++k)
                hstat[k] = in.old[k] + (unsigned long long)cnt[k];
        }
        if (h == 0 && b == 0) {
            // the ring slot of this call, from the device's own call count (so a
            // captured step replays correctly): slot = calls mod W
            const unsigned long long c = st.stats[ST_STEPS];
            *st.step_slot = (int)(c % (unsigned long long)s.W);
            st.stats[ST_STEPS] = c + 1;
        }
        if (h == 0) {
            st.m_buf[b] = m;
            if (bad)
                atomicAdd(&st.stats[ST_BAD_INPUT], 1ULL);
        }
    }
}

// Rings of up to 64 entries: one wave, the whole ring in registers
// (RingTile), loaded with the head's other inputs.
template <int SLOTS, bool BF16>
__global__ __launch_bounds__(64) void match_kernel(Shape s, State st, KvView kv,
                                                   const int32_t *__restrict__ seq_lens,
                                                   const float *__restrict__ q_pre,
                                                   const int32_t *__restrict__ ovr,
                                                   float *__restrict__ out, int hidden)
{
    const int h = blockIdx.x, b = blockIdx.y;
    const long idx = (long)b * s.Hq + h;
    RingTile<SLOTS, BF16> ring;
    if (s.reuse)
        ring.load(s, st, idx, 0, s.W);
    const int seq = seq_lens[b];
    HeadIn in;
    load_head(s, st, q_pre, ovr, b, h, hidden, in);
    bool bad;
    const int m = query_position(kv, seq, bad);
    store_queries(st, idx, m, in, out);
    float kd = INFINITY;
    int kp = INT_MIN, kj = -1;
    if (m >= 0 && s.reuse)
        ring.scan(q_pre + idx * D, 0, s.W, in.pos_l, m, kd, kp, kj);
    head_norm2(in);
    decide(s, st, b, h, m, bad, in, kd, kp, kj, hidden);
}

// Rings longer than one 64-slot tile, few heads (too few to give every CU a
// block of the one-launch kernel below): grid (tiles, Hq, B), one wave per
// 64-slot tile loads the tile's pre-RoPE queries (32 KB fp32, 16 KB bf16) and
// records the tile's nearest entry; match_tiled_kernel then reduces the
// tiles of each head.
template <bool BF16>
__global__ __launch_bounds__(64) void match_tiles_kernel(Shape s, State st, KvView kv,
                                                         const int32_t *__restrict__ seq_lens,
                                                         const float *__restrict__ q_pre,
                                                         int hidden)
{
    const int tile = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int ntiles = (s.W + TILE_W - 1) / TILE_W;
    const long idx = (long)b * s.Hq + h;
    const int lane = lane_id();
    const int base = tile * TILE_W;
    const int nslot = min(TILE_W, s.W - base);
    RingTile<TILE_W, BF16> ring;
    ring.load(s, st, idx, base, nslot);
    const int seq = seq_lens[b];
    const int pos_l = (lane < nslot && base + lane != hidden)
                          ? st.ring_pos[(long)b * s.W + base + lane]
                          : -1;
    bool bad;
    const int m = query_position(kv, seq, bad);
    float kd;
    int kp, kj;
    ring.scan(q_pre + idx * D, base, nslot, pos_l, m, kd, kp, kj);
    if (lane == 0) {
        float *o = st.tile_best + (idx * ntiles + tile) * 3;
        o[0] = kd;
        o[1] = __int_as_float(kp);
        o[2] = __int_as_float(kj);
    }
}

template <int OFF>
__device__ __forceinline__ void argmin_step(float &kd, int &kp, int &kj)
{
    const float d2 = xor_lanes<OFF>(kd);
    const int p2 = xor_lanes_i<OFF>(kp);
    const int j2 = xor_lanes_i<OFF>(kj);
    if (nearer(d2, p2, j2, kd, kp, kj)) {
        kd = d2;
        kp = p2;
        kj = j2;
    }
}

// One wave per head: the nearest of the head's tile entries (lane t holds
// tile t's), then the decision.
__global__ __launch_bounds__(64) void match_tiled_kernel(Shape s, State st, KvView kv,
                                                         const int32_t *__restrict__ seq_lens,
                                                         const float *__restrict__ q_pre,
                                                         const int32_t *__restrict__ ovr,
                                                         float *__restrict__ out, int hidden)
{
    const int h = blockIdx.x, b = blockIdx.y;
    const long idx = (long)b * s.Hq + h;
    const int lane = lane_id();
    const int ntiles = (s.W + TILE_W - 1) / TILE_W;
    float kd = INFINITY;
    int kp = INT_MIN, kj = -1;
    if (s.reuse && lane < ntiles) {
        const float *tb = st.tile_best + (idx * ntiles + lane) * 3;
        kd = tb[0];
        kp = __float_as_int(tb[1]);
        kj = __float_as_int(tb[2]);
    }
    const int seq = seq_lens[b];
    HeadIn in;
    load_head(s, st, q_pre, ovr, b, h, hidden, in);
    bool bad;
    const int m = query_position(kv, seq, bad);
    store_queries(st, idx, m, in, out);
    argmin_step<1>(kd, kp, kj);
    argmin_step<2>(kd, kp, kj);
    argmin_step<4>(kd, kp, kj);
    argmin_step<8>(kd, kp, kj);
    argmin_step<16>(kd, kp, kj);
    argmin_step<32>(kd, kp, kj);
    if (m < 0)
        kp = INT_MIN;
    head_norm2(in);
    decide(s, st, b, h, m, bad, in, kd, kp, kj, hidden);
}

// Longer rings (the pages' windows of 512-2048 entries, Figure 6, Tables 5
// and 7) with enough heads for two blocks per CU: up to MATCH_WAVES waves per
// head, wave w scanning sub-tiles w, w + waves, ... of SUB = 16 slots (in
// RingTile's layouts, so each slot's distance is summed as in the one-wave
// kernel), two sub-tiles in flight per wave; the waves' nearest entries meet
// in LDS and wave 0 decides.  One launch streams the whole ring, and at <= 128
// registers two blocks share a CU, so one block's deciding wave overlaps the
// other's scan.
constexpr int MATCH_WAVES = 8;

template <bool BF16>
__global__ __launch_bounds__(64 * MATCH_WAVES) __attribute__((amdgpu_waves_per_eu(4))) void
match_wide_kernel(
    Shape s, State st, KvView kv, const int32_t *__restrict__ seq_lens,
    const float *__restrict__ q_pre, const int32_t *__restrict__ ovr, float *__restrict__ out,
    int hidden)
{
    constexpr int SUB = 16;
    __shared__ float s_d[MATCH_WAVES];
    __shared__ int s_p[MATCH_WAVES], s_j[MATCH_WAVES];
    const int h = blockIdx.x, b = blockIdx.y;
    const long idx = (long)b * s.Hq + h;
    // (wave index read as wave-uniform, so values set by wave 0 alone stay scalar)
    const int lane = lane_id(), wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nwv = blockDim.x >> 6;
    const int nsub = (s.W + SUB - 1) / SUB;
    const int seq = seq_lens[b];
    bool bad;
    const int m = query_position(kv, seq, bad);
    float kd = INFINITY;
    int kp = INT_MIN, kj = -1;
    // wave 0 (the deciding wave) loads the head's other inputs and stores the
    // query copies before its share of the scan, off the block's tail
    HeadIn in;
    float q2s = 0.f;
    int ov_s = -2, band_s = 0;
    unsigned old_s[2 * HEAD_NSTAT];
    if (wv == 0) {
        load_head(s, st, q_pre, ovr, b, h, hidden, in);
        store_queries(st, idx, m, in, out);
        head_norm2(in);
        // across the scan decide needs |q|^2, the override, the band and the
        // head's counters (wave-uniform: scalar registers) and the first 64
        // stamps (one register); the ring tiles keep the vector registers
        q2s = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(in.q2)));
        ov_s = __builtin_amdgcn_readfirstlane(in.ov);
        band_s = __builtin_amdgcn_readfirstlane(in.band);
#pragma unroll
        for (int k = 0; k < HEAD_NSTAT; ++k) {
            old_s[2 * k] = __builtin_amdgcn_readfirstlane((unsigned)in.old[k]);
            old_s[2 * k + 1] = __builtin_amdgcn_readfirstlane((unsigned)(in.old[k] >> 32));
        }
    }
    if (m >= 0 && s.reuse) {
        // two sub-tiles per wave in flight: the next one's loads are issued
        // before the current one is scanned
        RingTile<SUB, BF16> ring[2];
        int pos_l[2];
        // the query is read once, ahead of the ring: a query load issued
        // after the next sub-tile's would make each scan wait for that
        // sub-tile too (loads complete in order)
        float qv[8];
        RingTile<SUB, BF16>::load_query(q_pre + idx * D, qv);
        // (fetch issues the same loads whatever j is, so that a scan waits
        // only for its own sub-tile; the stamps are masked when scanned)
        auto fetch = [&](int k, int j) {
            const int base = j * SUB, nslot = min(SUB, s.W - base);
            ring[k].template load<true>(s, st, idx, base, nslot);
            pos_l[k] = st.ring_pos[(long)b * s.W + base + min(lane, nslot - 1)];
        };
        auto scan = [&](int k, int j) {
            const int base = j * SUB, nslot = min(SUB, s.W - base);
            const int pl = (lane < nslot && base + lane != hidden) ? pos_l[k] : -1;
            float d;
            int p, jj;
            ring[k].scan(qv, base, nslot, pl, m, d, p, jj);
            if (nearer(d, p, jj, kd, kp, kj)) {
                kd = d;
                kp = p;
                kj = jj;
            }
        };
        // this wave's sub-tiles: wv, wv + nwv, ... below nsub; the loop body
        // prefetches unconditionally, the last one or two are peeled
        int j = wv;
        const int cnt = j < nsub ? (nsub - 1 - j) / nwv + 1 : 0;
        if (cnt > 0) {
            fetch(0, j);
            int left = cnt - 1;   // sub-tiles not yet fetched
            while (left >= 2) {
                fetch(1, j + nwv);
                scan(0, j);
                j += nwv;
                fetch(0, j + nwv);
                scan(1, j);
                j += nwv;
                left -= 2;
            }
            if (left == 1) {
                fetch(1, j + nwv);
                scan(0, j);
                scan(1, j + nwv);
            } else {
                scan(0, j);
            }
        }
    }
    if (lane == 0) {
        s_d[wv] = kd;
        s_p[wv] = kp;
        s_j[wv] = kj;
    }
    __syncthreads();
    if (wv != 0)
        return;
    in.q2 = q2s;
    in.ov = ov_s;
    in.band = band_s;
#pragma unroll
    for (int k = 0; k < HEAD_NSTAT; ++k)
        in.old[k] = lane == 0 ? ((unsigned long long)old_s[2 * k + 1] << 32 | old_s[2 * k]) : 0ULL;
    // nearest over the waves (a strict total order: the result does not
    // depend on the order of the comparisons)
    for (int k = 1; k < nwv; ++k) {
        if (nearer(s_d[k], s_p[k], s_j[k], kd, kp, kj)) {
            kd = s_d[k];
            kp = s_p[k];
            kj = s_j[k];
        }
    }
    decide(s, st, b, h, m, bad, in, kd, kp, kj, hidden);
}

}  // namespace

hipError_t launch_match(const Shape &s, const State &st, const KvView &kv, const int32_t *seq_lens,
                        const float *q_pre, const int32_t *override_pos, float *out, int hidden,
                        hipStream_t stream)
{
    const dim3 grid(s.Hq, s.B);
    if (s.W > TILE_W) {
        const int n_cu = st.n_workers / (st.slots * WAVES);
        if ((long)s.B * s.Hq < 2L * n_cu) {
            // too few heads for one block per CU: one wave per 64-slot tile,
            // then one per head (measured faster there: a head's ring is
            // spread over many CUs)
            if (s.reuse) {
                const dim3 tgrid((s.W + TILE_W - 1) / TILE_W, s.Hq, s.B);
                if (s.ring_bf16)
                    hipLaunchKernelGGL(match_tiles_kernel<true>, tgrid, dim3(64), 0, stream, s,
                                       st, kv, seq_lens, q_pre, hidden);
                else
                    hipLaunchKernelGGL(match_tiles_kernel<false>, tgrid, dim3(64), 0, stream, s,
                                       st, kv, seq_lens, q_pre, hidden);
            }
            hipLaunchKernelGGL(match_tiled_kernel, grid, dim3(64), 0, stream, s, st, kv, seq_lens,
                               q_pre, override_pos, out, hidden);
            return hipGetLastError();
        }
        // sub-tiles of 16 slots, at most MATCH_WAVES waves per head
        const int sub = 16;
        const int waves = s.reuse ? min((s.W + sub - 1) / sub, MATCH_WAVES) : 1;
        if (s.ring_bf16)
            hipLaunchKernelGGL(match_wide_kernel<true>, grid, dim3(64 * waves), 0, stream, s, st,
                               kv, seq_lens, q_pre, override_pos, out, hidden);
        else
            hipLaunchKernelGGL(match_wide_kernel<false>, grid, dim3(64 * waves), 0, stream, s,
                               st, kv, seq_lens, q_pre, override_pos, out, hidden);
        return hipGetLastError();
    }
    // the whole ring in registers
    const int slots = s.W > 32 ? 64 : s.W > 16 ? 32 : 16;
#define MAC_MATCH(SL, BF)                                                                      \
    hipLaunchKernelGGL((match_kernel<SL, BF>), grid, dim3(64), 0, stream, s, st, kv, seq_lens,  \
                       q_pre, override_pos, out, hidden)
    if (s.ring_bf16) {
        if (slots == 16)
            MAC_MATCH(16, true);
        else if (slots == 32)
            MAC_MATCH(32, true);
        else
            MAC_MATCH(64, true);
    } else {
        if (slots == 16)
            MAC_MATCH(16, false);
        else if (slots == 32)
            MAC_MATCH(32, false);
        else
            MAC_MATCH(64, false);
    }
#undef MAC_MATCH
    return hipGetLastError();
}

}  // namespace mac
