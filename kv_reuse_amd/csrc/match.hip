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

    // slots [base, base + nslot) of head idx
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
            v[u] = sl < nslot ? rq[(long)sl * VPR + c] : Vec{};
        }
    }

    // Nearest valid entry of the loaded slots (wave-uniform result): squared
    // L2 distance to the pre-RoPE query qsrc, summed over each slot's lanes;
    // pos_l is the stamp of slot base + lane; valid stamps are 0 .. m.
    __device__ __forceinline__ void scan(const float *qsrc, int base, int nslot, int pos_l, int m,
                                         float &kd, int &kp, int &kj) const
    {
        const int lane = lane_id();
        const int sub = lane / (64 / PER), c = lane % (64 / PER);
        float q[8];
        if constexpr (BF16) {
            const float4 a = reinterpret_cast<const float4 *>(qsrc)[2 * c];
            const float4 b = reinterpret_cast<const float4 *>(qsrc)[2 * c + 1];
            q[0] = a.x, q[1] = a.y, q[2] = a.z, q[3] = a.w;
            q[4] = b.x, q[5] = b.y, q[6] = b.z, q[7] = b.w;
        } else {
            const float4 a = reinterpret_cast<const float4 *>(qsrc)[c];
            q[0] = a.x, q[1] = a.y, q[2] = a.z, q[3] = a.w;
        }
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
            const int pos = __shfl(pos_l, sl & 63, 64);
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

// =========================================================== match tiles
// Rings longer than one 64-slot tile (the pages' windows of 512-2048 entries,
// Figure 6, Tables 5 and 7).  Grid (tiles, Hq, B), one wave per tile: the
// wave loads the tile's 64 pre-RoPE queries (32 KB fp32, 16 KB bf16) and
// records the tile's nearest entry; the match kernel then reduces the tiles
// of each head.
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

// ================================================================== match
// Grid (Hq, B), one wave per (request, query head).  A ring of up to 64
// entries is held in registers (RingTile); a longer one arrives as
// per-tile nearest entries from match_tiles_kernel.  The kernel is
// latency-bound, so every load that does not depend on the query position
// (query, angles, ring, stamps, override, the head's counters) is issued
// before any of them is waited on.  The head then takes its decision (hit iff
// the relative L2 distance of the nearest valid entry is within tau, compared
// squared), applies an override, rotates its query (rotate-half RoPE, angle in
// fp64) and records its key span: [max(p - r + 1, 0), m] on a hit, [0, m] on
// a miss.
template <int SLOTS, bool BF16>
__global__ __launch_bounds__(64) void match_kernel(Shape s, State st, KvView kv,
                                                   const int32_t *__restrict__ seq_lens,
                                                   const float *__restrict__ q_pre,
                                                   const int32_t *__restrict__ ovr,
                                                   float *__restrict__ out, int hidden)
{
    const int h = blockIdx.x, b = blockIdx.y;
    const long idx = (long)b * s.Hq + h;
    const int lane = lane_id();
    const bool tiled = s.W > TILE_W;
    const int ntiles = (s.W + TILE_W - 1) / TILE_W;
    unsigned long long *hstat = st.head_stats + idx * HEAD_NSTAT;

    // ---- loads independent of the position
    RingTile<SLOTS, BF16> ring;
    if (s.reuse && !tiled)
        ring.load(s, st, idx, 0, s.W);
    const int seq = seq_lens[b];
    const float qa = q_pre[idx * D + lane], qb = q_pre[idx * D + lane + 64];
    const double inv = st.inv_freq[lane];
    const int ov = ovr ? ovr[idx] : -2;
    const int band = st.band[h];
    const int pos_l =
        (s.reuse && lane < s.W && lane != hidden) ? st.ring_pos[(long)b * s.W + lane] : -1;
    unsigned long long old[HEAD_NSTAT] = {};
    if (lane == 0) {
#pragma unroll
        for (int k = 0; k < HEAD_NSTAT; ++k)
            old[k] = hstat[k];
    }
    float td = INFINITY;
    int tp = INT_MIN, tj = -1;
    if (s.reuse && tiled && lane < ntiles) {
        const float *tb = st.tile_best + (idx * ntiles + lane) * 3;
        td = tb[0];
        tp = __float_as_int(tb[1]);
        tj = __float_as_int(tb[2]);
    }

    bool bad;
    const int m = query_position(kv, seq, bad);
    const bool act = m >= 0;
    int slot = -1, p = -1, start = 0;
    float rel = NAN;
    int cnt[HEAD_NSTAT] = {0, 0, 0, 0};
    if (act) {
        st.q_copy[idx * D + lane] = qa;
        st.q_copy[idx * D + lane + 64] = qb;
        float ra, rb;
        rope_pair(qa, qb, m, inv, ra, rb);
        st.q_rot[idx * D + lane] = ra;
        st.q_rot[idx * D + lane + 64] = rb;
    } else {
        // idle request: its output is zero (no group of it gets work)
        out[idx * D + lane] = 0.f;
        out[idx * D + lane + 64] = 0.f;
    }
    if (act && s.reuse) {
        float kd;
        int kp, kj;
        if (!tiled) {
            ring.scan(q_pre + idx * D, 0, s.W, pos_l, m, kd, kp, kj);
        } else {
            // nearest entry over the head's tiles
            kd = td;
            kp = tp;
            kj = tj;
#define MAC_ARGMIN_STEP(OFF)                                                                 \
    {                                                                                       \
        const float d2 = xor_lanes<OFF>(kd);                                                \
        const int p2 = xor_lanes_i<OFF>(kp);                                                \
        const int j2 = xor_lanes_i<OFF>(kj);                                                \
        if (nearer(d2, p2, j2, kd, kp, kj)) {                                               \
            kd = d2;                                                                        \
            kp = p2;                                                                        \
            kj = j2;                                                                        \
        }                                                                                   \
    }
            MAC_ARGMIN_STEP(1)
            MAC_ARGMIN_STEP(2)
            MAC_ARGMIN_STEP(4)
            MAC_ARGMIN_STEP(8)
            MAC_ARGMIN_STEP(16)
            MAC_ARGMIN_STEP(32)
#undef MAC_ARGMIN_STEP
        }
        const float q2 = wave_sum(qa * qa + qb * qb);
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
        if (ov != -2) {
            slot = -1;
            p = -1;
            if (ov >= 0) {
                // the largest slot holding position ov, 64 slots at a time
                for (int c0 = 0; c0 < s.W; c0 += 64) {
                    const int sl = c0 + lane;
                    const int ps = c0 == 0 ? pos_l
                                           : (sl < s.W ? st.ring_pos[(long)b * s.W + sl] : -1);
                    const bool mine = sl < s.W && sl != hidden && ov <= m && ps == ov;
                    const unsigned long long bal = __ballot(mine);
                    if (bal) {
                        slot = c0 + 63 - __clzll(bal);
                        p = ov;
                    }
                }
                if (slot < 0)
                    cnt[HS_OVR_INVALID] = 1;
            }
        }
        if (slot >= 0)
            start = max(p - band + 1, 0);
    }
    if (lane == 0) {
        st.dec_slot[idx] = slot;
        st.dec_p[idx] = p;
        st.dec_start[idx] = start;
        st.dec_rel[idx] = rel;
        if (act) {
            // this wave owns the head's counters: no atomics
            cnt[slot >= 0 ? HS_HITS : HS_MISSES] = 1;
#pragma unroll
            for (int k = 0; k < HEAD_NSTAT; ++k)
                hstat[k] = old[k] + (unsigned long long)cnt[k];
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

}  // namespace

hipError_t launch_match_tiles(const Shape &s, const State &st, const KvView &kv,
                              const int32_t *seq_lens, const float *q_pre, int hidden,
                              hipStream_t stream)
{
    const dim3 grid((s.W + TILE_W - 1) / TILE_W, s.Hq, s.B);
    if (s.ring_bf16)
        hipLaunchKernelGGL(match_tiles_kernel<true>, grid, dim3(64), 0, stream, s, st, kv,
                           seq_lens, q_pre, hidden);
    else
        hipLaunchKernelGGL(match_tiles_kernel<false>, grid, dim3(64), 0, stream, s, st, kv,
                           seq_lens, q_pre, hidden);
    return hipGetLastError();
}

hipError_t launch_match(const Shape &s, const State &st, const KvView &kv, const int32_t *seq_lens,
                        const float *q_pre, const int32_t *override_pos, float *out, int hidden,
                        hipStream_t stream)
{
    // ring slots held in registers: the whole ring up to 64 (a longer one is
    // read by match_tiles_kernel)
    const int slots = s.W > 32 ? 64 : s.W > 16 ? 32 : 16;
    const dim3 grid(s.Hq, s.B);
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
