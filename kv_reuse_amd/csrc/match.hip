// match.hip -- match step of the MAC-Attention decode (Figure 2 (a)): pre-RoPE
// L2 nearest neighbour over each (request, query head) ring, relative-L2
// threshold, RoPE of the query, and the per-head and per-group key spans.
#include "mac_device.h"

namespace mac {
namespace {

// =========================================================== match tiles
// Rings longer than one 64-slot tile (the pages' windows of 512-2048 entries,
// Figure 6, Tables 5 and 7).  Grid (tiles, Hq, B), one wave per tile: the wave
// streams the tile's 64 pre-RoPE queries (32 KB) as coalesced 1 KB loads, two
// slots per load (lanes 0-31 and 32-63, four columns each), sums the squared
// differences over each half with DPP and ds_swizzle, and keeps the nearest
// entry (smallest distance, newest position, larger slot).  The match kernel
// then reduces the tiles of each head.
__device__ __forceinline__ float half_sum(float v)
{
    v = row16_sum(v);
    v += xor_lanes<16>(v);   // stays within each 32-lane half
    return v;
}

__global__ __launch_bounds__(64) void match_tiles_kernel(Shape s, State st, KvView kv,
                                                         const int32_t *__restrict__ seq_lens,
                                                         const float *__restrict__ q_pre)
{
    const int tile = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int ntiles = (s.W + TILE_W - 1) / TILE_W;
    const long idx = (long)b * s.Hq + h;
    const int lane = lane_id(), half = lane >> 5, c = lane & 31;
    const int base = tile * TILE_W;
    const int nslot = min(TILE_W, s.W - base);
    int m = seq_lens[b] - 1;
    if (m >= 0 && (m >= kv.max_seq_len || (kv.paged && m / PAGE >= kv.max_pages)))
        m = -1;
    const int pos_l = lane < nslot ? st.ring_pos[(long)b * s.W + base + lane] : -1;
    const float4 qv = reinterpret_cast<const float4 *>(q_pre + idx * D)[c];
    const float4 *rq = reinterpret_cast<const float4 *>(st.ring_q + (idx * s.W + base) * D);
    float kd = INFINITY;
    int kp = INT_MIN, kj = -1;
    for (int i = 0; i < TILE_W; i += 16) {
        float4 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int sl = min(i + 2 * u + half, nslot - 1);   // clamped: in-bounds re-read
            v[u] = rq[(long)sl * (D / 4) + c];
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int sl = i + 2 * u + half;
            const float t0 = qv.x - v[u].x, t1 = qv.y - v[u].y, t2 = qv.z - v[u].z,
                        t3 = qv.w - v[u].w;
            float d = t0 * t0;
            d = fmaf(t1, t1, d);
            d = fmaf(t2, t2, d);
            d = fmaf(t3, t3, d);
            d = half_sum(d);
            const int pos = __shfl(pos_l, sl & 63, 64);
            const bool valid = sl < nslot && pos >= 0 && pos <= m;
            const float cd = valid ? d : INFINITY;
            const int cp = valid ? pos : INT_MIN;
            const int cj = valid ? base + sl : -1;
            if (cd < kd || (cd == kd && (cp > kp || (cp == kp && cj > kj)))) {
                kd = cd;
                kp = cp;
                kj = cj;
            }
        }
    }
    {   // the two halves saw different slots
        const float d2 = xor_lanes<32>(kd);
        const int p2 = xor_lanes_i<32>(kp);
        const int j2 = xor_lanes_i<32>(kj);
        if (d2 < kd || (d2 == kd && (p2 > kp || (p2 == kp && j2 > kj)))) {
            kd = d2;
            kp = p2;
            kj = j2;
        }
    }
    if (lane == 0) {
        float *o = st.tile_best + (idx * ntiles + tile) * 3;
        o[0] = kd;
        o[1] = __int_as_float(kp);
        o[2] = __int_as_float(kj);
    }
}

// ================================================================== match
// Grid (Hkv, B), 64 to 256 threads: the block owns one GQA group, its waves
// take the group's query heads in turn.  Each head's ring tile (W x D fp32) is
// staged in the wave's own LDS region with coalesced 16-byte loads; 64/W lanes
// share a slot's distance, and a DPP/ds_swizzle butterfly finds the nearest
// entry.  The kernel is latency-bound, so every load that does not depend on
// the query position (queries, angles, ring tile, stamps, override, the
// group's counters) is issued before any of them is waited on.
__global__ __launch_bounds__(BLOCK) void match_kernel(Shape s, State st, KvView kv,
                                                      const int32_t *__restrict__ seq_lens,
                                                      const float *__restrict__ q_pre,
                                                      const int32_t *__restrict__ ovr,
                                                      float *__restrict__ out)
{
    extern __shared__ float lds[];
    __shared__ int h_start[64];
    __shared__ int wcnt[WAVES][4];   // per wave: hits, misses, near tau, invalid overrides
    const int b = blockIdx.y, kvh = blockIdx.x;
    const int lane = lane_id(), wv = threadIdx.x >> 6;
    const int nwv = blockDim.x >> 6;   // waves in the block (sized to the LDS budget)
    constexpr int RS = D + 4;          // LDS row stride (floats)
    const long g = (long)b * s.Hkv + kvh;
    unsigned long long *gstat = st.stats + MAC_NSTAT + g * GRP_NSTAT;

    // lanes per ring slot: a power of two, at most 32 so each lane owns a
    // whole number of float4 columns (D / L >= 4); one when the ring is tiled
    const bool tiled = s.W > TILE_W;   // nearest entries come from match_tiles_kernel
    int L = tiled ? 1 : 64 / s.W;
    while (L & (L - 1))
        L &= L - 1;
    if (L > 32)
        L = 32;
    const int j = lane / L, part = lane % L, span = D / L;
    const int jc = j < s.W ? j : s.W - 1;
    const int lc = lane < s.W ? lane : s.W - 1;
    const int ntiles = (s.W + TILE_W - 1) / TILE_W;

    // ---- loads independent of the position
    const int seq = seq_lens[b];
    const int pos_j = st.ring_pos[(long)b * s.W + jc];    // stamp of this lane's slot
    const int pos_l = st.ring_pos[(long)b * s.W + lc];    // stamp of slot `lane`
    const double inv = st.inv_freq[lane];
    unsigned long long old[GRP_NSTAT] = {};
    if (threadIdx.x == 0) {
#pragma unroll
        for (int k = 0; k < GRP_NSTAT; ++k)
            old[k] = gstat[k];
    }
    float *tile = lds + wv * (s.W * RS + D);
    float *qs = tile + s.W * RS;
    int my_cnt[4] = {0, 0, 0, 0};

    int m = seq - 1;
    const bool bad = m >= 0 && (m >= kv.max_seq_len || (kv.paged && m / PAGE >= kv.max_pages));
    if (bad)
        m = -1;

    for (int hb = 0; hb < s.G; hb += nwv) {
        const int hh = hb + wv;
        const bool head = hh < s.G;
        const long idx = (long)b * s.Hq + kvh * s.G + (head ? hh : 0);
        float qa = 0.f, qb = 0.f;
        int ov = -2;
        if (head) {
            qa = q_pre[idx * D + lane];
            qb = q_pre[idx * D + lane + 64];
            if (ovr)
                ov = ovr[idx];
            if (s.reuse && !tiled) {
                // a batch of 8 loads per lane is in flight before its LDS writes;
                // indices past the tile are clamped (in-bounds re-reads whose
                // values are not stored), so the batch stays in registers
                const float4 *src = reinterpret_cast<const float4 *>(st.ring_q + idx * s.W * D);
                const int n4 = s.W * (D / 4);
                for (int base = 0; base < n4; base += 64 * 8) {
                    float4 t0, t1, t2, t3, t4, t5, t6, t7;
#define MAC_LD(T, C) T = src[min(base + (C) * 64 + lane, n4 - 1)];
                    MAC_LD(t0, 0) MAC_LD(t1, 1) MAC_LD(t2, 2) MAC_LD(t3, 3)
                    MAC_LD(t4, 4) MAC_LD(t5, 5) MAC_LD(t6, 6) MAC_LD(t7, 7)
#undef MAC_LD
#define MAC_ST(T, C)                                                                         \
    {                                                                                       \
        const int i = base + (C) * 64 + lane;                                               \
        if (i < n4)                                                                         \
            *reinterpret_cast<float4 *>(tile + (i / (D / 4)) * RS + (i % (D / 4)) * 4) = T; \
    }
                    MAC_ST(t0, 0) MAC_ST(t1, 1) MAC_ST(t2, 2) MAC_ST(t3, 3)
                    MAC_ST(t4, 4) MAC_ST(t5, 5) MAC_ST(t6, 6) MAC_ST(t7, 7)
#undef MAC_ST
                }
                qs[lane] = qa;
                qs[lane + 64] = qb;
            }
        }
        const bool act = head && m >= 0;
        int slot = -1, p = -1, start = 0;
        float rel = NAN;
        if (act) {
            st.q_copy[idx * D + lane] = qa;
            st.q_copy[idx * D + lane + 64] = qb;
            // rotate-half RoPE, angle m * theta^(-2i/D) formed in fp64 and
            // reduced to [-pi, pi] in fp64 (Cody-Waite, 2*pi split in two
            // doubles, fma), so sincos stays on its short-argument path
            const double phi = (double)m * inv;
            const double k = rint(phi * 0.15915494309189535);   // 1 / (2*pi)
            double red = fma(-k, 6.283185307179586232, phi);      // 2*pi rounded to double
            red = fma(-k, 2.4492935982947064e-16, red);            // 2*pi minus that double
            double sn, cs;
            sincos(red, &sn, &cs);
            st.q_rot[idx * D + lane] = (float)((double)qa * cs - (double)qb * sn);
            st.q_rot[idx * D + lane + 64] = (float)((double)qb * cs + (double)qa * sn);
        } else if (head) {
            // idle request: its output is zero (no group of it gets work)
            out[idx * D + lane] = 0.f;
            out[idx * D + lane + 64] = 0.f;
        }
        if (act && s.reuse) {
            float kd;
            int kp, kj;
            if (tiled) {
                // nearest entry per 64-slot tile, reduced over the head's tiles
                kd = INFINITY;
                kp = INT_MIN;
                kj = -1;
                if (lane < ntiles) {
                    const float *tb = st.tile_best + (idx * ntiles + lane) * 3;
                    kd = tb[0];
                    kp = __float_as_int(tb[1]);
                    kj = __float_as_int(tb[2]);
                }
            } else {
            // this wave wrote its own tile above; LDS accesses of a wave are ordered
            float dp = 0.f;
            if (j < s.W) {
                const float *rr = tile + j * RS + part * span;
                const float *qq = qs + part * span;
                for (int e = 0; e < span; e += 4) {
                    const float4 x = *reinterpret_cast<const float4 *>(rr + e);
                    const float4 y = *reinterpret_cast<const float4 *>(qq + e);
                    const float t0 = y.x - x.x, t1 = y.y - x.y, t2 = y.z - x.z, t3 = y.w - x.w;
                    dp = fmaf(t0, t0, dp);
                    dp = fmaf(t1, t1, dp);
                    dp = fmaf(t2, t2, dp);
                    dp = fmaf(t3, t3, dp);
                }
            }
            if (L >= 2) dp += xor_lanes<1>(dp);
            if (L >= 4) dp += xor_lanes<2>(dp);
            if (L >= 8) dp += xor_lanes<4>(dp);
            if (L >= 16) dp += xor_lanes<8>(dp);
            if (L >= 32) dp += xor_lanes<16>(dp);
            const bool valid = j < s.W && pos_j >= 0 && pos_j <= m;
            kd = valid ? dp : INFINITY;
            kp = valid ? pos_j : INT_MIN;
            kj = valid ? j : -1;
            }
            // nearest entry: smallest distance, then newest position, then larger slot
#define MAC_ARGMIN_STEP(OFF)                                                                 \
    {                                                                                       \
        const float d2 = xor_lanes<OFF>(kd);                                                \
        const int p2 = xor_lanes_i<OFF>(kp);                                                \
        const int j2 = xor_lanes_i<OFF>(kj);                                                \
        if (d2 < kd || (d2 == kd && (p2 > kp || (p2 == kp && j2 > kj)))) {                  \
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
            const float q2 = wave_sum(qa * qa + qb * qb);
            if (kp >= 0) {
                rel = q2 > 0.f ? sqrtf(kd / q2) : (kd == 0.f ? 0.f : INFINITY);
                // relative-L2 test compared squared: D <= tau^2 |q~|^2
                if (s.tau >= 0.f && kd <= s.tau * s.tau * q2) {
                    slot = kj;
                    p = kp;
                }
                if (fabsf(rel - s.tau) < 1e-4f)
                    my_cnt[2] += 1;
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
                        const bool mine = sl < s.W && ov <= m && ps == ov;
                        const unsigned long long bal = __ballot(mine);
                        if (bal) {
                            slot = c0 + 63 - __clzll(bal);
                            p = ov;
                        }
                    }
                    if (slot < 0)
                        my_cnt[3] += 1;
                }
            }
            if (slot >= 0)
                start = max(p - s.r + 1, 0);
        }
        if (act)
            my_cnt[slot >= 0 ? 0 : 1] += 1;
        if (head && lane == 0) {
            st.dec_slot[idx] = slot;
            st.dec_p[idx] = p;
            st.dec_start[idx] = start;
            st.dec_rel[idx] = rel;
            h_start[hh] = start;
        }
    }
    if (lane == 0) {
#pragma unroll
        for (int k = 0; k < 4; ++k)
            wcnt[wv][k] = my_cnt[k];
    }
    __syncthreads();

    if (threadIdx.x == 0) {
        if (kvh == 0) {
            st.m_buf[b] = m;
            if (bad)
                atomicAdd(&st.stats[ST_BAD_INPUT], 1ULL);
        }
        int gs = -1;
        if (m >= 0) {
            gs = m + 1;
            for (int h = 0; h < s.G; ++h)
                gs = min(gs, h_start[h]);
        }
        st.grp_start[g] = gs;
        if (m >= 0) {
            // this block owns the group's counters for the step: no atomics
            unsigned long long c[4] = {0, 0, 0, 0};
            for (int w = 0; w < nwv; ++w)
                for (int k = 0; k < 4; ++k)
                    c[k] += (unsigned long long)wcnt[w][k];
            gstat[ST_HITS] = old[ST_HITS] + c[0];
            gstat[ST_MISSES] = old[ST_MISSES] + c[1];
            gstat[ST_DECISIONS] = old[ST_DECISIONS] + c[0] + c[1];
            gstat[ST_NEAR_TAU] = old[ST_NEAR_TAU] + c[2];
            gstat[ST_OVR_INVALID] = old[ST_OVR_INVALID] + c[3];
            gstat[ST_TOK_CRIT] = old[ST_TOK_CRIT] + (unsigned long long)(m - gs + 1);
            if (s.reuse && m - s.r >= 0)
                gstat[ST_TOK_AMEND] = old[ST_TOK_AMEND] + (unsigned long long)s.r;
        }
    }
}

// LDS a match wave needs: its ring tile and query (none when the ring is scanned
// by match_tiles_kernel).
size_t match_lds_per_wave(const Shape &s)
{
    return s.W > TILE_W ? 0 : (size_t)(s.W * (D + 4) + D) * sizeof(float);
}

}  // namespace

hipError_t launch_match_tiles(const Shape &s, const State &st, const KvView &kv,
                              const int32_t *seq_lens, const float *q_pre, hipStream_t stream)
{
    const dim3 grid((s.W + TILE_W - 1) / TILE_W, s.Hq, s.B);
    hipLaunchKernelGGL(match_tiles_kernel, grid, dim3(64), 0, stream, s, st, kv, seq_lens, q_pre);
    return hipGetLastError();
}

int match_waves(const Shape &s, size_t max_lds)
{
    const size_t per_wave = match_lds_per_wave(s);
    if (per_wave == 0)
        return s.G < WAVES ? s.G : WAVES;
    int n = (int)(max_lds / per_wave);
    n = n < 1 ? 1 : (n > WAVES ? WAVES : n);
    return n > s.G ? s.G : n;
}

hipError_t launch_match(const Shape &s, const State &st, const KvView &kv, const int32_t *seq_lens,
                        const float *q_pre, const int32_t *override_pos, float *out, int waves,
                        hipStream_t stream)
{
    const size_t lds = (size_t)waves * match_lds_per_wave(s);
    hipLaunchKernelGGL(match_kernel, dim3(s.Hkv, s.B), dim3(64 * waves), lds, stream, s, st, kv,
                       seq_lens, q_pre, override_pos, out);
    return hipGetLastError();
}

}  // namespace mac
