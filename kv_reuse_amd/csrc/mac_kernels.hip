// mac_kernels.hip -- gfx950 kernels of the MAC-Attention decode step.
//
// MAC-Attention (arXiv 2604.00235), paper card, Figure 2 and Figure 3:
//   match_kernel     (a) pre-RoPE L2 nearest neighbour over the ring, threshold,
//                    RoPE of the query, per-head and per-group key spans
//   complete_kernel  (b) split-KV flash-decode over each group's union span,
//                    equal page shares per wave (the load-balanced plan of
//                    Figure 3 (b), built on the device)
//   reduce_kernel    (b) combine the per-wave partial summaries, log-domain
//                    merge (+) with the matched entry's stored AS_{1:p-r}
//   amend_kernel     (c) recompute the last-r band, log-domain removal (-),
//                    ring insert; runs on the amend stream
//   append_kernel    KV manager side: write this step's key/value rows
//
// Wave64 throughout.  Key/value rows stream as 16-byte loads: for bf16 a row
// of 128 elements is 16 lanes, a wave load covers 4 tokens and a 16-token page
// is 4 loads of K and 4 of V; fp32 rows take 32 lanes.
#include <hip/hip_runtime.h>

#include <climits>
#include <cmath>
#include <type_traits>

#include "mac_internal.h"

namespace mac {
namespace {

constexpr float NEG_INF = -INFINITY;

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// ------------------------------------------------------------ lane exchange
// DPP for exchanges inside a quad, ds_swizzle (bit mode) inside 32 lanes,
// ds_bpermute across the two halves.
template <int OFF>
__device__ __forceinline__ int xor_lanes_i(int v)
{
    static_assert(OFF > 0 && OFF < 64 && (OFF & (OFF - 1)) == 0, "power of two");
    if constexpr (OFF == 1)
        return __builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, true);   // quad_perm [1,0,3,2]
    else if constexpr (OFF == 2)
        return __builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, true);   // quad_perm [2,3,0,1]
    else if constexpr (OFF < 32)
        return __builtin_amdgcn_ds_swizzle(v, (OFF << 10) | 0x1F);   // xor mask, and 0x1F
    else
        return __shfl_xor(v, 32, 64);
}

template <int OFF>
__device__ __forceinline__ float xor_lanes(float v)
{
    return __int_as_float(xor_lanes_i<OFF>(__float_as_int(v)));
}

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v)
{
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}

// Sum over each 16-lane row: after the two quad exchanges every quad is
// uniform, so the half mirror and the full mirror finish the reduction.
__device__ __forceinline__ float row16_sum(float v)
{
    v += dpp_f<0xB1>(v);
    v += dpp_f<0x4E>(v);
    v += dpp_f<0x141>(v);   // row_half_mirror
    v += dpp_f<0x140>(v);   // row_mirror
    return v;
}

__device__ __forceinline__ float wave_sum(float v)
{
    v = row16_sum(v);
    v += xor_lanes<16>(v);
    v += xor_lanes<32>(v);
    return v;
}

__device__ __forceinline__ float wave_max(float v)
{
    v = fmaxf(v, xor_lanes<1>(v));
    v = fmaxf(v, xor_lanes<2>(v));
    v = fmaxf(v, xor_lanes<4>(v));
    v = fmaxf(v, xor_lanes<8>(v));
    v = fmaxf(v, xor_lanes<16>(v));
    v = fmaxf(v, xor_lanes<32>(v));
    return v;
}

// ------------------------------------------------------- key/value element
template <typename T>
struct Kv;
template <>
struct Kv<uint16_t> {           // bf16 bit patterns
    static constexpr int E = 8;     // elements per 16-byte lane load
    static constexpr int LPR = 16;  // lanes per 128-element row
    static constexpr int RPL = 4;   // rows (tokens) per wave load
    static constexpr int LPP = 4;   // wave loads per 16-token page
};
template <>
struct Kv<float> {
    static constexpr int E = 4;
    static constexpr int LPR = 32;
    static constexpr int RPL = 2;
    static constexpr int LPP = 8;
};

__device__ __forceinline__ void to_f32(const uint4 &w, float (&f)[8])
{
    f[0] = __uint_as_float(w.x << 16);
    f[1] = __uint_as_float(w.x & 0xffff0000u);
    f[2] = __uint_as_float(w.y << 16);
    f[3] = __uint_as_float(w.y & 0xffff0000u);
    f[4] = __uint_as_float(w.z << 16);
    f[5] = __uint_as_float(w.z & 0xffff0000u);
    f[6] = __uint_as_float(w.w << 16);
    f[7] = __uint_as_float(w.w & 0xffff0000u);
}

__device__ __forceinline__ void to_f32(const uint4 &w, float (&f)[4])
{
    f[0] = __uint_as_float(w.x);
    f[1] = __uint_as_float(w.y);
    f[2] = __uint_as_float(w.z);
    f[3] = __uint_as_float(w.w);
}

template <typename T>
__device__ __forceinline__ float row_sum(float v)
{
    v = row16_sum(v);
    if constexpr (Kv<T>::LPR == 32)
        v += xor_lanes<16>(v);
    return v;
}

// Address of the 16 x D block holding tokens [16*page, 16*page+16) of
// (request b, KV head kvh).  A page id outside the pool is replaced by page 0
// and counted, so a corrupt table never reads outside the cache.
template <typename T>
__device__ __forceinline__ const T *kv_page(const KvView &kv, const void *base, int b, int kvh,
                                            int Hkv, int page, unsigned long long *bad)
{
    long off;
    if (kv.paged) {
        int pid = kv.page_table[(long)b * kv.max_pages + page];
        if ((unsigned)pid >= (unsigned)kv.num_pages) {
            atomicAdd(bad, 1ULL);
            pid = 0;
        }
        off = ((long)pid * Hkv + kvh) * (PAGE * D);
    } else {
        off = ((long)b * Hkv + kvh) * (long)kv.max_seq_len * D + (long)page * (PAGE * D);
    }
    return reinterpret_cast<const T *>(base) + off;
}

// ------------------------------------------------ flash-decode wave worker
// One wave keeps, per head of its GQA group and per row group of lanes (the
// tokens it loads), a running max M (log2 units), normaliser L and
// unnormalised output acc over its E output columns.
template <int G, int E>
struct WaveAcc {
    float M[G], L[G], acc[G][E];
    __device__ __forceinline__ void init()
    {
#pragma unroll
        for (int g = 0; g < G; ++g) {
            M[g] = NEG_INF;
            L[g] = 0.f;
#pragma unroll
            for (int e = 0; e < E; ++e)
                acc[g][e] = 0.f;
        }
    }
};

// Key/value rows are streamed once per step: non-temporal 16-byte loads keep
// them from displacing reusable lines in L2 and the Infinity Cache (used where
// a wave load covers whole 128-byte lines).
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_stream(const void *p)
{
    const u32x4 t = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
    return make_uint4(t[0], t[1], t[2], t[3]);
}

template <typename T>
struct PageRegs {
    uint4 k[Kv<T>::LPP], v[Kv<T>::LPP];
};

template <typename T>
__device__ __forceinline__ void load_page(PageRegs<T> &r, const T *kp, const T *vp)
{
    using K = Kv<T>;
    const int lane = lane_id(), row = lane / K::LPR, col = lane % K::LPR;
#pragma unroll
    for (int s = 0; s < K::LPP; ++s)
        r.k[s] = load_stream(kp + (s * K::RPL + row) * D + col * K::E);
#pragma unroll
    for (int s = 0; s < K::LPP; ++s)
        r.v[s] = load_stream(vp + (s * K::RPL + row) * D + col * K::E);
}

// Fold one page into the wave's state.  Token t of the page is valid for
// head g iff hs[g] <= t <= m; `masked` is false when every token is valid for
// every head (the common case), and rows past m are zeroed since a cache slot
// that was never written may hold any bits.
template <typename T, int G>
__device__ __forceinline__ void compute_page(const PageRegs<T> &r, int tok0, int m,
                                             const int (&hs)[G], bool masked,
                                             const float (&q)[G][Kv<T>::E],
                                             WaveAcc<G, Kv<T>::E> &st)
{
    using K = Kv<T>;
    constexpr int E = K::E;
    const int row = lane_id() / K::LPR;
    float lg[K::LPP][G];
#pragma unroll
    for (int s = 0; s < K::LPP; ++s) {
        float kf[E];
        to_f32(r.k[s], kf);
#pragma unroll
        for (int g = 0; g < G; ++g) {
            float a = 0.f;
#pragma unroll
            for (int e = 0; e < E; ++e)
                a = fmaf(q[g][e], kf[e], a);
            lg[s][g] = row_sum<T>(a);
        }
    }
    if (masked) {
#pragma unroll
        for (int s = 0; s < K::LPP; ++s) {
            const int t = tok0 + s * K::RPL + row;
#pragma unroll
            for (int g = 0; g < G; ++g)
                if (t < hs[g] || t > m)
                    lg[s][g] = NEG_INF;
        }
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
        float mx = lg[0][g];
#pragma unroll
        for (int s = 1; s < K::LPP; ++s)
            mx = fmaxf(mx, lg[s][g]);
        const float mn = fmaxf(st.M[g], mx);
        const float base = mn == NEG_INF ? 0.f : mn;
        const float alpha = exp2f(st.M[g] - base);
        st.M[g] = mn;
        st.L[g] *= alpha;
#pragma unroll
        for (int e = 0; e < E; ++e)
            st.acc[g][e] *= alpha;
#pragma unroll
        for (int s = 0; s < K::LPP; ++s)
            lg[s][g] = exp2f(lg[s][g] - base);
    }
#pragma unroll
    for (int s = 0; s < K::LPP; ++s) {
        float vf[E];
        to_f32(r.v[s], vf);
        if (masked && tok0 + s * K::RPL + row > m) {
#pragma unroll
            for (int e = 0; e < E; ++e)
                vf[e] = 0.f;
        }
#pragma unroll
        for (int g = 0; g < G; ++g) {
            st.L[g] += lg[s][g];
#pragma unroll
            for (int e = 0; e < E; ++e)
                st.acc[g][e] = fmaf(lg[s][g], vf[e], st.acc[g][e]);
        }
    }
}

// Combine the wave's row groups and store, per head, the unnormalised
// summary (acc[D], M, L) at dst[g*SUMM ..] (global memory or LDS).
template <typename T, int G>
__device__ __forceinline__ void store_wave_summary(WaveAcc<G, Kv<T>::E> &st, float *dst)
{
    using K = Kv<T>;
    constexpr int E = K::E;
    const int lane = lane_id(), row = lane / K::LPR, col = lane % K::LPR;
#pragma unroll
    for (int g = 0; g < G; ++g) {
        float Mt = st.M[g];
        if constexpr (K::LPR == 16)
            Mt = fmaxf(Mt, xor_lanes<16>(Mt));
        Mt = fmaxf(Mt, xor_lanes<32>(Mt));
        const float base = Mt == NEG_INF ? 0.f : Mt;
        const float sc = exp2f(st.M[g] - base);
        float Lr = st.L[g] * sc;
        float a[E];
#pragma unroll
        for (int e = 0; e < E; ++e)
            a[e] = st.acc[g][e] * sc;
        if constexpr (K::LPR == 16) {
            Lr += xor_lanes<16>(Lr);
#pragma unroll
            for (int e = 0; e < E; ++e)
                a[e] += xor_lanes<16>(a[e]);
        }
        Lr += xor_lanes<32>(Lr);
#pragma unroll
        for (int e = 0; e < E; ++e)
            a[e] += xor_lanes<32>(a[e]);
        if (row == 0) {
#pragma unroll
            for (int e = 0; e < E; e += 4)
                *reinterpret_cast<float4 *>(dst + g * SUMM + col * E + e) =
                    make_float4(a[e], a[e + 1], a[e + 2], a[e + 3]);
        }
        if (lane == 0) {
            dst[g * SUMM + D] = Mt;
            dst[g * SUMM + D + 1] = Lr;
        }
    }
}

// Queries of the G heads of (b, kvh), this lane's E columns, scaled so that
// q.k is the logit in log2 units.
template <typename T, int G>
__device__ __forceinline__ void load_group_queries(const Shape &s, const State &st, int b, int kvh,
                                                   float (&q)[G][Kv<T>::E])
{
    using K = Kv<T>;
    const int col = lane_id() % K::LPR;
#pragma unroll
    for (int g = 0; g < G; ++g) {
        const float *src = st.q_rot + ((long)b * s.Hq + kvh * G + g) * D + col * K::E;
#pragma unroll
        for (int e = 0; e < K::E; e += 4) {
            float4 x = *reinterpret_cast<const float4 *>(src + e);
            q[g][e + 0] = x.x * s.scale_log2;
            q[g][e + 1] = x.y * s.scale_log2;
            q[g][e + 2] = x.z * s.scale_log2;
            q[g][e + 3] = x.w * s.scale_log2;
        }
    }
}

// ------------------------------------------------------------------- plan
// Exclusive prefix sum of a[0..n) in LDS by the whole block; a[n] = total.
__device__ void block_exclusive_scan(int *a, int n)
{
    __shared__ int wsum[WAVES];
    const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
    const int per = (n + BLOCK - 1) / BLOCK;
    const int lo = min(n, t * per), hi = min(n, lo + per);
    int sum = 0;
    for (int i = lo; i < hi; ++i)
        sum += a[i];
    int x = sum;
    for (int off = 1; off < 64; off <<= 1) {
        int y = __shfl_up(x, off, 64);
        if (lane >= off)
            x += y;
    }
    if (lane == 63)
        wsum[wv] = x;
    __syncthreads();
    int pre = 0, tot = 0;
    for (int i = 0; i < WAVES; ++i) {
        if (i < wv)
            pre += wsum[i];
        tot += wsum[i];
    }
    int run = pre + x - sum;
    for (int i = lo; i < hi; ++i) {
        int v = a[i];
        a[i] = run;
        run += v;
    }
    if (t == 0)
        a[n] = tot;
    __syncthreads();
}

// Page offsets of every group's union span in the flattened work list:
// off[g] = pages of groups before g, off[nG] = all pages of the step.
__device__ void build_plan(const Shape &s, const State &st, int *off)
{
    const int nG = s.B * s.Hkv;
    for (int g = threadIdx.x; g < nG; g += BLOCK) {
        const int gs = st.grp_start[g];
        const int m = st.m_buf[g / s.Hkv];
        off[g] = (gs < 0 || m < 0) ? 0 : (m / PAGE - gs / PAGE + 1);
    }
    __syncthreads();
    block_exclusive_scan(off, nG);
}

// Waves that take part: every worker gets at least MIN_PAGES_PER_WORKER pages.
__device__ __forceinline__ int active_workers(int n_workers, int P)
{
    return min(n_workers, (P + MIN_PAGES_PER_WORKER - 1) / MIN_PAGES_PER_WORKER);
}

// Worker w owns flattened pages [w*P/nW, (w+1)*P/nW); owner of page x:
__device__ __forceinline__ int page_owner(long x, int nW, int P)
{
    return (int)(((x + 1) * (long)nW - 1) / P);
}

// Last group g with off[g] <= x (groups with no pages are skipped by caller).
__device__ __forceinline__ int find_group(const int *off, int nG, long x)
{
    int lo = 0, hi = nG - 1;
    while (lo < hi) {
        int mid = (lo + hi + 1) >> 1;
        if (off[mid] <= x)
            lo = mid;
        else
            hi = mid - 1;
    }
    return lo;
}

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

// =============================================================== complete
// Persistent grid of independent wave workers.  Every block rebuilds the
// plan (a scan over B*Hkv group spans) in LDS; the step's pages, group after
// group, are split into equal contiguous shares, one per active wave.  A
// worker writes one partial summary per group it touches, into slot
// (worker + group), which is unique along the flattened list.
template <typename T, int G>
__global__ __launch_bounds__(BLOCK) void complete_kernel(Shape s, State st, KvView kv)
{
    extern __shared__ int s_off[];
    using K = Kv<T>;
    const int nG = s.B * s.Hkv;
    build_plan(s, st, s_off);
    const int P = s_off[nG];
    if (P == 0)
        return;
    const int nW = active_workers(st.n_workers, P);
    const int w = blockIdx.x * WAVES + (threadIdx.x >> 6);
    if (w >= nW)
        return;
    long x = (long)w * P / nW;
    const long x1 = (long)(w + 1) * P / nW;
    int g = find_group(s_off, nG, x);
    while (x < x1) {
        while (s_off[g + 1] <= x)
            ++g;
        const long gend = min((long)s_off[g + 1], x1);
        const int b = g / s.Hkv, kvh = g % s.Hkv;
        const int m = st.m_buf[b];
        const int first_page = st.grp_start[g] / PAGE;
        int hs[G];
        int hmax = 0;
#pragma unroll
        for (int h = 0; h < G; ++h) {
            hs[h] = st.dec_start[(long)b * s.Hq + kvh * G + h];
            hmax = max(hmax, hs[h]);
        }
        float q[G][K::E];
        load_group_queries<T, G>(s, st, b, kvh, q);
        WaveAcc<G, K::E> acc;
        acc.init();

        PageRegs<T> r0, r1;
        int page = first_page + (int)(x - s_off[g]);
        const int last = first_page + (int)(gend - s_off[g]) - 1;
        load_page<T>(r0, kv_page<T>(kv, kv.k, b, kvh, s.Hkv, page, &st.stats[ST_BAD_INPUT]),
                     kv_page<T>(kv, kv.v, b, kvh, s.Hkv, page, &st.stats[ST_BAD_INPUT]));
        while (true) {
            if (page + 1 <= last)
                load_page<T>(r1,
                             kv_page<T>(kv, kv.k, b, kvh, s.Hkv, page + 1, &st.stats[ST_BAD_INPUT]),
                             kv_page<T>(kv, kv.v, b, kvh, s.Hkv, page + 1, &st.stats[ST_BAD_INPUT]));
            {
                const int tok0 = page * PAGE;
                compute_page<T, G>(r0, tok0, m, hs, tok0 < hmax || tok0 + PAGE - 1 > m, q, acc);
            }
            if (++page > last)
                break;
            if (page + 1 <= last)
                load_page<T>(r0,
                             kv_page<T>(kv, kv.k, b, kvh, s.Hkv, page + 1, &st.stats[ST_BAD_INPUT]),
                             kv_page<T>(kv, kv.v, b, kvh, s.Hkv, page + 1, &st.stats[ST_BAD_INPUT]));
            {
                const int tok0 = page * PAGE;
                compute_page<T, G>(r1, tok0, m, hs, tok0 < hmax || tok0 + PAGE - 1 > m, q, acc);
            }
            if (++page > last)
                break;
        }
        store_wave_summary<T, G>(acc, st.partials + ((long)w + g) * G * SUMM);
        x = gend;
    }
}

// ========================================================== complete (MFMA)
// bf16 cache, G <= 4 query heads per KV head.  Q.K^T runs on the matrix cores:
// v_mfma_f32_16x16x32_bf16 with the page's 16 tokens as the 16 columns of B
// (lane l feeds token l%16, columns 32s + 8(l/16) .. +7 at k-step s, straight
// from its 16-byte K load) and the group's queries as the rows of A,
// replicated so that row i holds head i % G: every lane receives the logits of
// all G heads for token l%16.  A carries the query split into two bf16 parts
// (hi + lo), so the logits keep ~16 mantissa bits of the fp32 query.
// P.V stays on the vector units with V loaded as contiguous 1 KB wave loads
// (lane (r, c) = (l/16, l%16) holds token 4s + r, columns 8c .. 8c+7); each
// token's probabilities reach the lanes that hold its V row through a
// 256-byte per-wave LDS exchange.  The softmax reference max is uniform over
// the wave (one per head) and only moves when a logit exceeds it by more than
// LAZY_RESCALE (log2 units): exp2(s - M) <= 256 is accumulated as is, and the
// rescale, when it happens, is exact.
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr float LAZY_RESCALE = 8.f;

struct MPage {
    uint4 k[4], v[4];
};

// K arrives in the MFMA layout: one wave load covers 64 of the 128 bytes of 16
// rows, so every cache line is shared by two consecutive loads and is read
// with the default policy (a streaming hint makes the second half refetch).
// V arrives as contiguous 1 KB wave loads of whole lines and is streamed.
__device__ __forceinline__ void load_mpage(MPage &r, const uint16_t *kp, const uint16_t *vp)
{
    const int lane = lane_id(), t = lane & 15, q = lane >> 4;
#pragma unroll
    for (int s = 0; s < 4; ++s)
        r.k[s] = *reinterpret_cast<const uint4 *>(kp + t * D + 32 * s + 8 * q);
#pragma unroll
    for (int s = 0; s < 4; ++s)
        r.v[s] = load_stream(vp + (4 * s + q) * D + 8 * t);
}

// HPL: heads whose logits one lane receives from the MFMA (4 row groups of 4
// rows; row i holds head i % G).  For G = 8 the lanes of row groups 0 and 2
// hold heads 0..3 and those of row groups 1 and 3 hold heads 4..7.
template <int G>
struct MAcc {
    static constexpr int HPL = G < 4 ? G : 4;
    float M[G];           // wave-uniform reference max per head (log2 units)
    float Ml[HPL];        // M of this lane's own heads (M[v], or M[4 + v] for G = 8)
    float L[HPL];         // normaliser of this lane's heads over this lane's tokens
    float acc[G][8];      // P.V over this lane's V rows and 8 columns
};

// Per-lane choice between two registers by a lane mask.  Written as the
// instruction itself: a C select between two elements of a register array is
// folded by the compiler into an indexed access, which moves the array to
// scratch memory.
__device__ __forceinline__ float lane_pick(unsigned long long mask, float if_set, float if_clear)
{
    float r;
    asm volatile("v_cndmask_b32_e64 %0, %1, %2, %3"
                 : "=v"(r)
                 : "v"(if_clear), "v"(if_set), "s"(mask));
    return r;
}

__device__ __forceinline__ int lane_pick(unsigned long long mask, int if_set, int if_clear)
{
    return __float_as_int(lane_pick(mask, __int_as_float(if_set), __int_as_float(if_clear)));
}

// hsl: first key of each of this lane's own heads' spans.  half_mask: lanes
// holding heads 4..7 (G = 8; zero otherwise).
template <int G>
__device__ __forceinline__ void compute_mpage(const MPage &r, const uint4 *qa, float4 *px,
                                              int tok0, int m, const int (&hsl)[MAcc<G>::HPL],
                                              bool masked, unsigned long long half_mask,
                                              MAcc<G> &st)
{
    constexpr int HPL = MAcc<G>::HPL;
    constexpr int NPX = G > 4 ? 2 : 1;   // float4 of probabilities per token
    const int lane = lane_id(), t = lane & 15, q = lane >> 4;
    const int half = G > 4 ? (q & 1) : 0;   // which four heads this lane holds
    floatx4 S0 = {0.f, 0.f, 0.f, 0.f}, S1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        const bf16x8 kb = __builtin_bit_cast(bf16x8, r.k[s]);
        const uint4 ahi = qa[(2 * s) * 64 + lane], alo = qa[(2 * s + 1) * 64 + lane];
        S0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ahi), kb, S0, 0,
                                                     0, 0);
        S1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, alo), kb, S1, 0,
                                                     0, 0);
    }
    float lg[HPL];
#pragma unroll
    for (int v = 0; v < HPL; ++v)
        lg[v] = S0[v] + S1[v];
    if (masked) {
        const int tok = tok0 + t;
#pragma unroll
        for (int v = 0; v < HPL; ++v)
            if (tok < hsl[v] || tok > m)
                lg[v] = NEG_INF;
    }
    bool need = false;
#pragma unroll
    for (int v = 0; v < HPL; ++v)
        need |= lg[v] > st.Ml[v] + LAZY_RESCALE;
    if (__any(need)) {
        float alpha[G];
#pragma unroll
        for (int h = 0; h < G; ++h) {
            const bool mine = G > 4 ? (h / 4 == half) : true;
            const float cand = mine ? lg[h % HPL] : NEG_INF;
            const float mn = fmaxf(st.M[h], wave_max(cand));
            alpha[h] = mn == st.M[h] ? 1.f : exp2f(st.M[h] - mn);   // 0 from -inf
            st.M[h] = mn;
#pragma unroll
            for (int e = 0; e < 8; ++e)
                st.acc[h][e] *= alpha[h];
        }
#pragma unroll
        for (int v = 0; v < HPL; ++v) {
            if constexpr (G > 4) {
                st.L[v] *= lane_pick(half_mask, alpha[4 + v], alpha[v]);
                st.Ml[v] = lane_pick(half_mask, st.M[4 + v], st.M[v]);
            } else {
                st.L[v] *= alpha[v];
                st.Ml[v] = st.M[v];
            }
        }
    }
    float p[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int v = 0; v < HPL; ++v) {
        p[v] = lg[v] == NEG_INF ? 0.f : exp2f(lg[v] - st.Ml[v]);
        st.L[v] += p[v];
    }
    // token t's probabilities -> the lanes holding V rows of token t
    if (q < NPX)
        px[t * NPX + q] = make_float4(p[0], p[1], p[2], p[3]);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    float pt[4][4 * NPX];
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int k = 0; k < NPX; ++k) {
            const float4 x = px[(4 * s + q) * NPX + k];
            pt[s][4 * k + 0] = x.x;
            pt[s][4 * k + 1] = x.y;
            pt[s][4 * k + 2] = x.z;
            pt[s][4 * k + 3] = x.w;
        }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        float vf[8];
        to_f32(r.v[s], vf);
        if (masked && tok0 + 4 * s + q > m) {
#pragma unroll
            for (int e = 0; e < 8; ++e)
                vf[e] = 0.f;
        }
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
            for (int e = 0; e < 8; ++e)
                st.acc[h][e] = fmaf(pt[s][h], vf[e], st.acc[h][e]);
    }
}

__device__ __forceinline__ float row16_max(float v)
{
    v = fmaxf(v, dpp_f<0xB1>(v));
    v = fmaxf(v, dpp_f<0x4E>(v));
    v = fmaxf(v, dpp_f<0x141>(v));
    v = fmaxf(v, dpp_f<0x140>(v));
    return v;
}

// Sum over the four row groups (tokens 4s + r) and, for L, over the 16 token
// lanes of a row holding the head; the first row stores columns 8c .. 8c+7.
template <int G>
__device__ __forceinline__ void store_msummary(MAcc<G> &st, float *dst)
{
    constexpr int HPL = MAcc<G>::HPL;
    const int lane = lane_id(), t = lane & 15, q = lane >> 4;
#pragma unroll
    for (int h = 0; h < G; ++h) {
        float a[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            a[e] = st.acc[h][e];
            a[e] += xor_lanes<16>(a[e]);
            a[e] += xor_lanes<32>(a[e]);
        }
        if (q == 0) {
            float *o = dst + h * SUMM + 8 * t;
            *reinterpret_cast<float4 *>(o) = make_float4(a[0], a[1], a[2], a[3]);
            *reinterpret_cast<float4 *>(o + 4) = make_float4(a[4], a[5], a[6], a[7]);
        }
        if (lane == 0)
            dst[h * SUMM + D] = st.M[h];
    }
#pragma unroll
    for (int v = 0; v < HPL; ++v) {
        const float Lt = row16_sum(st.L[v]);
        if (lane == 0)
            dst[v * SUMM + D + 1] = Lt;
        if (G > 4 && lane == 16)
            dst[((4 + v) % G) * SUMM + D + 1] = Lt;
    }
}

__device__ __forceinline__ uint32_t bf16_rne_bits(float x)
{
    const uint32_t u = __float_as_uint(x);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// A operands of this lane (row l%16 -> head (l%16) % G, k-group l/16) for the
// 4 k-steps, hi and lo parts interleaved: qa[2s] = hi, qa[2s+1] = lo.  hi
// keeps the top 16 bits of the scaled fp32 query; lo = bf16(q - hi), where
// q - hi is exact in fp32.
template <int G>
__device__ __forceinline__ void build_qa(const Shape &s, const State &st, int b, int kvh,
                                         uint4 *qa)
{
    const int lane = lane_id(), row = lane & 15, q = lane >> 4;
    const float *src = st.q_rot + ((long)b * s.Hq + kvh * G + row % G) * D;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        uint32_t hi[8], lo[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float x = src[32 * k + 8 * q + e] * s.scale_log2;
            hi[e] = __float_as_uint(x) >> 16;
            lo[e] = bf16_rne_bits(x - __uint_as_float(hi[e] << 16));
        }
        qa[2 * k] = make_uint4(hi[0] | hi[1] << 16, hi[2] | hi[3] << 16, hi[4] | hi[5] << 16,
                               hi[6] | hi[7] << 16);
        qa[2 * k + 1] = make_uint4(lo[0] | lo[1] << 16, lo[2] | lo[3] << 16, lo[4] | lo[5] << 16,
                                   lo[6] | lo[7] << 16);
    }
}

template <int G>
__global__ __launch_bounds__(BLOCK, G > 4 ? 2 : 3) void complete_mfma_kernel(Shape s, State st,
                                                                     KvView kv)
{
    extern __shared__ int s_off[];
    __shared__ uint4 qlds[WAVES][8][64];   // per wave: 8 A-operand registers x 64 lanes
    __shared__ float4 plds[WAVES][32];     // per wave: probabilities of the page's 16 tokens
    const int nG = s.B * s.Hkv;
    build_plan(s, st, s_off);
    const int P = s_off[nG];
    if (P == 0)
        return;
    const int nW = active_workers(st.n_workers, P);
    const int wv = threadIdx.x >> 6, lane = lane_id();
    const int w = blockIdx.x * WAVES + wv;
    if (w >= nW)
        return;
    long x = (long)w * P / nW;
    const long x1 = (long)(w + 1) * P / nW;
    int g = find_group(s_off, nG, x);
    unsigned long long *bad = &st.stats[ST_BAD_INPUT];
    const uint16_t *kb = reinterpret_cast<const uint16_t *>(kv.k);
    const uint16_t *vb = reinterpret_cast<const uint16_t *>(kv.v);
    while (x < x1) {
        while (s_off[g + 1] <= x)
            ++g;
        const long gend = min((long)s_off[g + 1], x1);
        const int b = g / s.Hkv, kvh = g % s.Hkv;
        const int m = st.m_buf[b];
        const int first_page = st.grp_start[g] / PAGE;
        constexpr int HPL = MAcc<G>::HPL;
        const unsigned long long half_mask = G > 4 ? __ballot((lane >> 4) & 1) : 0ULL;
        int hs[G];
        int hmax = 0;
#pragma unroll
        for (int h = 0; h < G; ++h) {
            hs[h] = st.dec_start[(long)b * s.Hq + kvh * G + h];
            hmax = max(hmax, hs[h]);
        }
        int hsl[HPL];
#pragma unroll
        for (int v = 0; v < HPL; ++v) {
            if constexpr (G > 4)
                hsl[v] = lane_pick(half_mask, hs[(4 + v) % G], hs[v]);
            else
                hsl[v] = hs[v];
        }
        {
            uint4 qa[8];
            build_qa<G>(s, st, b, kvh, qa);
#pragma unroll
            for (int i = 0; i < 8; ++i)
                qlds[wv][i][lane] = qa[i];
        }
        MAcc<G> acc;
#pragma unroll
        for (int h = 0; h < G; ++h) {
            acc.M[h] = NEG_INF;
#pragma unroll
            for (int e = 0; e < 8; ++e)
                acc.acc[h][e] = 0.f;
        }
#pragma unroll
        for (int v = 0; v < HPL; ++v) {
            acc.L[v] = 0.f;
            acc.Ml[v] = NEG_INF;
        }
        int page = first_page + (int)(x - s_off[g]);
        const int last = first_page + (int)(gend - s_off[g]) - 1;
        // one page in flight per wave: at <= 168 VGPRs (G <= 4) three waves
        // share each SIMD, which hides the load latency better than double
        // buffering at two waves per SIMD (measured)
        MPage r0;
        while (true) {
            load_mpage(r0, kv_page<uint16_t>(kv, kb, b, kvh, s.Hkv, page, bad),
                       kv_page<uint16_t>(kv, vb, b, kvh, s.Hkv, page, bad));
            const int tok0 = page * PAGE;
            compute_mpage<G>(r0, &qlds[wv][0][0], plds[wv], tok0, m, hsl,
                             tok0 < hmax || tok0 + PAGE - 1 > m, half_mask, acc);
            if (++page > last)
                break;
        }
        store_msummary<G>(acc, st.partials + ((long)w + g) * G * SUMM);
        x = gend;
    }
}

// ================================================================== reduce
// Grid (Hkv * G, B), 1024 threads: one block per (request, query head).  A
// group's partial summaries (slots w + g, w in [wlo, whi]) can number in the
// hundreds when few long spans share the workers, so the block's 16 waves
// split them (wave k takes wlo + k, wlo + k + 16, ...); each wave forms the
// partials' weights lane-parallel, accumulates its share, and one LDS combine
// follows.  Then the head is merged (+) with the matched entry's stored
// AS_{1:p-r}; writes out (normalised) and keeps AS_{1:m} for amend.
constexpr int REDUCE_WAVES = 16;

template <int G>
__global__ __launch_bounds__(64 * REDUCE_WAVES) void reduce_kernel(Shape s, State st,
                                                                   float *__restrict__ out)
{
    extern __shared__ int s_off[];
    __shared__ float red[REDUCE_WAVES][D + 4];
    const int b = blockIdx.y, kvh = blockIdx.x / G, hh = blockIdx.x % G;
    const int g = b * s.Hkv + kvh;
    const int lane = lane_id(), wv = threadIdx.x >> 6;
    const long idx = (long)b * s.Hq + kvh * G + hh;
    // the stored summary to merge with, fetched before the plan scan
    float2 so = make_float2(0.f, 0.f);
    float Ms = NEG_INF, Ls = 0.f;
    if (wv == 0) {
        const int slot = st.dec_slot[idx];
        if (slot >= 0) {
            const float *rs = st.ring_s + (idx * s.W + slot) * SUMM;
            so = *reinterpret_cast<const float2 *>(rs + 2 * lane);
            Ms = rs[D];
            Ls = rs[D + 1];
        }
    }
    const int nG = s.B * s.Hkv;
    build_plan(s, st, s_off);
    const int P = s_off[nG];
    if (st.m_buf[b] < 0 || s_off[g + 1] == s_off[g])
        return;   // idle request: match wrote its zero output
    const int nW = active_workers(st.n_workers, P);
    const int wlo = page_owner(s_off[g], nW, P);
    const int whi = page_owner((long)s_off[g + 1] - 1, nW, P);
    const float *part = st.partials + hh * SUMM;
    const long pstride = (long)G * SUMM;   // one slot

    // this wave's partials: wlo + wv + REDUCE_WAVES * k
    float Mx = NEG_INF;
    for (int w = wlo + wv + REDUCE_WAVES * lane; w <= whi; w += REDUCE_WAVES * 64)
        Mx = fmaxf(Mx, part[((long)w + g) * pstride + D]);
    Mx = wave_max(Mx);
    const float base = Mx == NEG_INF ? 0.f : Mx;
    float Lw = 0.f, a0 = 0.f, a1 = 0.f;
    for (int w0 = wlo + wv; w0 <= whi; w0 += REDUCE_WAVES * 64) {
        const int wl = w0 + REDUCE_WAVES * lane;
        float sc_l = 0.f;
        if (wl <= whi) {
            const float *pl = part + ((long)wl + g) * pstride;
            sc_l = exp2f(pl[D] - base);
            Lw = fmaf(pl[D + 1], sc_l, Lw);
        }
        const int n = min(64, (whi - w0) / REDUCE_WAVES + 1);
#pragma unroll 8
        for (int k = 0; k < n; ++k) {
            const float sc = __shfl(sc_l, k, 64);
            const float2 v = *reinterpret_cast<const float2 *>(
                part + ((long)w0 + REDUCE_WAVES * k + g) * pstride + 2 * lane);
            a0 = fmaf(v.x, sc, a0);
            a1 = fmaf(v.y, sc, a1);
        }
    }
    Lw = wave_sum(Lw);
    *reinterpret_cast<float2 *>(&red[wv][2 * lane]) = make_float2(a0, a1);
    if (lane == 0) {
        red[wv][D] = Mx;
        red[wv][D + 1] = Lw;
    }
    __syncthreads();
    if (wv != 0)
        return;
    float Mt = NEG_INF;
#pragma unroll
    for (int k = 0; k < REDUCE_WAVES; ++k)
        Mt = fmaxf(Mt, red[k][D]);
    const float bt = Mt == NEG_INF ? 0.f : Mt;
    float c0 = 0.f, c1 = 0.f, Lt = 0.f;
#pragma unroll
    for (int k = 0; k < REDUCE_WAVES; ++k) {
        const float sc = exp2f(red[k][D] - bt);   // 0 for a wave with no partials
        Lt = fmaf(red[k][D + 1], sc, Lt);
        c0 = fmaf(red[k][2 * lane], sc, c0);
        c1 = fmaf(red[k][2 * lane + 1], sc, c1);
    }
    float o0 = c0 / Lt, o1 = c1 / Lt, Mo = Mt, Lo = Lt;
    if (Ls > 0.f) {
        const float Mn = fmaxf(Ms, Mt);
        const float ca = Ls * exp2f(Ms - Mn), cb = Lt * exp2f(Mt - Mn);
        const float Ln = ca + cb;
        o0 = (ca * so.x + cb * o0) / Ln;
        o1 = (ca * so.y + cb * o1) / Ln;
        Mo = Mn;
        Lo = Ln;
    }
    *reinterpret_cast<float2 *>(out + idx * D + 2 * lane) = make_float2(o0, o1);
    float *asf = st.as_full + idx * SUMM;
    *reinterpret_cast<float2 *>(asf + 2 * lane) = make_float2(o0, o1);
    if (lane == 0) {
        asf[D] = Mo;
        asf[D + 1] = Lo;
    }
}

// ================================================================== amend
// Grid (Hkv, B), 8 waves: the waves share the band [m-r+1, m] page by page
// (two or three pages each at r = 256), combine in LDS, then per head
// AS_{1:m-r} = AS_{1:m} (-) band and the ring slot receives (q~_m, AS_{1:m-r}, m).
constexpr int AMEND_WAVES = 8;

template <typename T, int G>
__global__ __launch_bounds__(64 * AMEND_WAVES) void amend_kernel(Shape s, State st, KvView kv,
                                                                 int slot_new)
{
    __shared__ float red[AMEND_WAVES][G][SUMM];
    using K = Kv<T>;
    const int b = blockIdx.y, kvh = blockIdx.x;
    const int lane = lane_id(), wv = threadIdx.x >> 6;
    const int m = st.m_buf[b];
    if (m < 0)
        return;
    const bool has_prefix = m - s.r >= 0;
    if (has_prefix) {
        const int lo = m - s.r + 1;
        int hs[G];
#pragma unroll
        for (int h = 0; h < G; ++h)
            hs[h] = lo;
        float q[G][K::E];
        load_group_queries<T, G>(s, st, b, kvh, q);
        WaveAcc<G, K::E> acc;
        acc.init();
        PageRegs<T> r;
        for (int page = lo / PAGE + wv; page <= m / PAGE; page += AMEND_WAVES) {
            load_page<T>(r, kv_page<T>(kv, kv.k, b, kvh, s.Hkv, page, &st.stats[ST_BAD_INPUT]),
                         kv_page<T>(kv, kv.v, b, kvh, s.Hkv, page, &st.stats[ST_BAD_INPUT]));
            const int tok0 = page * PAGE;
            compute_page<T, G>(r, tok0, m, hs, tok0 < lo || tok0 + PAGE - 1 > m, q, acc);
        }
        store_wave_summary<T, G>(acc, &red[wv][0][0]);
    }
    __syncthreads();
    for (int hh = wv; hh < G; hh += AMEND_WAVES) {
        const long idx = (long)b * s.Hq + kvh * G + hh;
        float so0 = 0.f, so1 = 0.f, sM = NEG_INF, sL = 0.f;   // EMPTY
        if (has_prefix) {
            float Mx = NEG_INF;
#pragma unroll
            for (int w = 0; w < AMEND_WAVES; ++w)
                Mx = fmaxf(Mx, red[w][hh][D]);
            const float base = Mx == NEG_INF ? 0.f : Mx;
            float a0 = 0.f, a1 = 0.f, Lb = 0.f;
#pragma unroll
            for (int w = 0; w < AMEND_WAVES; ++w) {
                const float sc = exp2f(red[w][hh][D] - base);
                Lb = fmaf(red[w][hh][D + 1], sc, Lb);
                a0 = fmaf(red[w][hh][2 * lane], sc, a0);
                a1 = fmaf(red[w][hh][2 * lane + 1], sc, a1);
            }
            const float *z = st.as_full + idx * SUMM;
            const float Mz = z[D], Lz = z[D + 1];
            const float c = Lb * exp2f(Mx - Mz);
            const float l = Lz - c;
            if (l > Lz * 0x1p-24f) {
                const float2 zo = *reinterpret_cast<const float2 *>(z + 2 * lane);
                so0 = (Lz * zo.x - c * (a0 / Lb)) / l;
                so1 = (Lz * zo.y - c * (a1 / Lb)) / l;
                sM = Mz;
                sL = l;
            }
        }
        float *dst = st.ring_s + (idx * s.W + slot_new) * SUMM;
        *reinterpret_cast<float2 *>(dst + 2 * lane) = make_float2(so0, so1);
        if (lane == 0) {
            dst[D] = sM;
            dst[D + 1] = sL;
        }
        const float2 qv = *reinterpret_cast<const float2 *>(st.q_copy + idx * D + 2 * lane);
        *reinterpret_cast<float2 *>(st.ring_q + (idx * s.W + slot_new) * D + 2 * lane) = qv;
    }
    if (kvh == 0 && threadIdx.x == 0)
        st.ring_pos[(long)b * s.W + slot_new] = m;
}

// ================================================================= append
// Grid (Hkv, B), 64 threads: copy one K row and one V row, 16 bytes a thread.
template <typename T>
__global__ __launch_bounds__(64) void append_kernel(Shape s, State st, KvView kv,
                                                    const T *__restrict__ kn,
                                                    const T *__restrict__ vn,
                                                    const int32_t *__restrict__ positions)
{
    constexpr int CH = D * (int)sizeof(T) / 16;
    const int b = blockIdx.y, kvh = blockIdx.x, t = threadIdx.x;
    const int pos = positions[b];
    if (pos < 0)
        return;
    bool bad = pos >= kv.max_seq_len || (kv.paged && pos / PAGE >= kv.max_pages);
    long off = 0;
    if (!bad) {
        if (kv.paged) {
            const int pid = kv.page_table[(long)b * kv.max_pages + pos / PAGE];
            if ((unsigned)pid >= (unsigned)kv.num_pages)
                bad = true;
            else
                off = (((long)pid * s.Hkv + kvh) * PAGE + pos % PAGE) * D;
        } else {
            off = (((long)b * s.Hkv + kvh) * kv.max_seq_len + pos) * D;
        }
    }
    if (bad) {
        if (t == 0 && kvh == 0)
            atomicAdd(&st.stats[ST_BAD_INPUT], 1ULL);
        return;
    }
    const long src = ((long)b * s.Hkv + kvh) * D;
    T *k = reinterpret_cast<T *>(kv.k);
    T *v = reinterpret_cast<T *>(kv.v);
    if (t < CH)
        reinterpret_cast<uint4 *>(k + off)[t] = reinterpret_cast<const uint4 *>(kn + src)[t];
    else if (t < 2 * CH)
        reinterpret_cast<uint4 *>(v + off)[t - CH] =
            reinterpret_cast<const uint4 *>(vn + src)[t - CH];
}

// ================================================================== reset
__global__ void reset_kernel(int32_t *ring_pos, long n_pos, unsigned long long *stats,
                             long n_stats)
{
    const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n_pos)
        ring_pos[i] = -1;
    if (i < n_stats)
        stats[i] = 0ULL;
}

size_t plan_lds_bytes(const Shape &s) { return (size_t)(s.B * s.Hkv + 1) * sizeof(int); }

template <typename T>
hipError_t launch_complete_t(const Shape &s, const State &st, const KvView &kv, int n_blocks,
                             hipStream_t stream)
{
    const size_t lds = plan_lds_bytes(s);
    if constexpr (std::is_same<T, uint16_t>::value) {
        switch (s.G) {
        case 1: hipLaunchKernelGGL(complete_mfma_kernel<1>, dim3(n_blocks), dim3(BLOCK), lds,
                                   stream, s, st, kv); break;
        case 2: hipLaunchKernelGGL(complete_mfma_kernel<2>, dim3(n_blocks), dim3(BLOCK), lds,
                                   stream, s, st, kv); break;
        case 4: hipLaunchKernelGGL(complete_mfma_kernel<4>, dim3(n_blocks), dim3(BLOCK), lds,
                                   stream, s, st, kv); break;
        default: hipLaunchKernelGGL(complete_mfma_kernel<8>, dim3(n_blocks), dim3(BLOCK), lds,
                                    stream, s, st, kv); break;
        }
        return hipGetLastError();
    } else {
        switch (s.G) {
#define MAC_CASE(GG)                                                                          \
    case GG:                                                                                  \
        hipLaunchKernelGGL((complete_kernel<T, GG>), dim3(n_blocks), dim3(BLOCK), lds, stream, \
                           s, st, kv);                                                        \
        break;
            MAC_CASE(1)
            MAC_CASE(2)
            MAC_CASE(4)
            MAC_CASE(8)
#undef MAC_CASE
        default:
            return hipErrorInvalidValue;
        }
        return hipGetLastError();
    }
}

template <typename T>
hipError_t launch_amend_t(const Shape &s, const State &st, const KvView &kv, int slot_new,
                          hipStream_t stream)
{
    const dim3 grid(s.Hkv, s.B);
    switch (s.G) {
#define MAC_CASE(GG)                                                                          \
    case GG:                                                                                  \
        hipLaunchKernelGGL((amend_kernel<T, GG>), grid, dim3(64 * AMEND_WAVES), 0, stream, s,  \
                           st, kv, slot_new);                                                 \
        break;
        MAC_CASE(1)
        MAC_CASE(2)
        MAC_CASE(4)
        MAC_CASE(8)
#undef MAC_CASE
    default:
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

bool supported_group(int G) { return G == 1 || G == 2 || G == 4 || G == 8; }

hipError_t launch_match_tiles(const Shape &s, const State &st, const KvView &kv,
                              const int32_t *seq_lens, const float *q_pre, hipStream_t stream)
{
    const dim3 grid((s.W + TILE_W - 1) / TILE_W, s.Hq, s.B);
    hipLaunchKernelGGL(match_tiles_kernel, grid, dim3(64), 0, stream, s, st, kv, seq_lens, q_pre);
    return hipGetLastError();
}

// LDS a match wave needs: its ring tile and query (none when the ring is scanned
// by match_tiles_kernel).
size_t match_lds_per_wave(const Shape &s)
{
    return s.W > TILE_W ? 0 : (size_t)(s.W * (D + 4) + D) * sizeof(float);
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

hipError_t launch_complete(const Shape &s, const State &st, const KvView &kv, bool kv_fp32,
                           int n_blocks, hipStream_t stream)
{
    return kv_fp32 ? launch_complete_t<float>(s, st, kv, n_blocks, stream)
                   : launch_complete_t<uint16_t>(s, st, kv, n_blocks, stream);
}

hipError_t launch_reduce(const Shape &s, const State &st, float *out, hipStream_t stream)
{
    const size_t lds = plan_lds_bytes(s);
    const dim3 grid(s.Hq, s.B), block(64 * REDUCE_WAVES);
    switch (s.G) {
    case 1: hipLaunchKernelGGL(reduce_kernel<1>, grid, block, lds, stream, s, st, out); break;
    case 2: hipLaunchKernelGGL(reduce_kernel<2>, grid, block, lds, stream, s, st, out); break;
    case 4: hipLaunchKernelGGL(reduce_kernel<4>, grid, block, lds, stream, s, st, out); break;
    case 8: hipLaunchKernelGGL(reduce_kernel<8>, grid, block, lds, stream, s, st, out); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_amend(const Shape &s, const State &st, const KvView &kv, bool kv_fp32,
                        int slot_new, hipStream_t stream)
{
    return kv_fp32 ? launch_amend_t<float>(s, st, kv, slot_new, stream)
                   : launch_amend_t<uint16_t>(s, st, kv, slot_new, stream);
}

hipError_t launch_append(const Shape &s, const State &st, const KvView &kv, bool kv_fp32,
                         const void *k_new, const void *v_new, const int32_t *positions,
                         hipStream_t stream)
{
    const dim3 grid(s.Hkv, s.B);
    if (kv_fp32)
        hipLaunchKernelGGL(append_kernel<float>, grid, dim3(64), 0, stream, s, st, kv,
                           (const float *)k_new, (const float *)v_new, positions);
    else
        hipLaunchKernelGGL(append_kernel<uint16_t>, grid, dim3(64), 0, stream, s, st, kv,
                           (const uint16_t *)k_new, (const uint16_t *)v_new, positions);
    return hipGetLastError();
}

hipError_t launch_reset(const Shape &s, const State &st, hipStream_t stream)
{
    const long n = (long)s.B * s.W;
    const long ns = stats_count(s.B * s.Hkv);
    const long tot = n > ns ? n : ns;
    hipLaunchKernelGGL(reset_kernel, dim3((unsigned)((tot + 255) / 256)), dim3(256), 0, stream,
                       st.ring_pos, n, st.stats, ns);
    return hipGetLastError();
}

int complete_blocks_per_cu(bool kv_fp32, int G, size_t lds)
{
    int n = 0;
    hipError_t e = hipErrorInvalidValue;
#define MAC_OCC(TT, GG)                                                                        \
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, complete_kernel<TT, GG>, BLOCK, lds)
    if (kv_fp32) {
        if (G == 1) MAC_OCC(float, 1); else if (G == 2) MAC_OCC(float, 2);
        else if (G == 4) MAC_OCC(float, 4); else MAC_OCC(float, 8);
    } else {
        if (G == 1)
            e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, complete_mfma_kernel<1>, BLOCK, lds);
        else if (G == 2)
            e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, complete_mfma_kernel<2>, BLOCK, lds);
        else if (G == 4)
            e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, complete_mfma_kernel<4>, BLOCK, lds);
        else
            e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, complete_mfma_kernel<8>, BLOCK, lds);
    }
#undef MAC_OCC
    return (e == hipSuccess && n > 0) ? n : 1;
}

}  // namespace mac
