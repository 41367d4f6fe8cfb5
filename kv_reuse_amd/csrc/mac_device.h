// mac_device.h -- device helpers shared by the gfx950 kernels of the
// MAC-Attention decode step (match.hip, complete.hip, reduce.hip, amend.hip,
// prefill.hip): wave64 lane exchanges (DPP, ds_swizzle), RoPE, key/value row
// loads, the VALU flash-decode wave worker and the device-side work plan.
//
// Key/value rows stream as 16-byte loads: for bf16 a row of 128 elements is
// 16 lanes, a wave load covers 4 tokens and a 16-token page is 4 loads of K
// and 4 of V; fp32 rows take 32 lanes.
#pragma once
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

// Rotate-half RoPE of the column pair (i, i + D/2) at position m, with
// inv = theta^(-2i/D): the angle m * inv is formed in fp64 and reduced to
// [-pi, pi] in fp64 (Cody-Waite, 2*pi split in two doubles, fma), so sincos
// stays on its short-argument path.
__device__ __forceinline__ void rope_pair(float qa, float qb, int m, double inv, float &ra,
                                          float &rb)
{
    const double phi = (double)m * inv;
    const double k = rint(phi * 0.15915494309189535);   // 1 / (2*pi)
    double red = fma(-k, 6.283185307179586232, phi);      // 2*pi rounded to double
    red = fma(-k, 2.4492935982947064e-16, red);            // 2*pi minus that double
    double sn, cs;
    sincos(red, &sn, &cs);
    ra = (float)((double)qa * cs - (double)qb * sn);
    rb = (float)((double)qb * cs + (double)qa * sn);
}

// bf16 bit pattern of x rounded to nearest, ties to even (finite inputs; an
// overflow rounds to infinity).
__device__ __forceinline__ uint32_t bf16_rne_bits(float x)
{
    const uint32_t u = __float_as_uint(x);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
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
            if (lane_id() == 0)
                atomicAdd(bad, 1ULL);   // once per wave and page
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
// Exclusive prefix sum of a[0..n) in LDS by the whole block (any size up to
// 1024 threads); a[n] = total.
constexpr int MAX_BLOCK_WAVES = 16;

__device__ inline void block_exclusive_scan(int *a, int n)
{
    __shared__ int wsum[MAX_BLOCK_WAVES];
    const int nt = blockDim.x, nwv = nt >> 6;
    const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
    const int per = (n + nt - 1) / nt;
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
    for (int i = 0; i < nwv; ++i) {
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

// First key of group g's union span: the smallest first key of its heads'
// spans (every span ends at the query position m).
__device__ __forceinline__ int group_start(const Shape &s, const State &st, int g)
{
    const int b = g / s.Hkv, kvh = g % s.Hkv;
    const int32_t *ds = st.dec_start + (long)b * s.Hq + kvh * s.G;
    int gs = ds[0];
    for (int h = 1; h < s.G; ++h)
        gs = min(gs, ds[h]);
    return gs;
}

// One segment of the work list: request b, KV head kvh, query position m,
// keys [lo, hi] (empty when lo > hi).  Without fused amend a group's segment
// is its whole union span [start, m]; with it, part 0 is [start, m - r] and
// part 1 the band [m - r + 1, m] (every head's span reaches back past m - r,
// since a hit's p is at most m - 1), so the reduce can form AS_{1:m-r} from
// part 0 and the stored prefix alone.  seg = group * nseg + part.
struct Seg {
    int b, kvh, m, lo, hi;
};

__device__ __forceinline__ Seg segment(const Shape &s, const State &st, int seg)
{
    const int g = seg / s.nseg, part = seg % s.nseg;
    Seg r;
    r.b = g / s.Hkv;
    r.kvh = g % s.Hkv;
    // the heads' starts are loaded together with m (one round trip, not two)
    r.m = st.m_buf[r.b];
    const int gs = group_start(s, st, g);
    r.lo = 0;
    r.hi = -1;
    if (r.m < 0)
        return r;
    if (s.nseg == 1) {
        r.lo = gs;
        r.hi = r.m;
    } else {
        // first key of the band part (the group's heads share one band)
        const int cut = max(gs, r.m - st.band[r.kvh * s.G] + 1);
        r.lo = part == 0 ? gs : cut;
        r.hi = part == 0 ? cut - 1 : r.m;
    }
    return r;
}

__device__ __forceinline__ int segment_pages(const Seg &sg)
{
    return sg.lo > sg.hi ? 0 : sg.hi / PAGE - sg.lo / PAGE + 1;
}

// Page offsets of every segment in the flattened work list: off[i] = pages
// of the segments before i, off[nS] = all pages of the step.  With
// s.plan_bounds the plan also keeps each segment's first key (off[nS + 1 +
// i]) and each request's query position (off[2 nS + 1 + b]), so a wave sets
// up its first segment from LDS and its first page-table lookup goes out
// with its query loads.
__device__ inline void build_plan(const Shape &s, const State &st, int *off)
{
    const int nS = s.B * s.Hkv * s.nseg;
    for (int i = threadIdx.x; i < nS; i += blockDim.x) {
        const Seg sd = segment(s, st, i);
        off[i] = segment_pages(sd);
        if (s.plan_bounds)
            off[nS + 1 + i] = sd.lo;
    }
    if (s.plan_bounds)
        for (int b = threadIdx.x; b < s.B; b += blockDim.x)
            off[2 * nS + 1 + b] = st.m_buf[b];
    __syncthreads();
    block_exclusive_scan(off, nS);
}

// Segment seg as the plan holds it (LDS) or, for long work lists, as
// segment() reads it from the decisions.
__device__ __forceinline__ Seg plan_segment(const Shape &s, const State &st, const int *off, int seg)
{
    if (!s.plan_bounds)
        return segment(s, st, seg);
    const int nS = s.B * s.Hkv * s.nseg;
    const int g = seg / s.nseg, part = seg % s.nseg;
    Seg r;
    r.b = g / s.Hkv;
    r.kvh = g % s.Hkv;
    r.m = off[2 * nS + 1 + r.b];
    r.lo = off[nS + 1 + seg];
    // a fused group's part 0 ends where its band part starts
    r.hi = (s.nseg == 2 && part == 0) ? off[nS + 1 + seg + 1] - 1 : r.m;
    if (r.m < 0) {
        r.lo = 0;
        r.hi = -1;
    }
    return r;
}

// floor(a / b) for 0 <= a < 2^53, b > 0: the fp64 quotient, corrected by one
// where its rounding crossed an integer.
__device__ __forceinline__ long div_floor(long a, int b)
{
    long q = (long)((double)a / (double)b);
    if (q * b > a)
        --q;
    else if ((q + 1) * b <= a)
        ++q;
    return q;
}

// Waves that take part: every worker gets at least MIN_PAGES_PER_WORKER pages.
__device__ __forceinline__ int active_workers(int n_workers, int P)
{
    return min(n_workers, (P + MIN_PAGES_PER_WORKER - 1) / MIN_PAGES_PER_WORKER);
}

// Worker w owns flattened pages [w*P/nW, (w+1)*P/nW); owner of page x:
__device__ __forceinline__ int page_owner(long x, int nW, int P)
{
    return (int)div_floor((x + 1) * (long)nW - 1, P);
}

// Dispatch-round weights.  The grid holds `slots` blocks per CU, dispatched
// round by round (block b in round b / CUs), and the CU's issue arbiter
// favours older waves: with equal shares the first round's waves finish
// first.  At three rounds (G <= 4) the last round also holds the slowest
// waves and sets the end of the launch, so with many pages per wave the
// balanced plan weights the rounds' shares (per mille) by ROUND_W3.  A wave
// timeline at 128K x 16 under 1120 / 1000 / 880 (an earlier, symmetric
// choice) had round 0 ending last (median / max 998 / 1027 us against 960 /
// 995 and 973 / 1018); 1090 / 1030 / 880 then measured, same box, six runs
// each: the mixed step 1080.3 -> 1073.2 us, full attention 1340.5 -> 1333.9
// us (complete 1325.4 -> 1320.0 us).  Other round counts take
// 1000 + SLOT_TILT * (slots - 1 - 2k).
// At two rounds (G = 8) the rounds' slowest waves end together (310 / 312 us
// of 8 x 122880) and weights only lengthened the first round (+2.8 %).
constexpr int ROUND_W3[3] = {1090, 1030, 880};
constexpr int SLOT_TILT = 60;

// (selects with constant indices: an indexed read of the table would be a
// memory load, and the plan calls this in dependent chains)
__device__ __forceinline__ int round_weight(int k, int S)
{
    if (S == 3)
        return k == 0 ? ROUND_W3[0] : k == 1 ? ROUND_W3[1] : ROUND_W3[2];
    return 1000 + SLOT_TILT * (S - 1 - 2 * k);
}

// Three or more dispatch rounds (G <= 4): the rounds' waves end in order.
__device__ __forceinline__ bool tilt_rounds(const State &st) { return st.slots >= 3; }

// (P < 2^26 keeps P * cum(nW) below 2^53 for the fp64 quotient of share_start.)
__device__ __forceinline__ bool tilted_plan(const State &st, int nW, int P)
{
    return tilt_rounds(st) && nW == st.n_workers && P >= 16 * nW && P < (1 << 26);
}

// XCD weights.  The dispatcher hands a launch's blocks to the 8 XCDs in turn
// (block b on XCD b % 8), and a wave timeline at 128K x 16 (mean block end
// per XCD, three runs, each round alike) had the even XCDs' blocks end 30-50
// us after the odd ones' (mixed step ~1030 against ~993 us, full attention
// ~1264 against ~1216 us).  So the tilted plan also weights a wave's share by
// its XCD's parity, 28 : 27 for the odd ones.  Measured, two boxes, four runs
// each: the mixed step 1071.7 -> 1064.1 and 1075.0 -> 1065.6 us, full
// attention 1317.0 -> 1305.0 and 1318.6 -> 1308.8 us; 21 : 20 and 16 : 15
// landed alike, 13 : 12 lost the gain.  Without whole XCD cycles per round
// (CUs not a multiple of 8) the XCD weights are left out.
constexpr int NXCD = 8;
constexpr int XCD_W_EVEN = 27, XCD_W_ODD = 28;

__device__ __forceinline__ int xcd_weight(int x) { return (x & 1) ? XCD_W_ODD : XCD_W_EVEN; }

// Sum of the weights of XCDs 0 .. n-1.
__device__ __forceinline__ int xcd_prefix(int n)
{
    return (n >> 1) * (XCD_W_EVEN + XCD_W_ODD) + ((n & 1) ? XCD_W_EVEN : 0);
}

// Weight of the workers before worker w (nW = slots * Nk workers; worker w is
// wave w % 4 of block w / 4, in round w / Nk, on XCD (w / 4) % 8): round
// weight x XCD weight per worker, summed in closed form.
__device__ __forceinline__ long cum_weight(int w, int Nk, int S)
{
    const int k = w / Nk, j = w % Nk;
    int c = 0;
    for (int i = 0; i < k; ++i)
        c += round_weight(i, S);
    if (Nk % (WAVES * NXCD) != 0)
        return (long)c * Nk + (long)j * round_weight(k, S);
    const long round_x = (long)(Nk / (WAVES * NXCD)) * xcd_prefix(NXCD) * WAVES;
    const int jb = j / WAVES, jw = j % WAVES;
    const long part_x = (long)(jb / NXCD) * xcd_prefix(NXCD) * WAVES +
                        (long)xcd_prefix(jb % NXCD) * WAVES + (long)jw * xcd_weight(jb % NXCD);
    return (long)c * round_x + (long)round_weight(k, S) * part_x;
}

// First flattened page of worker w's share (w = nW gives P).  The weighted
// form is floor(P * cum(w) / cum(nW)), with P * cum(w) < 2^53 (P < 2^26,
// cum(nW) = waves x round x XCD weights < 2^27).
__device__ __forceinline__ long share_start(const State &st, int w, int nW, int P)
{
    if (!tilted_plan(st, nW, P))
        return div_floor((long)w * P, nW);
    const int S = st.slots, Nk = nW / S;
    return div_floor((long)P * cum_weight(w, Nk, S), (int)cum_weight(nW, Nk, S));
}

// Owner of flattened page x under share_start: the last worker whose share
// starts at or before x (every share holds at least 13 pages when tilted).
// Tilting shares of under 16 pages measured slower (same box, three runs:
// complete at 32K x 1, full attention, 32.9 -> 37.1 us with 4 pages as the
// floor), although the last round's waves end ~4 us after the first's there.
__device__ inline int share_owner(const State &st, long x, int nW, int P)
{
    if (!tilted_plan(st, nW, P))
        return page_owner(x, nW, P);
    int lo = 0, hi = nW - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (share_start(st, mid, nW, P) <= x)
            lo = mid;
        else
            hi = mid - 1;
    }
    return lo;
}

// Waves of the unbalanced plan given to each segment (the host checks that
// every segment gets at least one).
__device__ __forceinline__ int waves_per_segment(const State &st, int nS)
{
    return st.n_workers / nS;
}

// Worker w's share [x0, x1) of the flattened page list (x0 >= x1: none).
// Balanced plan (the default, Figure 3 (b)): the nW active waves split all P
// pages of the step evenly (weighted by dispatch round when the shares are
// long), whatever segment they belong to.  Unbalanced plan
// (MAC_F_UNBALANCED_PLAN, the baseline of Figure 8 (b)): every segment gets
// the same k waves, which split that segment's own pages evenly (one wave per
// page when it has fewer than k), so the longest span sets the time.
__device__ __forceinline__ void worker_share(const Shape &s, const State &st, const int *off,
                                             int nS, int nW, int P, int w, long &x0, long &x1)
{
    if (!s.unbalanced) {
        x0 = share_start(st, w, nW, P);
        x1 = share_start(st, w + 1, nW, P);
        return;
    }
    const int k = waves_per_segment(st, nS), sg = w / k, j = w % k;
    x0 = x1 = 0;
    if (sg >= nS)
        return;
    const int n = off[sg + 1] - off[sg], kk = min(k, n);
    if (j >= kk)
        return;
    x0 = off[sg] + (long)j * n / kk;
    x1 = off[sg] + (long)(j + 1) * n / kk;
}

// Last segment i with off[i] <= x, which holds page x (x < off[nS]): up to
// 4096 segments a two-level wave ballot over the LDS offsets (two LDS reads
// per lane), beyond that a binary search.  Called by whole waves.
__device__ __forceinline__ int find_segment(const int *off, int nS, long x)
{
    if (nS <= 64 * 64) {
        const int lane = lane_id();
        const int step = (nS + 63) / 64;
        const int j = lane * step;
        const unsigned long long b1 = __ballot(j < nS && off[j] <= x);   // off[0] = 0 <= x
        const int i0 = (63 - __clzll(b1)) * step;
        const int j2 = i0 + lane;
        const unsigned long long b2 = __ballot(lane < step && j2 < nS && off[j2] <= x);
        return i0 + 63 - __clzll(b2);
    }
    int lo = 0, hi = nS - 1;
    while (lo < hi) {
        int mid = (lo + hi + 1) >> 1;
        if (off[mid] <= x)
            lo = mid;
        else
            hi = mid - 1;
    }
    return lo;
}

// Block 0 of the complete grid records, per segment, the first and last
// worker whose share touches it (the slots of its partial summaries), so the
// reduce needs no plan of its own, and adds the keys each group streams this
// step (m - start + 1, its segments together) to the group's counter, which
// only this block writes.  Empty segments get the range (0, -1).
__device__ inline void publish_plan(const Shape &s, const State &st, const int *off, int nW)
{
    const int nG = s.B * s.Hkv, nS = nG * s.nseg, P = off[nS];
    const int k = s.unbalanced ? waves_per_segment(st, nS) : 0;
    for (int i = threadIdx.x; i < nS; i += blockDim.x) {
        int2 r = make_int2(0, -1);
        const int n = off[i + 1] - off[i];
        if (n > 0 && s.unbalanced)
            r = make_int2(i * k, i * k + min(k, n) - 1);
        else if (n > 0)
            r = make_int2(share_owner(st, off[i], nW, P),
                          share_owner(st, (long)off[i + 1] - 1, nW, P));
        reinterpret_cast<int2 *>(st.grp_parts)[i] = r;
    }
    for (int g = threadIdx.x; g < nG; g += blockDim.x) {
        const int m = st.m_buf[g / s.Hkv];
        if (m >= 0)
            st.grp_stats[(long)g * GRP_NSTAT + GS_TOK_CRIT] +=
                (unsigned long long)(m - group_start(s, st, g) + 1);
    }
}

// Bytes of LDS the plan (one int per segment, plus the total) occupies.
inline size_t plan_lds_bytes(const Shape &s)
{
    const size_t nS = (size_t)s.B * s.Hkv * s.nseg;
    return (s.plan_bounds ? 2 * nS + 1 + s.B : nS + 1) * sizeof(int);
}

}  // namespace
}  // namespace mac
