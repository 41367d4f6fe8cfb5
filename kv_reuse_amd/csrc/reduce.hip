// reduce.hip -- end of the complete step (Figure 2 (b)): combine the per-wave
// partial summaries of each head and merge them in the log domain with the
// matched ring entry's stored summary AS_{1:p-r}.
#include "mac_device.h"

namespace mac {
namespace {

// ================================================================== reduce
// Grid (Hq, B), 1024 threads: one block per (request, query head).  Each
// segment of the head's group has n partial summaries (slots w + segment for
// the worker range the complete kernel published); n is a few dozen when
// most groups stream their whole context and reaches the thousands when one
// long span shares the workers with short ones.  The block is laid out as
// RLANES partials x RCH float4 column chunks: thread (k, c) folds chunk c of
// partials k, k + RLANES, ... into an online-softmax state (running max,
// rescaled sums), RUNROLL partials per round with all their loads in flight;
// the RLANES states are then combined in LDS.
//
// Then, per head, with the matched entry's stored prefix S = AS_{1:p-r}
// (EMPTY on a miss) and (+) the log-domain merge:
//   one segment:  O = S (+) span; AS_{1:m} = O is kept for amend;
//   fused amend:  X = S (+) part 0 is AS_{1:m-r} and goes into the ring slot
//                 of this step together with the pre-RoPE query and m;
//                 O = X (+) band.
// out receives O's normalised output.
//
// When the grid has fewer heads than the GPU has CUs (a small batch), a head
// whose segments hold more than SPLIT_MIN partials (say one missing head among
// hits, its span cut over thousands of waves) is folded by gridDim.z = RSPLIT
// blocks, each over an equal part of the partials.  Each writes its summaries
// to split_buf, then adds one to the head's counter (agent-scope fence
// before, so the other XCDs' L2s see the summaries); the block that brings it
// to RSPLIT (fence after) folds the RSPLIT summaries, finishes the head as
// above and clears the counter for the next step.  Otherwise block z = 0 does
// the whole head and the others return at once.  With a block per CU or more
// already in the grid, splitting measured slower (1097 -> 1102 us at 128K x 16,
// 101 -> 112 us on its all-hit steps); at batch 1 x 32 heads it takes the
// reduce from 15.0 to 11.6 us.
constexpr int REDUCE_THREADS = 1024;
constexpr int RCH = D / 4;                       // float4 chunks of a row
constexpr int RLANES = REDUCE_THREADS / RCH;     // partials combined side by side
constexpr int RUNROLL = 4;                       // partials per round of loads
constexpr int RSPLIT = REDUCE_SPLIT;             // blocks per head for long partial lists
constexpr int SPLIT_MIN = 256;                   // partials above which a head is split

// A summary as threads 0..RCH-1 hold it: normalised output chunk c (o), the
// reference max M (log2 units) and the normaliser L; EMPTY is (0, -inf, 0).
struct Sum4 {
    float4 o;
    float M, L;
};

// X (+) Y for the chunk this thread holds.
__device__ __forceinline__ Sum4 merge(const Sum4 &x, const Sum4 &y)
{
    if (!(y.L > 0.f))
        return x;
    if (!(x.L > 0.f))
        return y;
    const float Mn = fmaxf(x.M, y.M);
    const float ca = x.L * exp2f(x.M - Mn), cb = y.L * exp2f(y.M - Mn);
    const float Ln = ca + cb;
    Sum4 r;
    r.o.x = (ca * x.o.x + cb * y.o.x) / Ln;
    r.o.y = (ca * x.o.y + cb * y.o.y) / Ln;
    r.o.z = (ca * x.o.z + cb * y.o.z) / Ln;
    r.o.w = (ca * x.o.w + cb * y.o.w) / Ln;
    r.M = Mn;
    r.L = Ln;
    return r;
}

__device__ __forceinline__ void fold(float4 &a, float &L, float &M, const float4 (&ov)[RUNROLL],
                                     const float (&mv)[RUNROLL], const float (&lv)[RUNROLL], int cnt)
{
    float mn = M;
#pragma unroll
    for (int u = 0; u < RUNROLL; ++u)
        if (u < cnt)
            mn = fmaxf(mn, mv[u]);
    if (mn == NEG_INF)
        return;   // nothing but empty partials so far
    const float al = exp2f(M - mn);   // 0 when M is -inf
    a.x *= al;
    a.y *= al;
    a.z *= al;
    a.w *= al;
    L *= al;
    M = mn;
#pragma unroll
    for (int u = 0; u < RUNROLL; ++u) {
        if (u < cnt) {
            const float sc = exp2f(mv[u] - mn);
            a.x = fmaf(ov[u].x, sc, a.x);
            a.y = fmaf(ov[u].y, sc, a.y);
            a.z = fmaf(ov[u].z, sc, a.z);
            a.w = fmaf(ov[u].w, sc, a.w);
            L = fmaf(lv[u], sc, L);
        }
    }
}

struct ReduceLds {
    float4 o[RLANES][RCH];
    float l[RLANES], m[RLANES];
};

// Combine NSETS (1 or 2) sets of partials -- set j: n_j rows at part_j,
// part_j + pstride, ... (this head's rows) -- into normalised summaries r0,
// r1, valid in threads 0..RCH-1 (EMPTY for a set with no rows).  The block's
// RLANES partial lanes are split evenly between the sets, so both are read in
// the same rounds.  Every thread of the block calls it (one barrier).
template <int NSETS>
__device__ __forceinline__ void combine_partials(const float *part0, int n0, const float *part1,
                                                 int n1, long pstride, ReduceLds &lds, Sum4 &r0,
                                                 Sum4 &r1)
{
    constexpr int PER = RLANES / NSETS;   // partial lanes per set
    const int t = threadIdx.x, c = t % RCH, k = t / RCH;
    const int set = k / PER, kk = k % PER;
    const float *part = set == 0 ? part0 : part1;
    const int n = set == 0 ? n0 : n1;
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
    float L = 0.f, M = NEG_INF;
    for (int i = kk; i < n; i += RUNROLL * PER) {
        float4 ov[RUNROLL];
        float mv[RUNROLL], lv[RUNROLL];
        const int cnt = min(RUNROLL, (n - i + PER - 1) / PER);
#pragma unroll
        for (int u = 0; u < RUNROLL; ++u) {
            if (u < cnt) {
                const float *pi = part + (long)(i + u * PER) * pstride;
                ov[u] = *reinterpret_cast<const float4 *>(pi + 4 * c);
                mv[u] = pi[D];
                lv[u] = pi[D + 1];
            }
        }
        fold(a, L, M, ov, mv, lv, cnt);
    }
    lds.o[k][c] = a;
    if (c == 0) {
        lds.l[k] = L;
        lds.m[k] = M;
    }
    __syncthreads();
    if (t >= 64)
        return;
    // wave 0: lanes 32j .. 32j+31 finish set j (set 0 only when NSETS == 1)
    Sum4 r;
    r.o = make_float4(0.f, 0.f, 0.f, 0.f);
    r.M = NEG_INF;
    r.L = 0.f;
    const int mine = t / RCH;
    if (mine < NSETS) {
        const int q0 = mine * PER;
        float Mx = lds.m[q0];
#pragma unroll
        for (int q = 1; q < PER; ++q)
            Mx = fmaxf(Mx, lds.m[q0 + q]);
        const float base = Mx == NEG_INF ? 0.f : Mx;
        float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
        float Lt = 0.f;
#pragma unroll
        for (int q = 0; q < PER; ++q) {
            const float sc = exp2f(lds.m[q0 + q] - base);   // 0 for a lane that saw no partial
            const float4 x = lds.o[q0 + q][c];
            o.x = fmaf(x.x, sc, o.x);
            o.y = fmaf(x.y, sc, o.y);
            o.z = fmaf(x.z, sc, o.z);
            o.w = fmaf(x.w, sc, o.w);
            Lt = fmaf(lds.l[q0 + q], sc, Lt);
        }
        if (Lt > 0.f) {
            r.o = make_float4(o.x / Lt, o.y / Lt, o.z / Lt, o.w / Lt);
            r.M = Mx;
            r.L = Lt;
        }
    }
    r0 = r;
    if constexpr (NSETS == 2) {
        r1.o.x = __shfl(r.o.x, t + 32, 64);
        r1.o.y = __shfl(r.o.y, t + 32, 64);
        r1.o.z = __shfl(r.o.z, t + 32, 64);
        r1.o.w = __shfl(r.o.w, t + 32, 64);
        r1.M = __shfl(r.M, t + 32, 64);
        r1.L = __shfl(r.L, t + 32, 64);
    } else {
        r1 = r;
    }
}

__global__ __launch_bounds__(REDUCE_THREADS) void reduce_kernel(Shape s, State st,
                                                                float *__restrict__ out,
                                                                int slot_new)
{
    __shared__ ReduceLds lds;
    const int b = blockIdx.y, h = blockIdx.x, kvh = h / s.G, hh = h % s.G;
    const int g = b * s.Hkv + kvh;
    const int t = threadIdx.x, c = t % RCH;
    const long idx = (long)b * s.Hq + h;
    // the stored summary to merge with (threads 0..RCH-1)
    Sum4 S;
    S.o = make_float4(0.f, 0.f, 0.f, 0.f);
    S.M = NEG_INF;
    S.L = 0.f;
    if (t < RCH) {
        const int slot = st.dec_slot[idx];
        if (slot >= 0) {
            const float *rs = st.ring_s + (idx * s.W + slot) * SUMM;
            S.o = *reinterpret_cast<const float4 *>(rs + 4 * c);
            S.M = rs[D];
            S.L = rs[D + 1];
        }
    }
    // loaded together with the position (independent loads, one round trip)
    const int2 *ranges = reinterpret_cast<const int2 *>(st.grp_parts);
    const int seg0 = g * s.nseg;
    const int2 rg0 = ranges[seg0];
    const int2 rg1 = s.nseg == 2 ? ranges[seg0 + 1] : make_int2(0, -1);
    const int m = st.m_buf[b];
    if (m < 0)
        return;   // idle request: match wrote its zero output, nothing is stored
    const long pstride = (long)s.G * SUMM;   // one slot
    const int n0 = rg0.y - rg0.x + 1, n1 = rg1.y - rg1.x + 1;
    const int nsplit = gridDim.z;   // RSPLIT or 1
    const bool split = nsplit > 1 && n0 + n1 > SPLIT_MIN;
    const int z = blockIdx.z;
    if (!split && z > 0)
        return;
    // this block's part of each set: all of it, or the z-th of RSPLIT parts
    const int a0 = split ? (int)((long)z * n0 / nsplit) : 0;
    const int e0 = split ? (int)((long)(z + 1) * n0 / nsplit) : n0;
    const int a1 = split ? (int)((long)z * n1 / nsplit) : 0;
    const int e1 = split ? (int)((long)(z + 1) * n1 / nsplit) : n1;
    const float *p0 = st.partials + ((long)rg0.x + a0 + seg0) * pstride + hh * SUMM;
    Sum4 part0, part1;
    if (s.nseg == 2)
        combine_partials<2>(p0, e0 - a0,
                            st.partials + ((long)rg1.x + a1 + seg0 + 1) * pstride + hh * SUMM,
                            e1 - a1, pstride, lds, part0, part1);
    else
        combine_partials<1>(p0, e0 - a0, nullptr, 0, pstride, lds, part0, part1);
    if (t >= 64)
        return;
    if (split) {
        // wave 0 alone from here: publish this block's summaries, count in
        float *mine = st.split_buf + ((idx * RSPLIT + z) * 2) * SUMM;
        if (t < RCH) {
            *reinterpret_cast<float4 *>(mine + 4 * c) = part0.o;
            *reinterpret_cast<float4 *>(mine + SUMM + 4 * c) = part1.o;
            if (t == 0) {
                mine[D] = part0.M;
                mine[D + 1] = part0.L;
                mine[SUMM + D] = part1.M;
                mine[SUMM + D + 1] = part1.L;
            }
        }
        __threadfence();
        int prior = 0;
        if (t == 0)
            prior = atomicAdd(&st.split_cnt[idx], 1);
        prior = __shfl(prior, 0, 64);
        if (prior != nsplit - 1)
            return;   // another block finishes this head
        __threadfence();
        if (t < RCH) {
            Sum4 x0, x1;
            x0.o = x1.o = make_float4(0.f, 0.f, 0.f, 0.f);
            x0.M = x1.M = NEG_INF;
            x0.L = x1.L = 0.f;
            for (int q = 0; q < nsplit; ++q) {
                const float *o = st.split_buf + ((idx * RSPLIT + q) * 2) * SUMM;
                Sum4 y0, y1;
                y0.o = *reinterpret_cast<const float4 *>(o + 4 * c);
                y0.M = o[D];
                y0.L = o[D + 1];
                y1.o = *reinterpret_cast<const float4 *>(o + SUMM + 4 * c);
                y1.M = o[SUMM + D];
                y1.L = o[SUMM + D + 1];
                x0 = merge(x0, y0);
                x1 = merge(x1, y1);
            }
            part0 = x0;
            part1 = x1;
        }
        if (t == 0)
            st.split_cnt[idx] = 0;   // ready for the next step
    }
    if (t >= RCH)
        return;
    Sum4 O;
    if (s.nseg == 1) {
        O = merge(S, part0);
        float *asf = st.as_full + idx * SUMM;
        *reinterpret_cast<float4 *>(asf + 4 * c) = O.o;
        if (t == 0) {
            asf[D] = O.M;
            asf[D + 1] = O.L;
        }
    } else {
        const Sum4 X = merge(S, part0);   // AS_{1:m-r}
        O = merge(X, part1);
        float *dst = st.ring_s + (idx * s.W + slot_new) * SUMM;
        *reinterpret_cast<float4 *>(dst + 4 * c) = X.o;
        const float4 qv = *reinterpret_cast<const float4 *>(st.q_copy + idx * D + 4 * c);
        const long row = (idx * s.W + slot_new) * D;
        if (s.ring_bf16)
            reinterpret_cast<uint2 *>(static_cast<uint16_t *>(st.ring_q) + row)[c] =
                make_uint2(bf16_rne_bits(qv.x) | bf16_rne_bits(qv.y) << 16,
                           bf16_rne_bits(qv.z) | bf16_rne_bits(qv.w) << 16);
        else
            reinterpret_cast<float4 *>(static_cast<float *>(st.ring_q) + row)[c] = qv;
        if (t == 0) {
            dst[D] = X.M;
            dst[D + 1] = X.L;
            if (h == 0)
                st.ring_pos[(long)b * s.W + slot_new] = m;
        }
    }
    *reinterpret_cast<float4 *>(out + idx * D + 4 * c) = O.o;
}

}  // namespace

hipError_t launch_reduce(const Shape &s, const State &st, float *out, int slot_new,
                         hipStream_t stream)
{
    if (!supported_group(s.G) || s.nseg < 1 || s.nseg > 2)
        return hipErrorInvalidValue;
    const int n_cu = st.n_workers / (WAVES * (st.slots > 0 ? st.slots : 1));
    const int nsplit = (long)s.B * s.Hq < n_cu ? RSPLIT : 1;
    hipLaunchKernelGGL(reduce_kernel, dim3(s.Hq, s.B, nsplit), dim3(REDUCE_THREADS), 0, stream, s,
                       st, out, slot_new);
    return hipGetLastError();
}

}  // namespace mac
