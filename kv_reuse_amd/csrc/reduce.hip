// reduce.hip -- end of the complete step (Figure 2 (b)): combine the per-wave
// partial summaries of each head and merge them in the log domain with the
// matched ring entry's stored summary AS_{1:p-r}.
#include "mac_device.h"

namespace mac {
namespace {

// ================================================================== reduce
// Grid (Hq, B, slices), REDUCE_THREADS threads: each (request, query head) is
// combined by `slices` blocks, block z taking the row's float4 column chunks
// [z CH, (z + 1) CH) of every partial (CH = 32 / slices) together with the
// partials' (M, l), which every slice reads, so all slices agree on the
// scales.  Each segment of the head's group has n partial summaries (slots
// w + segment for the worker range the complete kernel published); n is a
// few dozen when most groups stream their whole context and reaches the
// thousands when one long span shares the workers with short ones.  A block
// is laid out as 512 / CH partial lanes x CH chunks: thread (k, c) folds
// chunk c of partials k, k + lanes, ... into an online-softmax state (running
// max, rescaled sums), RUNROLL partials per round with all their loads in
// flight (RLONG per round while a whole such round is left), and the lanes'
// states are then combined in LDS.  Narrower slices give a long list more
// lanes, so fewer dependent rounds of loads.
//
// Then, per head, with the matched entry's stored prefix S = AS_{1:p-r}
// (EMPTY on a miss) and (+) the log-domain merge:
//   one segment:  O = S (+) span; AS_{1:m} = O is kept for amend;
//   fused amend:  X = S (+) part 0 is AS_{1:m-r} and goes into the ring slot
//                 of this step together with the pre-RoPE query and m;
//                 O = X (+) band.
// out receives O's normalised output.
constexpr int REDUCE_THREADS = 512;
constexpr int RCH = D / 4;                       // float4 chunks of a row
constexpr int RUNROLL = 4;                       // partials per round of loads
constexpr int RLONG = 8;                         // the same, for long lists

// A summary as threads 0..CH-1 hold it: normalised output chunk c (o), the
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

template <int U>
__device__ __forceinline__ void fold(float4 &a, float &L, float &M, const float4 (&ov)[U],
                                     const float (&mv)[U], const float (&lv)[U], int cnt)
{
    float mn = M;
#pragma unroll
    for (int u = 0; u < U; ++u)
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
    for (int u = 0; u < U; ++u) {
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

template <int CH>
struct ReduceLds {
    static constexpr int LANES = REDUCE_THREADS / CH;   // partials combined side by side
    float4 o[LANES][CH];
    float l[LANES], m[LANES];
};

// Combine NSETS (1 or 2) sets of partials -- set j: n_j rows at part_j,
// part_j + pstride, ... (this head's rows) -- over the CH chunks starting at
// float `col0` into normalised summaries r0, r1, valid in threads 0..CH-1
// (EMPTY for a set with no rows).  The block's partial lanes are split evenly
// between the sets, so both are read in the same rounds.  Every thread of the
// block calls it (one barrier).
template <int NSETS, int CH>
__device__ __forceinline__ void combine_partials(const float *part0, int n0, const float *part1,
                                                 int n1, long pstride, int col0,
                                                 ReduceLds<CH> &lds, Sum4 &r0, Sum4 &r1)
{
    constexpr int LANES = ReduceLds<CH>::LANES;
    constexpr int PER = LANES / NSETS;   // partial lanes per set
    const int t = threadIdx.x, c = t % CH, k = t / CH;
    const int set = k / PER, kk = k % PER;
    const float *part = set == 0 ? part0 : part1;
    const int n = set == 0 ? n0 : n1;
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
    float L = 0.f, M = NEG_INF;
    int i = kk;
    for (; i + (RLONG - 1) * PER < n; i += RLONG * PER) {
        float4 ov[RLONG];
        float mv[RLONG], lv[RLONG];
#pragma unroll
        for (int u = 0; u < RLONG; ++u) {
            const float *pi = part + (long)(i + u * PER) * pstride;
            ov[u] = *reinterpret_cast<const float4 *>(pi + col0 + 4 * c);
            const float2 ml = *reinterpret_cast<const float2 *>(pi + D);
            mv[u] = ml.x;
            lv[u] = ml.y;
        }
        fold<RLONG>(a, L, M, ov, mv, lv, RLONG);
    }
    for (; i < n; i += RUNROLL * PER) {
        float4 ov[RUNROLL];
        float mv[RUNROLL], lv[RUNROLL];
        const int cnt = min(RUNROLL, (n - i + PER - 1) / PER);
#pragma unroll
        for (int u = 0; u < RUNROLL; ++u) {
            if (u < cnt) {
                const float *pi = part + (long)(i + u * PER) * pstride;
                ov[u] = *reinterpret_cast<const float4 *>(pi + col0 + 4 * c);
                mv[u] = pi[D];
                lv[u] = pi[D + 1];
            }
        }
        fold<RUNROLL>(a, L, M, ov, mv, lv, cnt);
    }
    lds.o[k][c] = a;
    if (c == 0) {
        lds.l[k] = L;
        lds.m[k] = M;
    }
    __syncthreads();
    if (t >= 64)
        return;
    // wave 0: lanes [j TPS, (j + 1) TPS) finish set j; lane jj CH + c of a
    // set folds chunk c of lanes jj, jj + J, ..., then the J folds of a chunk
    // meet by lane exchanges (lanes CH, 2 CH, ... apart, inside the set)
    constexpr int TPS = 64 / NSETS;
    constexpr int J = TPS / CH;
    static_assert(J >= 1 && J * CH == TPS, "chunk count must divide the set's lanes");
    const int q0 = (t / TPS) * PER, jj = (t % TPS) / CH;
    float Mx = NEG_INF;
#pragma unroll
    for (int q = jj; q < PER; q += J)
        Mx = fmaxf(Mx, lds.m[q0 + q]);
#pragma unroll
    for (int off = CH; off < TPS; off <<= 1)
        Mx = fmaxf(Mx, __shfl_xor(Mx, off, 64));
    const float base = Mx == NEG_INF ? 0.f : Mx;
    float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
    float Lt = 0.f;
#pragma unroll
    for (int q = jj; q < PER; q += J) {
        const float sc = exp2f(lds.m[q0 + q] - base);   // 0 for a lane that saw no partial
        const float4 x = lds.o[q0 + q][c];
        o.x = fmaf(x.x, sc, o.x);
        o.y = fmaf(x.y, sc, o.y);
        o.z = fmaf(x.z, sc, o.z);
        o.w = fmaf(x.w, sc, o.w);
        Lt = fmaf(lds.l[q0 + q], sc, Lt);
    }
#pragma unroll
    for (int off = CH; off < TPS; off <<= 1) {
        o.x += __shfl_xor(o.x, off, 64);
        o.y += __shfl_xor(o.y, off, 64);
        o.z += __shfl_xor(o.z, off, 64);
        o.w += __shfl_xor(o.w, off, 64);
        Lt += __shfl_xor(Lt, off, 64);
    }
    Sum4 r;
    r.o = make_float4(0.f, 0.f, 0.f, 0.f);
    r.M = NEG_INF;
    r.L = 0.f;
    if (Lt > 0.f) {
        r.o = make_float4(o.x / Lt, o.y / Lt, o.z / Lt, o.w / Lt);
        r.M = Mx;
        r.L = Lt;
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

// 512 threads at <= 128 VGPRs: two blocks per CU, so a CU works on two heads
// at once (1024-thread blocks, one per CU, took two rounds over the CUs for
// 512 heads and measured ~2 us slower on short steps).
template <int CH>
__global__ __launch_bounds__(REDUCE_THREADS) __attribute__((amdgpu_waves_per_eu(4))) void
reduce_kernel(Shape s, State st, float *__restrict__ out)
{
    __shared__ ReduceLds<CH> lds;
    const int b = blockIdx.y, h = blockIdx.x, kvh = h / s.G, hh = h % s.G;
    const int g = b * s.Hkv + kvh;
    const int t = threadIdx.x;
    const int chunk = (int)blockIdx.z * CH + t % CH;   // this thread's float4 column chunk
    const long idx = (long)b * s.Hq + h;
    // the stored summary to merge with (threads 0..CH-1)
    Sum4 S;
    S.o = make_float4(0.f, 0.f, 0.f, 0.f);
    S.M = NEG_INF;
    S.L = 0.f;
    if (t < CH) {
        const int slot = st.dec_slot[idx];
        if (slot >= 0) {
            const float *rs = st.ring_s + (idx * s.W + slot) * SUMM;
            S.o = *reinterpret_cast<const float4 *>(rs + 4 * chunk);
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
    const float *p0 = st.partials + ((long)rg0.x + seg0) * pstride + hh * SUMM;
    const int col0 = 4 * CH * (int)blockIdx.z;
    Sum4 part0, part1;
    if (s.nseg == 2)
        combine_partials<2, CH>(p0, rg0.y - rg0.x + 1,
                                st.partials + ((long)rg1.x + seg0 + 1) * pstride + hh * SUMM,
                                rg1.y - rg1.x + 1, pstride, col0, lds, part0, part1);
    else
        combine_partials<1, CH>(p0, rg0.y - rg0.x + 1, nullptr, 0, pstride, col0, lds, part0,
                                part1);
    if (t >= CH)
        return;
    const bool lead = blockIdx.z == 0 && t == 0;   // writes the scalars
    Sum4 O;
    if (s.nseg == 1) {
        O = merge(S, part0);
        float *asf = st.as_full + idx * SUMM;
        *reinterpret_cast<float4 *>(asf + 4 * chunk) = O.o;
        if (lead) {
            asf[D] = O.M;
            asf[D + 1] = O.L;
        }
    } else {
        const Sum4 X = merge(S, part0);   // AS_{1:m-r}
        O = merge(X, part1);
        const int slot_new = *st.step_slot;   // this call's ring slot (match)
        float *dst = st.ring_s + (idx * s.W + slot_new) * SUMM;
        *reinterpret_cast<float4 *>(dst + 4 * chunk) = X.o;
        const float4 qv = *reinterpret_cast<const float4 *>(st.q_copy + idx * D + 4 * chunk);
        const long row = (idx * s.W + slot_new) * D;
        if (s.ring_bf16)
            reinterpret_cast<uint2 *>(static_cast<uint16_t *>(st.ring_q) + row)[chunk] =
                make_uint2(bf16_rne_bits(qv.x) | bf16_rne_bits(qv.y) << 16,
                           bf16_rne_bits(qv.z) | bf16_rne_bits(qv.w) << 16);
        else
            reinterpret_cast<float4 *>(static_cast<float *>(st.ring_q) + row)[chunk] = qv;
        if (lead) {
            dst[D] = X.M;
            dst[D + 1] = X.L;
            if (h == 0)
                st.ring_pos[(long)b * s.W + slot_new] = m;
        }
    }
    *reinterpret_cast<float4 *>(out + idx * D + 4 * chunk) = O.o;
}

}  // namespace

hipError_t launch_reduce(const Shape &s, const State &st, float *out, hipStream_t stream)
{
    if (!supported_group(s.G) || s.nseg < 1 || s.nseg > 2)
        return hipErrorInvalidValue;
    // column slices per head while the blocks stay within one per CU: at
    // 32 heads, four slices took the reduce from 10.1-11.6 to 8.7-9.3 us
    // (32K x 1); at 512 heads (128K x 16) two and four slices cost 2.5 and
    // 7 us (same box, HIP events)
    const long heads = (long)s.B * s.Hq;
    const long n_cu = st.n_workers / (st.slots * WAVES);
    const int slices = 4 * heads <= n_cu ? 4 : 2 * heads <= n_cu ? 2 : 1;
    switch (slices) {
    case 4: hipLaunchKernelGGL(reduce_kernel<RCH / 4>, dim3(s.Hq, s.B, 4), dim3(REDUCE_THREADS), 0,
                               stream, s, st, out); break;
    case 2: hipLaunchKernelGGL(reduce_kernel<RCH / 2>, dim3(s.Hq, s.B, 2), dim3(REDUCE_THREADS), 0,
                               stream, s, st, out); break;
    default: hipLaunchKernelGGL(reduce_kernel<RCH>, dim3(s.Hq, s.B, 1), dim3(REDUCE_THREADS), 0,
                                stream, s, st, out); break;
    }
    return hipGetLastError();
}

}  // namespace mac
