// reduce.hip -- end of the complete step (Figure 2 (b)): combine the per-wave
// partial summaries of each head and merge them in the log domain with the
// matched ring entry's stored summary AS_{1:p-r}.
#include "mac_device.h"

namespace mac {
namespace {

// ================================================================== reduce
// Grid (Hq, B), 1024 threads: one block per (request, query head).  The
// head's group has n partial summaries (slots w + g for the worker range the
// complete kernel published); n is a few dozen when most groups stream their
// whole context and reaches the thousands when one long span shares the
// workers with short ones.  The block is laid out as RLANES partials x RCH
// float4 column chunks: thread (k, c) folds chunk c of partials k, k + RLANES,
// ... into an online-softmax state (running max, rescaled sums), RUNROLL
// partials per round with all their loads in flight; the RLANES states are
// then combined in LDS.  The head is merged (+) with the matched entry's
// stored AS_{1:p-r}; out receives the normalised output and AS_{1:m} is kept
// for amend.
constexpr int REDUCE_THREADS = 1024;
constexpr int RCH = D / 4;                       // float4 chunks of a row
constexpr int RLANES = REDUCE_THREADS / RCH;     // partials combined side by side
constexpr int RUNROLL = 4;                       // partials per round of loads

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

__global__ __launch_bounds__(REDUCE_THREADS) void reduce_kernel(Shape s, State st,
                                                                float *__restrict__ out)
{
    __shared__ float4 red_o[RLANES][RCH];
    __shared__ float red_l[RLANES], red_m[RLANES];
    const int b = blockIdx.y, h = blockIdx.x, kvh = h / s.G, hh = h % s.G;
    const int g = b * s.Hkv + kvh;
    const int t = threadIdx.x;
    const int c = t % RCH, k = t / RCH;
    const long idx = (long)b * s.Hq + h;
    // the stored summary to merge with (threads 0..RCH-1)
    float4 so = make_float4(0.f, 0.f, 0.f, 0.f);
    float Ms = NEG_INF, Ls = 0.f;
    if (t < RCH) {
        const int slot = st.dec_slot[idx];
        if (slot >= 0) {
            const float *rs = st.ring_s + (idx * s.W + slot) * SUMM;
            so = *reinterpret_cast<const float4 *>(rs + 4 * c);
            Ms = rs[D];
            Ls = rs[D + 1];
        }
    }
    const int2 range = reinterpret_cast<const int2 *>(st.grp_parts)[g];
    if (st.m_buf[b] < 0 || range.y < range.x)
        return;   // idle request: match wrote its zero output
    const int n = range.y - range.x + 1;
    const long pstride = (long)s.G * SUMM;   // one slot
    const float *part = st.partials + ((long)range.x + g) * pstride + hh * SUMM;

    float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
    float L = 0.f, M = NEG_INF;
    for (int i = k; i < n; i += RUNROLL * RLANES) {
        float4 ov[RUNROLL];
        float mv[RUNROLL], lv[RUNROLL];
        const int cnt = min(RUNROLL, (n - i + RLANES - 1) / RLANES);
#pragma unroll
        for (int u = 0; u < RUNROLL; ++u) {
            const int iu = i + u * RLANES;
            if (u < cnt) {
                const float *pi = part + (long)iu * pstride;
                ov[u] = *reinterpret_cast<const float4 *>(pi + 4 * c);
                mv[u] = pi[D];
                lv[u] = pi[D + 1];
            }
        }
        fold(a, L, M, ov, mv, lv, cnt);
    }
    red_o[k][c] = a;
    if (c == 0) {
        red_l[k] = L;
        red_m[k] = M;
    }
    __syncthreads();
    if (t >= RCH)
        return;
    float Mx = red_m[0];
#pragma unroll
    for (int r = 1; r < RLANES; ++r)
        Mx = fmaxf(Mx, red_m[r]);
    const float base = Mx == NEG_INF ? 0.f : Mx;
    float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
    float Lt = 0.f;
#pragma unroll
    for (int r = 0; r < RLANES; ++r) {
        const float sc = exp2f(red_m[r] - base);   // 0 for a lane that saw no partial
        const float4 x = red_o[r][c];
        o.x = fmaf(x.x, sc, o.x);
        o.y = fmaf(x.y, sc, o.y);
        o.z = fmaf(x.z, sc, o.z);
        o.w = fmaf(x.w, sc, o.w);
        Lt = fmaf(red_l[r], sc, Lt);
    }
    o.x /= Lt;
    o.y /= Lt;
    o.z /= Lt;
    o.w /= Lt;
    float Mo = Mx, Lo = Lt;
    if (Ls > 0.f) {
        const float Mn = fmaxf(Ms, Mx);
        const float ca = Ls * exp2f(Ms - Mn), cb = Lt * exp2f(Mx - Mn);
        const float Ln = ca + cb;
        o.x = (ca * so.x + cb * o.x) / Ln;
        o.y = (ca * so.y + cb * o.y) / Ln;
        o.z = (ca * so.z + cb * o.z) / Ln;
        o.w = (ca * so.w + cb * o.w) / Ln;
        Mo = Mn;
        Lo = Ln;
    }
    *reinterpret_cast<float4 *>(out + idx * D + 4 * c) = o;
    float *asf = st.as_full + idx * SUMM;
    *reinterpret_cast<float4 *>(asf + 4 * c) = o;
    if (t == 0) {
        asf[D] = Mo;
        asf[D + 1] = Lo;
    }
}

}  // namespace

hipError_t launch_reduce(const Shape &s, const State &st, float *out, hipStream_t stream)
{
    if (!supported_group(s.G))
        return hipErrorInvalidValue;
    hipLaunchKernelGGL(reduce_kernel, dim3(s.Hq, s.B), dim3(REDUCE_THREADS), 0, stream, s, st,
                       out);
    return hipGetLastError();
}

}  // namespace mac
