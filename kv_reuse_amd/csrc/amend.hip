// amend.hip -- amend step of the MAC-Attention decode (Figure 2 (c)): recompute
// the last-r band, remove it from AS_{1:m} in the log domain, insert the
// (pre-RoPE query, summary) pair into the ring; plus the KV manager's append
// and the ring reset.
#include "mac_device.h"
#include "mfma_page.h"

namespace mac {
namespace {

// ================================================================== amend
// fp32 caches, and bf16 ones at G = 1 (one query row is no matrix tile; the
// vector worker measured as fast there); bf16 at G >= 2 takes
// amend_mfma_kernel below.
// Grid (Hkv, B), 8 waves (4 for 8 query heads per KV head, whose VALU worker
// needs more than the 256 VGPRs two waves per SIMD allow): the waves share the
// band [m-r+1, m] page by page (two to five pages each at r = 256), combine in
// LDS, then per head AS_{1:m-r} = AS_{1:m} (-) band and the ring slot receives
// (q~_m, AS_{1:m-r}, m).
template <int G>
constexpr int amend_waves() { return G > 4 ? 4 : 8; }

// The inputs of amend's epilogue for the heads hh = wv, wv + NW, ... that
// wave wv finishes: AS_{1:m} and the pre-RoPE query (two columns per lane).
// Loaded before the band, so they are in flight with the pages.
template <int G, int NW>
struct AmendIn {
    static constexpr int HPW = (G + NW - 1) / NW;
    float2 zo[HPW], qv[HPW];
    float zM[HPW], zL[HPW];

    __device__ __forceinline__ void load(const Shape &s, const State &st, int b, int kvh)
    {
        const int lane = lane_id(), wv = threadIdx.x >> 6;
#pragma unroll
        for (int j = 0; j < HPW; ++j) {
            const int hh = wv + j * NW;
            if (hh < G) {
                const long idx = (long)b * s.Hq + kvh * G + hh;
                const float *z = st.as_full + idx * SUMM;
                zo[j] = *reinterpret_cast<const float2 *>(z + 2 * lane);
                zM[j] = z[D];
                zL[j] = z[D + 1];
                qv[j] = *reinterpret_cast<const float2 *>(st.q_copy + idx * D + 2 * lane);
            }
        }
    }
};

// The end of amend for one group, after the waves' band summaries are in red
// (unnormalised o, M, l per wave and head): per head AS_{1:m-r} = AS_{1:m} (-)
// band (EMPTY when m - r_h < 0, or when the removal leaves under 2^-24 of l),
// written with the pre-RoPE query into the ring slot of this step; then the
// slot's position and the group's amend counter.
template <int G, int NW>
__device__ __forceinline__ void amend_finish(const Shape &s, const State &st,
                                             const float (&red)[NW][G][SUMM],
                                             const AmendIn<G, NW> &in, int b, int kvh, int m,
                                             int lo, bool has_prefix, int slot_new)
{
    const int lane = lane_id(), wv = threadIdx.x >> 6;
#pragma unroll
    for (int j = 0; j < AmendIn<G, NW>::HPW; ++j) {
        const int hh = wv + j * NW;
        if (hh >= G)
            break;
        const long idx = (long)b * s.Hq + kvh * G + hh;
        float so0 = 0.f, so1 = 0.f, sM = NEG_INF, sL = 0.f;   // EMPTY
        if (m - st.band[kvh * G + hh] >= 0) {
            float Mx = NEG_INF;
#pragma unroll
            for (int w = 0; w < NW; ++w)
                Mx = fmaxf(Mx, red[w][hh][D]);
            const float base = Mx == NEG_INF ? 0.f : Mx;
            float a0 = 0.f, a1 = 0.f, Lb = 0.f;
#pragma unroll
            for (int w = 0; w < NW; ++w) {
                const float sc = exp2f(red[w][hh][D] - base);
                Lb = fmaf(red[w][hh][D + 1], sc, Lb);
                a0 = fmaf(red[w][hh][2 * lane], sc, a0);
                a1 = fmaf(red[w][hh][2 * lane + 1], sc, a1);
            }
            const float Mz = in.zM[j], Lz = in.zL[j];
            const float c = Lb * exp2f(Mx - Mz);
            const float l = Lz - c;
            if (l > Lz * 0x1p-24f) {
                so0 = (Lz * in.zo[j].x - c * (a0 / Lb)) / l;
                so1 = (Lz * in.zo[j].y - c * (a1 / Lb)) / l;
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
        const long row = (idx * s.W + slot_new) * D;
        if (s.ring_bf16)
            reinterpret_cast<uint32_t *>(static_cast<uint16_t *>(st.ring_q) + row)[lane] =
                bf16_rne_bits(in.qv[j].x) | bf16_rne_bits(in.qv[j].y) << 16;
        else
            reinterpret_cast<float2 *>(static_cast<float *>(st.ring_q) + row)[lane] = in.qv[j];
    }
    if (threadIdx.x == 0) {
        if (kvh == 0)
            st.ring_pos[(long)b * s.W + slot_new] = m;
        if (has_prefix)   // this block owns the group's amend counter
            st.grp_stats[((long)b * s.Hkv + kvh) * GRP_NSTAT + GS_TOK_AMEND] +=
                (unsigned long long)(m - lo + 1);
    }
}

template <typename T, int G>
__global__ __launch_bounds__(64 * amend_waves<G>()) void amend_kernel(Shape s, State st, KvView kv)
{
    constexpr int AMEND_WAVES = amend_waves<G>();
    __shared__ float red[AMEND_WAVES][G][SUMM];
    using K = Kv<T>;
    const int b = blockIdx.y, kvh = blockIdx.x;
    const int wv = threadIdx.x >> 6;
    const int m = st.m_buf[b];
    if (m < 0)
        return;
    // head h removes its own band [m - r_h + 1, m] (nothing when m - r_h < 0:
    // its stored summary is EMPTY); the waves walk the union of the bands
    int hs[G];
    int lo = m + 1, hmax = 0;
#pragma unroll
    for (int h = 0; h < G; ++h) {
        const int rh = st.band[kvh * G + h];
        hs[h] = m - rh >= 0 ? m - rh + 1 : m + 1;
        lo = min(lo, hs[h]);
        hmax = max(hmax, hs[h]);
    }
    AmendIn<G, AMEND_WAVES> in;
    in.load(s, st, b, kvh);
    const bool has_prefix = lo <= m;   // some head keeps a prefix
    if (has_prefix) {
        float q[G][K::E];
        load_group_queries<T, G>(s, st, b, kvh, q);
        WaveAcc<G, K::E> acc;
        acc.init();
        PageRegs<T> r;
        for (int page = lo / PAGE + wv; page <= m / PAGE; page += AMEND_WAVES) {
            load_page<T>(r, kv_page<T>(kv, kv.k, b, kvh, s.Hkv, page, &st.stats[ST_BAD_INPUT]),
                         kv_page<T>(kv, kv.v, b, kvh, s.Hkv, page, &st.stats[ST_BAD_INPUT]));
            const int tok0 = page * PAGE;
            compute_page<T, G>(r, tok0, m, hs, tok0 < hmax || tok0 + PAGE - 1 > m, q, acc);
        }
        store_wave_summary<T, G>(acc, &red[wv][0][0]);
    }
    __syncthreads();
    amend_finish<G, AMEND_WAVES>(s, st, red, in, b, kvh, m, lo, has_prefix, *st.step_slot);
}

// bf16 caches, G >= 2: the band's pages go through the MFMA page path of
// complete (mfma_page.h), 8 waves per group for every G (G = 8 fits two waves
// per SIMD there).  The waves share one copy of the group's A operands in LDS; wave w
// takes pages lo/16 + w, + 8, ..., the next page's loads in flight while one
// is computed; the epilogue is amend_finish.
constexpr int AMEND_MFMA_WAVES = 8;

template <int G>
__global__ __launch_bounds__(64 * AMEND_MFMA_WAVES) void amend_mfma_kernel(Shape s, State st,
                                                                          KvView kv)
{
    constexpr int NW = AMEND_MFMA_WAVES;
    constexpr int HPL = MAcc<G>::HPL;
    __shared__ uint4 qlds[8][64];            // the group's A operands (hi, lo per k-step)
    __shared__ float4 plds[NW][32];          // per wave: probabilities of the page's tokens
    __shared__ uint4 klds[NW][16 * 16];      // per wave: the page's K rows, swizzled
    __shared__ float red[NW][G][SUMM];
    const int b = blockIdx.y, kvh = blockIdx.x;
    const int lane = lane_id(), wv = threadIdx.x >> 6;
    const int m = st.m_buf[b];
    if (m < 0)
        return;
    int hs[G];
    int lo = m + 1, hmax = 0;
#pragma unroll
    for (int h = 0; h < G; ++h) {
        const int rh = st.band[kvh * G + h];
        hs[h] = m - rh >= 0 ? m - rh + 1 : m + 1;
        lo = min(lo, hs[h]);
        hmax = max(hmax, hs[h]);
    }
    const bool has_prefix = lo <= m;   // block-uniform
    AmendIn<G, NW> in;
    in.load(s, st, b, kvh);
    const uint16_t *kb = reinterpret_cast<const uint16_t *>(kv.k);
    const uint16_t *vb = reinterpret_cast<const uint16_t *>(kv.v);
    unsigned long long *bad = &st.stats[ST_BAD_INPUT];
    // this wave's pages are lo/16 + wv, + NW, ...; the first one's loads are
    // issued before the barrier that publishes the A operands
    const int p_last = m / PAGE;
    int page = lo / PAGE + wv;
    MPage cur, nxt;
    // (K and V share a page's element offset: one page-table lookup per page)
    if (has_prefix && page <= p_last) {
        const long off = kv_page<uint16_t>(kv, kb, b, kvh, s.Hkv, page, bad) - kb;
        load_mpage(cur, kb + off, vb + off);
    }
    if (has_prefix && wv == 0) {
        float4 qf[8];
        load_qa_rows<G>(s, st, b, kvh, qf);
        uint4 qa[8];
        build_qa(qf, s.scale_log2, qa);
#pragma unroll
        for (int i = 0; i < 8; ++i)
            qlds[i][lane] = qa[i];
    }
    __syncthreads();
    if (has_prefix) {
        const unsigned long long half_mask = G > 4 ? __ballot((lane >> 4) & 1) : 0ULL;
        int hsl[HPL];
#pragma unroll
        for (int v = 0; v < HPL; ++v) {
            if constexpr (G > 4)
                hsl[v] = lane_pick(half_mask, hs[(4 + v) % G], hs[v]);
            else
                hsl[v] = hs[v];
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
        // the next page's loads go out before this page is computed; the
        // loop issues them unconditionally and the wave's last page is
        // peeled, since loads under a branch leave the compiler unable to
        // count them and the K store would then wait for the next page too
        while (page + NW <= p_last) {
            const long off = kv_page<uint16_t>(kv, kb, b, kvh, s.Hkv, page + NW, bad) - kb;
            load_mpage(nxt, kb + off, vb + off);
            kstore_page(cur, klds[wv]);
            const int tok0 = page * PAGE;
            compute_mpage<G>(klds[wv], cur.v, &qlds[0][0], plds[wv], tok0, m, hsl,
                             tok0 < hmax || tok0 + PAGE - 1 > m, half_mask, acc);
            page += NW;
            cur = nxt;
        }
        if (page <= p_last) {
            kstore_page(cur, klds[wv]);
            const int tok0 = page * PAGE;
            compute_mpage<G>(klds[wv], cur.v, &qlds[0][0], plds[wv], tok0, m, hsl,
                             tok0 < hmax || tok0 + PAGE - 1 > m, half_mask, acc);
        }
        store_msummary<G>(acc, &red[wv][0][0]);
    }
    __syncthreads();
    amend_finish<G, NW>(s, st, red, in, b, kvh, m, lo, has_prefix, *st.step_slot);
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

template <typename T>
hipError_t launch_amend_t(const Shape &s, const State &st, const KvView &kv, hipStream_t stream)
{
    const dim3 grid(s.Hkv, s.B);
    switch (s.G) {
#define MAC_CASE(GG)                                                                          \
    case GG:                                                                                  \
        if constexpr (sizeof(T) == 2 && GG > 1)                                               \
            hipLaunchKernelGGL(amend_mfma_kernel<GG>, grid, dim3(64 * AMEND_MFMA_WAVES), 0,    \
                               stream, s, st, kv);                                            \
        else                                                                                  \
            hipLaunchKernelGGL((amend_kernel<T, GG>), grid, dim3(64 * amend_waves<GG>()), 0,   \
                               stream, s, st, kv);                                            \
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

hipError_t launch_amend(const Shape &s, const State &st, const KvView &kv, bool kv_fp32,
                        hipStream_t stream)
{
    return kv_fp32 ? launch_amend_t<float>(s, st, kv, stream)
                   : launch_amend_t<uint16_t>(s, st, kv, stream);
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
    const long ns = stats_count((long)s.B * s.Hq, (long)s.B * s.Hkv);
    const long tot = n > ns ? n : ns;
    hipLaunchKernelGGL(reset_kernel, dim3((unsigned)((tot + 255) / 256)), dim3(256), 0, stream,
                       st.ring_pos, n, st.stats, ns);
    return hipGetLastError();
}

}  // namespace mac
