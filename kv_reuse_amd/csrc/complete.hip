// complete.hip -- complete step of the MAC-Attention decode (Figure 2 (b)):
// split-KV flash-decode over each GQA group's union span, equal page shares
// per wave (the load-balanced plan of Figure 3 (b), built on the device).
#include "mac_device.h"
#include "mfma_page.h"

namespace mac {
namespace {

// =============================================================== complete
// Persistent grid of independent wave workers.  Every block rebuilds the
// plan (a scan over the work list's segments: each group's union span, cut
// before the band when amend is fused) in LDS; the step's pages, segment
// after segment, are split into equal contiguous shares, one per active wave.
// A worker writes one partial summary per segment it touches, into slot
// (worker + segment), which is unique along the flattened list.  Vector
// units only: the fp32 cache, and the bf16 cache at G = 1.
template <typename T, int G>
__global__ __launch_bounds__(BLOCK) void complete_kernel(Shape s, State st, KvView kv)
{
    extern __shared__ int s_off[];
    using K = Kv<T>;
    const int nS = s.B * s.Hkv * s.nseg;
    build_plan(s, st, s_off);
    const int P = s_off[nS];
    if (P == 0)
        return;
    const int nW = s.unbalanced ? st.n_workers : active_workers(st.n_workers, P);
    // the plan is published by the last block when its waves have no pages
    // (a small step), else by block 0 (the first dispatch round, whose waves
    // end first; the last round sets the end of a full launch)
    const int pub = nW <= ((int)gridDim.x - 1) * WAVES ? (int)gridDim.x - 1 : 0;
    if ((int)blockIdx.x == pub)
        publish_plan(s, st, s_off, nW);
    const int w = blockIdx.x * WAVES + (threadIdx.x >> 6);
    if (w >= nW)
        return;
    long x, x1;
    worker_share(s, st, s_off, nS, nW, P, w, x, x1);
    int sg = find_segment(s_off, nS, x);
    unsigned long long *bad = &st.stats[ST_BAD_INPUT];
    while (x < x1) {
        while (s_off[sg + 1] <= x)
            ++sg;
        const long send = min((long)s_off[sg + 1], x1);
        const Seg sd = plan_segment(s, st, s_off, sg);
        const int b = sd.b, kvh = sd.kvh, hi = sd.hi;
        // head h attends keys [max(start_h, lo), hi] of this segment
        int hs[G];
        int hmax = 0;
#pragma unroll
        for (int h = 0; h < G; ++h) {
            hs[h] = max(st.dec_start[(long)b * s.Hq + kvh * G + h], sd.lo);
            hmax = max(hmax, hs[h]);
        }
        const int first_page = sd.lo / PAGE;
        float q[G][K::E];
        load_group_queries<T, G>(s, st, b, kvh, q);
        WaveAcc<G, K::E> acc;
        acc.init();

        PageRegs<T> r0, r1;
        int page = first_page + (int)(x - s_off[sg]);
        const int last = first_page + (int)(send - s_off[sg]) - 1;
        // two pages in flight: while one is computed the next one's loads
        // are out.  fp32: the loop issues them unconditionally and the
        // segment's last one or two pages are peeled (loads under a branch
        // leave the compiler unable to count them, and each compute would
        // then wait for the next page too), and K and V share one page-table
        // lookup; 8 x 64K, 32q/8kv fp32 with the headline queries: complete
        // 200 -> 181 us.  bf16 (G = 1, three waves per SIMD) keeps the guarded
        // form, which measured 0.7 % faster there (16 x 128K, 32 KV heads).
        if constexpr (!std::is_same<T, float>::value) {
            load_page<T>(r0, kv_page<T>(kv, kv.k, b, kvh, s.Hkv, page, bad),
                         kv_page<T>(kv, kv.v, b, kvh, s.Hkv, page, bad));
            while (true) {
                if (page + 1 <= last)
                    load_page<T>(r1, kv_page<T>(kv, kv.k, b, kvh, s.Hkv, page + 1, bad),
                                 kv_page<T>(kv, kv.v, b, kvh, s.Hkv, page + 1, bad));
                {
                    const int tok0 = page * PAGE;
                    compute_page<T, G>(r0, tok0, hi, hs, tok0 < hmax || tok0 + PAGE - 1 > hi, q,
                                       acc);
                }
                if (++page > last)
                    break;
                if (page + 1 <= last)
                    load_page<T>(r0, kv_page<T>(kv, kv.k, b, kvh, s.Hkv, page + 1, bad),
                                 kv_page<T>(kv, kv.v, b, kvh, s.Hkv, page + 1, bad));
                {
                    const int tok0 = page * PAGE;
                    compute_page<T, G>(r1, tok0, hi, hs, tok0 < hmax || tok0 + PAGE - 1 > hi, q,
                                       acc);
                }
                if (++page > last)
                    break;
            }
        } else {
            auto fetch = [&](PageRegs<T> &r, int pg) {
                const T *kp = kv_page<T>(kv, kv.k, b, kvh, s.Hkv, pg, bad);
                load_page<T>(r, kp,
                             static_cast<const T *>(kv.v) + (kp - static_cast<const T *>(kv.k)));
            };
            auto fold = [&](PageRegs<T> &r, int pg) {
                const int tok0 = pg * PAGE;
                compute_page<T, G>(r, tok0, hi, hs, tok0 < hmax || tok0 + PAGE - 1 > hi, q, acc);
            };
            fetch(r0, page);
            while (page + 2 <= last) {
                fetch(r1, page + 1);
                fold(r0, page);
                fetch(r0, page + 2);
                fold(r1, page + 1);
                page += 2;
            }
            if (page + 1 <= last) {
                fetch(r1, page + 1);
                fold(r0, page);
                fold(r1, page + 1);
            } else {
                fold(r0, page);
            }
        }
        store_wave_summary<T, G>(acc, st.partials + ((long)w + sg) * G * SUMM);
        x = send;
    }
}

// ========================================================== complete (MFMA)
// bf16 cache, G >= 2: the page machinery (MFMA Q.K^T, swizzled K tile, lazy
// rescale) is in mfma_page.h.

// Element offsets of the (page, KV head) blocks a wave walks in one segment.
// Paged caches: the page ids are fetched 64 at a time, one per lane, and each
// page reads its id from that lane, so a page's K/V loads wait on no table
// lookup of their own.  An id outside the pool is replaced by page 0
// and counted (once per wave and page).
struct PageWalker {
    const int32_t *row;   // paged: the request's page-table row
    long base;            // contiguous: offset of (request, KV head)
    int kvh, Hkv, num_pages, chunk0, pid_l, last;
    bool paged;

    __device__ __forceinline__ PageWalker(const KvView &kv, int b, int kvh_, int Hkv_, int first,
                                          int last_)
        : kvh(kvh_), Hkv(Hkv_), num_pages(kv.num_pages), chunk0(first - 64), pid_l(0),
          last(last_), paged(kv.paged != 0)
    {
        row = kv.page_table + (long)b * kv.max_pages;
        base = ((long)b * Hkv + kvh) * (long)kv.max_seq_len * D;
    }

    __device__ __forceinline__ long offset(int page, unsigned long long *bad)
    {
        if (!paged)
            return base + (long)page * (PAGE * D);
        if (page >= chunk0 + 64) {
            chunk0 = page;
            const int tp = page + lane_id();
            pid_l = tp <= last ? row[tp] : 0;
        }
        // the lane index is wave-uniform: v_readlane into a scalar register,
        // no LDS round trip (a ds_bpermute would queue behind the page's LDS work)
        int pid = __builtin_amdgcn_readlane(pid_l, page - chunk0);
        if ((unsigned)pid >= (unsigned)num_pages) {
            if (lane_id() == 0)
                atomicAdd(bad, 1ULL);
            pid = 0;
        }
        return ((long)pid * Hkv + kvh) * (PAGE * D);
    }
};

template <int G>
__global__ __launch_bounds__(BLOCK, G > 4 ? 2 : 3) void complete_mfma_kernel(Shape s, State st,
                                                                     KvView kv)
{
    extern __shared__ int s_off[];
    __shared__ uint4 qlds[WAVES][8][64];   // per wave: 8 A-operand registers x 64 lanes
    __shared__ float4 plds[WAVES][32];     // per wave: probabilities of the page's 16 tokens
    __shared__ uint4 klds[WAVES][16 * 16];  // per wave: the page's K rows, swizzled
    const int nS = s.B * s.Hkv * s.nseg;
    build_plan(s, st, s_off);
    const int P = s_off[nS];
    if (P == 0)
        return;
    int nW = s.unbalanced ? st.n_workers : active_workers(st.n_workers, P);
    // Short shares (under 8 pages per wave): only the first two dispatch
    // rounds take part.  The third round's waves start with the lowest issue
    // priority and end last (~4 us after the first round's at 32K x 1); with
    // few pages per wave, 1.5 times the pages on the first two rounds costs
    // less.  Measured, same box: full attention at batch 1 (contiguous) over
    // 63 contexts from 32K to 48K tokens, complete 34.7 -> 33.7 us on average
    // (45 points better by over 0.5 us, 2 worse), 16K x 1 23.0 -> 20.9 us;
    // 128K x 16 with every head hitting (2176 pages) 16.8 -> 15.7 us; paged
    // 1 x 32K and 2 x 16K unchanged; with 10 or more pages per wave on three
    // rounds (64K x 1) it lost 8 %.
    if (!s.unbalanced && tilt_rounds(st) && nW > st.n_workers / st.slots * 2 &&
        P < 8 * st.n_workers)
        nW = st.n_workers / st.slots * 2;
    // the plan is published by the last block when its waves have no pages
    // (a small step), else by block 0 (the first dispatch round, whose waves
    // end first; the last round sets the end of a full launch)
    const int pub = nW <= ((int)gridDim.x - 1) * WAVES ? (int)gridDim.x - 1 : 0;
    if ((int)blockIdx.x == pub)
        publish_plan(s, st, s_off, nW);
    const int wv = threadIdx.x >> 6, lane = lane_id();
    const int w = blockIdx.x * WAVES + wv;
    if (w >= nW)
        return;
    long x, x1;
    worker_share(s, st, s_off, nS, nW, P, w, x, x1);
    int sg = find_segment(s_off, nS, x);
    unsigned long long *bad = &st.stats[ST_BAD_INPUT];
    const uint16_t *kb = reinterpret_cast<const uint16_t *>(kv.k);
    const uint16_t *vb = reinterpret_cast<const uint16_t *>(kv.v);
    while (x < x1) {
        while (s_off[sg + 1] <= x)
            ++sg;
        const long send = min((long)s_off[sg + 1], x1);
        float4 qf[8];   // issued before the segment's bounds are read
        load_qa_rows<G>(s, st, (sg / s.nseg) / s.Hkv, (sg / s.nseg) % s.Hkv, qf);
        const Seg sd = plan_segment(s, st, s_off, sg);
        const int b = sd.b, kvh = sd.kvh, hi = sd.hi;
        constexpr int HPL = MAcc<G>::HPL;
        const unsigned long long half_mask = G > 4 ? __ballot((lane >> 4) & 1) : 0ULL;
        // head h attends keys [max(start_h, lo), hi] of this segment
        int hs[G];
        int hmax = 0;
#pragma unroll
        for (int h = 0; h < G; ++h) {
            hs[h] = max(st.dec_start[(long)b * s.Hq + kvh * G + h], sd.lo);
            hmax = max(hmax, hs[h]);
        }
        const int first_page = sd.lo / PAGE;
        int page = first_page + (int)(x - s_off[sg]);
        const int last = first_page + (int)(send - s_off[sg]) - 1;
        int hsl[HPL];
#pragma unroll
        for (int v = 0; v < HPL; ++v) {
            if constexpr (G > 4)
                hsl[v] = lane_pick(half_mask, hs[(4 + v) % G], hs[v]);
            else
                hsl[v] = hs[v];
        }
        // the segment's first page id is looked up before the A operands are
        // built, so it arrives together with the queries (G > 4: from the
        // lane-gathered table rows)
        PageWalker pw(kv, b, kvh, s.Hkv, page, last);
        const long off0 = G > 4 ? pw.offset(page, bad)
                                : kv_page<uint16_t>(kv, kb, b, kvh, s.Hkv, page, bad) - kb;
        {
            uint4 qa[8];
            build_qa(qf, s.scale_log2, qa);
#pragma unroll
            for (int i = 0; i < 8; ++i)
                qlds[wv][i][lane] = qa[i];
        }
        MPage cur;
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
        if constexpr (G > 4) {
            // two waves per SIMD (G = 8 needs ~220 VGPRs): the next page's
            // loads are issued before the current page is computed
            MPage nxt;
            load_mpage(cur, kb + off0, vb + off0);
            kstore_page(cur, klds[wv]);
            while (true) {
                if (page + 1 <= last) {
                    const long off = pw.offset(page + 1, bad);
                    load_mpage(nxt, kb + off, vb + off);
                }
                const int tok0 = page * PAGE;
                compute_mpage<G>(klds[wv], cur.v, &qlds[wv][0][0], plds[wv], tok0, hi, hsl,
                                 tok0 < hmax || tok0 + PAGE - 1 > hi, half_mask, acc);
                if (++page > last)
                    break;
                kstore_page(nxt, klds[wv]);
                cur.v[0] = nxt.v[0];
                cur.v[1] = nxt.v[1];
                cur.v[2] = nxt.v[2];
                cur.v[3] = nxt.v[3];
            }
        } else {
            // one page in flight per wave: at <= 168 VGPRs three waves share
            // each SIMD, which hides the load latency better than double
            // buffering (which needs more registers than that) does (measured)
            // (the page id comes from a wave-uniform scalar load here: with one
            // page in flight the lane-fetched ids of PageWalker measured slower)
            (void)pw;
            long off = off0;
            while (true) {
                load_mpage(cur, kb + off, vb + off);
                kstore_page(cur, klds[wv]);
                const int tok0 = page * PAGE;
                compute_mpage<G>(klds[wv], cur.v, &qlds[wv][0][0], plds[wv], tok0, hi, hsl,
                                 tok0 < hmax || tok0 + PAGE - 1 > hi, half_mask, acc);
                if (++page > last)
                    break;
                off = kv_page<uint16_t>(kv, kb, b, kvh, s.Hkv, page, bad) - kb;
            }
        }
        store_msummary<G>(acc, st.partials + ((long)w + sg) * G * SUMM);
        x = send;
    }
}

template <typename T>
hipError_t launch_complete_t(const Shape &s, const State &st, const KvView &kv, int n_blocks,
                             hipStream_t stream)
{
    const size_t lds = plan_lds_bytes(s);
    if constexpr (std::is_same<T, uint16_t>::value) {
        // G = 1: one query row is no matrix tile; the vector worker is as fast
        // on streaming steps and faster on short ones (measured), so the
        // matrix cores start at G = 2
        switch (s.G) {
        case 1: hipLaunchKernelGGL((complete_kernel<uint16_t, 1>), dim3(n_blocks), dim3(BLOCK),
                                   lds, stream, s, st, kv); break;
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

}  // namespace

bool supported_group(int G) { return G == 1 || G == 2 || G == 4 || G == 8; }

hipError_t launch_complete(const Shape &s, const State &st, const KvView &kv, bool kv_fp32,
                           int n_blocks, hipStream_t stream)
{
    return kv_fp32 ? launch_complete_t<float>(s, st, kv, n_blocks, stream)
                   : launch_complete_t<uint16_t>(s, st, kv, n_blocks, stream);
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
            e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, complete_kernel<uint16_t, 1>,
                                                             BLOCK, lds);
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
