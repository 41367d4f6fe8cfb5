// amend.hip -- amend step of the MAC-Attention decode (Figure 2 (c)): recompute
// the last-r band, remove it from AS_{1:m} in the log domain, insert the
// (pre-RoPE query, summary) pair into the ring; plus the KV manager's append
// and the ring reset.
#include "mac_device.h"

namespace mac {
namespace {

// ================================================================== amend
// Grid (Hkv, B), 8 waves (4 for 8 query heads per KV head, whose VALU worker
// needs more than the 256 VGPRs two waves per SIMD allow): the waves share the
// band [m-r+1, m] page by page (two to five pages each at r = 256), combine in
// LDS, then per head AS_{1:m-r} = AS_{1:m} (-) band and the ring slot receives
// (q~_m, AS_{1:m-r}, m).
template <int G>
constexpr int amend_waves() { return G > 4 ? 4 : 8; }

template <typename T, int G>
__global__ __launch_bounds__(64 * amend_waves<G>()) void amend_kernel(Shape s, State st, KvView kv,
                                                                      int slot_new)
{
    constexpr int AMEND_WAVES = amend_waves<G>();
    __shared__ float red[AMEND_WAVES][G][SUMM];
    using K = Kv<T>;
    const int b = blockIdx.y, kvh = blockIdx.x;
    const int lane = lane_id(), wv = threadIdx.x >> 6;
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
    for (int hh = wv; hh < G; hh += AMEND_WAVES) {
        const long idx = (long)b * s.Hq + kvh * G + hh;
        float so0 = 0.f, so1 = 0.f, sM = NEG_INF, sL = 0.f;   // EMPTY
        if (m - st.band[kvh * G + hh] >= 0) {
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
        const long row = (idx * s.W + slot_new) * D;
        if (s.ring_bf16)
            reinterpret_cast<uint32_t *>(static_cast<uint16_t *>(st.ring_q) + row)[lane] =
                bf16_rne_bits(qv.x) | bf16_rne_bits(qv.y) << 16;
        else
            reinterpret_cast<float2 *>(static_cast<float *>(st.ring_q) + row)[lane] = qv;
    }
    if (threadIdx.x == 0) {
        if (kvh == 0)
            st.ring_pos[(long)b * s.W + slot_new] = m;
        if (has_prefix)   // this block owns the group's amend counter
            st.grp_stats[((long)b * s.Hkv + kvh) * GRP_NSTAT + GS_TOK_AMEND] +=
                (unsigned long long)(m - lo + 1);
    }
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
hipError_t launch_amend_t(const Shape &s, const State &st, const KvView &kv, int slot_new,
                          hipStream_t stream)
{
    const dim3 grid(s.Hkv, s.B);
    switch (s.G) {
#define MAC_CASE(GG)                                                                          \
    case GG:                                                                                  \
        hipLaunchKernelGGL((amend_kernel<T, GG>), grid, dim3(64 * amend_waves<GG>()), 0, stream, \
                           s, st, kv, slot_new);                                              \
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
    const long ns = stats_count((long)s.B * s.Hq, (long)s.B * s.Hkv);
    const long tot = n > ns ? n : ns;
    hipLaunchKernelGGL(reset_kernel, dim3((unsigned)((tot + 255) / 256)), dim3(256), 0, stream,
                       st.ring_pos, n, st.stats, ns);
    return hipGetLastError();
}

}  // namespace mac
