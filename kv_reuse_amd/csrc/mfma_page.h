// mfma_page.h -- one wave folds a 16-token page of a bf16 KV cache into the
// running summaries of a GQA group's heads, Q.K^T on the matrix cores.  Used
// by the complete kernel (the split-KV flash-decode of Figure 2 (b)) and by
// amend (its band recompute, Figure 2 (c)).
#pragma once
#include "mac_device.h"

namespace mac {

// bf16 cache, G <= 8 query heads per KV head.  Q.K^T runs on the matrix cores:
// v_mfma_f32_16x16x32_bf16 with the page's 16 tokens as the 16 columns of B
// (lane l feeds token l%16, columns 32s + 8(l/16) .. +7 at k-step s, read
// from the wave's swizzled LDS copy of the page) and the group's queries as the rows of A,
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

// K and V both arrive as contiguous 1 KB wave loads of whole 128-byte lines
// (lane (q, t) = (l/16, l%16) holds token 4s + q, columns 8t .. 8t+7), with a
// streaming hint: every line is read once, by one instruction.  K then passes
// through the wave's LDS tile into the MFMA layout (see kstore_page).
__device__ __forceinline__ void load_mpage(MPage &r, const uint16_t *kp, const uint16_t *vp)
{
    const int lane = lane_id(), t = lane & 15, q = lane >> 4;
#pragma unroll
    for (int s = 0; s < 4; ++s)
        r.k[s] = load_stream(kp + (4 * s + q) * D + 8 * t);
#pragma unroll
    for (int s = 0; s < 4; ++s)
        r.v[s] = load_stream(vp + (4 * s + q) * D + 8 * t);
}

// The MFMA B operand wants lane l to hold token l%16, columns 32s + 8(l/16) ..
// +7 at k-step s: read straight from memory, each wave load would cover half
// of every line it touches.  Instead the page's K rows (16 rows x 16 chunks of
// 16 bytes) go through a 4 KB per-wave LDS tile, chunk c of row j stored at
// slot c ^ j: the writes of a wave load fill whole rows, and the reads of the
// MFMA layout (16 rows, one chunk index each) land on 16 distinct slots, so
// neither side has bank conflicts.  compute_mpage reads each k-step's operand
// from the tile just before its MFMA.
__device__ __forceinline__ void kstore_page(const MPage &r, uint4 *tile)
{
    const int lane = lane_id(), t = lane & 15, q = lane >> 4;
#pragma unroll
    for (int s = 0; s < 4; ++s)
        tile[(4 * s + q) * 16 + (t ^ (4 * s + q))] = r.k[s];
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
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

// Fold one page (tokens tok0 .. tok0+15) into the wave's state.  hsl: first
// key of each of this lane's own heads' spans; hi: the segment's last key.
// half_mask: lanes holding heads 4..7 (G = 8; zero otherwise).
template <int G>
__device__ __forceinline__ void compute_mpage(const uint4 *ktile, const uint4 (&vr)[4], const uint4 *qa, float4 *px,
                                              int tok0, int hi, const int (&hsl)[MAcc<G>::HPL],
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
        const bf16x8 kb = __builtin_bit_cast(bf16x8, ktile[t * 16 + ((4 * s + q) ^ t)]);
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
            if (tok < hsl[v] || tok > hi)
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
        to_f32(vr[s], vf);
        if (masked && tok0 + 4 * s + q > hi) {
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

// This lane's query values for the MFMA A operand (row l%16 -> head
// (l%16) % G, k-group l/16): columns 32k + 8(l/16) .. +7 for the 4 k-steps,
// two float4 each.  Loaded on their own so they can be in flight while the
// segment's bounds are read.
template <int G>
__device__ __forceinline__ void load_qa_rows(const Shape &s, const State &st, int b, int kvh,
                                             float4 (&qf)[8])
{
    const int lane = lane_id(), row = lane & 15, q = lane >> 4;
    const float4 *src = reinterpret_cast<const float4 *>(
        st.q_rot + ((long)b * s.Hq + kvh * G + row % G) * D);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        qf[2 * k] = src[(32 * k + 8 * q) / 4];
        qf[2 * k + 1] = src[(32 * k + 8 * q) / 4 + 1];
    }
}

// The A operands for the 4 k-steps, hi and lo parts interleaved: qa[2s] = hi,
// qa[2s+1] = lo.  hi keeps the top 16 bits of the scaled fp32 query; lo =
// bf16(q - hi), where q - hi is exact in fp32.
__device__ __forceinline__ void build_qa(const float4 (&qf)[8], float scale, uint4 *qa)
{
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const float v[8] = {qf[2 * k].x, qf[2 * k].y, qf[2 * k].z, qf[2 * k].w,
                            qf[2 * k + 1].x, qf[2 * k + 1].y, qf[2 * k + 1].z, qf[2 * k + 1].w};
        uint32_t hi[8], lo[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float x = v[e] * scale;
            hi[e] = __float_as_uint(x) >> 16;
            lo[e] = bf16_rne_bits(x - __uint_as_float(hi[e] << 16));
        }
        qa[2 * k] = make_uint4(hi[0] | hi[1] << 16, hi[2] | hi[3] << 16, hi[4] | hi[5] << 16,
                               hi[6] | hi[7] << 16);
        qa[2 * k + 1] = make_uint4(lo[0] | lo[1] << 16, lo[2] | lo[3] << 16, lo[4] | lo[5] << 16,
                                   lo[6] | lo[7] << 16);
    }
}

}  // namespace mac
