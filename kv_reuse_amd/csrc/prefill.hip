// prefill.hip -- MAC-Attention over the prompt (the pages' Table 8 ablation:
// reuse enabled in prefill as well as in decode, with an unbounded window).
//
// Prompt token t of a request is a decode step at position t over keys
// [0, t]: it matches the pre-RoPE queries of every earlier prompt token of its
// (request, query head) and, on a hit at p, attends only [p - r + 1, t] and
// merges the summary p stored, AS_{1:p-r}.  Token t stores AS_{1:t-r}.  The
// decisions depend on the queries alone, so all of them are taken at once.
// The stored summaries chain: with the band split of the fused amend,
//   S_t = S_p (+) A(q_t, [lo_t, t - r])      (S_p = EMPTY on a miss),
//   O_t = S_t (+) A(q_t, [max(lo_t, t - r + 1), t]),
// so every token's two pieces are computed independently and S is resolved
// by pointer jumping along the parent links t -> p in ceil(log2 N) rounds.
//
// Kernels, in launch order:
//   prefill_rope    RoPE of every prompt query (fp64 angle)
//   prefill_match   nearest earlier query per token, fp32 distances, newest
//                   wins ties; threshold and override as in decode
//   prefill_attend  one wave per (request, KV head, token): the two pieces of
//                   each head of the group, unnormalised
//   prefill_count   counters (tokens, decisions, hits, keys), one atomic
//                   per (request, KV head) block
//   prefill_chain_init / _step / prefill_out   the scan and O
#include <mutex>

#include "mac_device.h"

namespace mac {

// Scratch of mac_prefill_noalloc: one array per GPU, held from the library's
// load until the process ends.  Host code never passes `scratch` itself to a
// kernel (on the host the name is a stand-in, not a device address): it takes
// the device address once per device, at mac_init, and uses that.
static __device__ __align__(256) unsigned char scratch[PREFILL_STATIC_BYTES];

namespace {

constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[MAX_DEVICES] = {};

}  // namespace

hipError_t prefill_static_scratch_init(int device)
{
    if (device < 0 || device >= MAX_DEVICES)
        return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[device])
        return hipSuccess;
    void *p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess)
        return e;
    g_scratch_ptr[device] = p;
    return hipSuccess;
}

void *prefill_static_scratch(int device)
{
    if (device < 0 || device >= MAX_DEVICES)
        return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    return g_scratch_ptr[device];
}

namespace {

// Scratch of one prefill call (device memory; rows = B * N * Hq, row index
// (b * N + t) * Hq + h).
struct Pf {
    int N;          // rows per request (the call's num_tokens)
    float *qrot;    // [rows][D] post-RoPE queries
    int32_t *p;     // [rows] matched position, -1 on a miss
    int32_t *lo;    // [rows] first key of the span
    float *part;    // [B][N][2][Hq][SUMM] unnormalised pieces 0 and 1
    float *sa, *sb; // [rows][SUMM] normalised chain summaries (ping-pong)
    int32_t *pa, *pb;   // [rows] chain parents (ping-pong)
};

// A request's prompt length n (tokens 0 .. n-1), 0 for an idle request; a
// length beyond the rows given or the cache is bad input (request idled).
__device__ __forceinline__ int prompt_len(const KvView &kv, int seq, int N, bool &bad)
{
    bad = seq > N || (seq > 0 && (seq - 1 >= kv.max_seq_len ||
                                  (kv.paged && (seq - 1) / PAGE >= kv.max_pages)));
    return (bad || seq < 0) ? 0 : seq;
}

__device__ __forceinline__ long row3(const Pf &pf, int Hq, int b, int t, int h)
{
    return ((long)b * pf.N + t) * Hq + h;
}

// Kernels over rows (request, token, head) run one wave per row, ROW_WAVES
// rows per block; RowId decodes the row index (b * N + t) * Hq + h.
constexpr int ROW_WAVES = 4;

struct RowId {
    long r;
    int b, t, h;
    bool valid;
};

__device__ __forceinline__ RowId row_id(const Shape &s, const Pf &pf)
{
    RowId x;
    x.r = (long)blockIdx.x * ROW_WAVES + (threadIdx.x >> 6);
    x.valid = x.r < (long)s.B * pf.N * s.Hq;
    x.h = (int)(x.r % s.Hq);
    x.t = (int)((x.r / s.Hq) % pf.N);
    x.b = (int)(x.r / ((long)s.Hq * pf.N));
    return x;
}

// ==================================================================== rope
__global__ __launch_bounds__(64 * ROW_WAVES) void prefill_rope_kernel(
    Shape s, State st, KvView kv, Pf pf, const int32_t *__restrict__ seq_lens,
    const float *__restrict__ q_pre)
{
    const RowId x = row_id(s, pf);
    if (!x.valid)
        return;
    const int h = x.h, t = x.t, b = x.b, lane = lane_id();
    bool bad;
    if (t >= prompt_len(kv, seq_lens[b], pf.N, bad))
        return;
    const long i = row3(pf, s.Hq, b, t, h) * D;
    float ra, rb;
    rope_pair(q_pre[i + lane], q_pre[i + lane + 64], t, st.inv_freq[lane], ra, rb);
    pf.qrot[i + lane] = ra;
    pf.qrot[i + lane + 64] = rb;
}

// =================================================================== match
// Grid (ceil(N/64), Hq, B), 4 waves: lane l of every wave holds the query of
// token 64 * tile + l in registers.  The candidates (the pre-RoPE queries of
// earlier tokens, rounded to bf16 with MAC_F_RING_BF16) pass through LDS in
// chunks of PFM_CHUNK rows, double-buffered: the block loads chunk c + 1 into
// registers while its waves scan chunk c, wave w taking rows w, w + 4, ...; a
// candidate row is the same for every lane, so its reads are LDS broadcasts.
// (Rows read straight through the scalar cache ran at ~40 % of the VALU
// rate: each quarter row waited on its scalar loads.)  Distances are direct
// fp32 sums of squared differences: the Gram form |a|^2 + |b|^2 - 2 a.b would
// lose about 1e-5 of the distance to cancellation for the nearest rows, the
// size of the near-tie margin.  The four partial winners of a token are then
// combined (smaller distance, then the later token).
constexpr int PFM_WAVES = 4;
constexpr int PFM_CHUNK = 16;                          // candidate rows per LDS stage
constexpr int PFM_LOADS = PFM_CHUNK * (D / 4) / (64 * PFM_WAVES);   // float4 per thread

template <bool BF16>
__global__ __launch_bounds__(64 * PFM_WAVES) void prefill_match_kernel(
    Shape s, State st, KvView kv, Pf pf, const int32_t *__restrict__ seq_lens,
    const float *__restrict__ q_pre, const int32_t *__restrict__ ovr, int32_t *__restrict__ p_out)
{
    __shared__ float bd[PFM_WAVES][64];
    __shared__ int bjs[PFM_WAVES][64];
    __shared__ float4 rows[2][PFM_CHUNK][D / 4];
    const int tile = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int lane = lane_id(), wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    bool bad;
    const int n = prompt_len(kv, seq_lens[b], pf.N, bad);
    const int t0 = tile * 64;
    const int t = t0 + lane;
    const bool act = t < n;
    if (t0 >= n) {
        if (bad && tile == 0 && h == 0 && threadIdx.x == 0)
            atomicAdd(&st.stats[ST_BAD_INPUT], 1ULL);
        if (wv == 0 && p_out && t < pf.N)
            p_out[row3(pf, s.Hq, b, t, h)] = -1;   // rows of no token
        return;
    }
    float4 q[D / 4];
    {
        const float4 *src = reinterpret_cast<const float4 *>(
            q_pre + row3(pf, s.Hq, b, act ? t : t0, h) * D);
#pragma unroll
        for (int k = 0; k < D / 4; ++k)
            q[k] = src[k];
    }
    float best = INFINITY;
    int bj = -1;
    if (s.reuse) {
        // candidates 0 .. jend: every earlier token of the tile's last token
        const int jend = min(t0 + 63, n - 1);
        const int nch = (jend + PFM_CHUNK) / PFM_CHUNK;
        float4 pre[PFM_LOADS];
        // thread x moves float4 x, x + 256, ... of a chunk (row e / 32, column e % 32)
        auto gload = [&](int c) {
#pragma unroll
            for (int i = 0; i < PFM_LOADS; ++i) {
                const int e = threadIdx.x + i * 64 * PFM_WAVES;
                const int j = c * PFM_CHUNK + e / (D / 4);
                pre[i] = j <= jend ? reinterpret_cast<const float4 *>(
                                         q_pre + row3(pf, s.Hq, b, j, h) * D)[e % (D / 4)]
                                   : make_float4(0.f, 0.f, 0.f, 0.f);
            }
        };
        auto lstore = [&](int buf) {
#pragma unroll
            for (int i = 0; i < PFM_LOADS; ++i) {
                const int e = threadIdx.x + i * 64 * PFM_WAVES;
                float4 c = pre[i];
                if constexpr (BF16) {
                    c.x = __uint_as_float(bf16_rne_bits(c.x) << 16);
                    c.y = __uint_as_float(bf16_rne_bits(c.y) << 16);
                    c.z = __uint_as_float(bf16_rne_bits(c.z) << 16);
                    c.w = __uint_as_float(bf16_rne_bits(c.w) << 16);
                }
                rows[buf][e / (D / 4)][e % (D / 4)] = c;
            }
        };
        gload(0);
        lstore(0);
        __syncthreads();
        for (int c = 0; c < nch; ++c) {
            if (c + 1 < nch)
                gload(c + 1);   // in flight while this chunk is scanned
            const int cur = c & 1;
            for (int r = wv; r < PFM_CHUNK; r += PFM_WAVES) {
                const int j = c * PFM_CHUNK + r;
                if (j > jend)
                    break;
                // four partial sums (one per float4 component) break the chain
                // of dependent fmas; their order of addition is fixed
                float da = 0.f, db = 0.f, dc = 0.f, dd = 0.f;
#pragma unroll
                for (int k = 0; k < D / 4; ++k) {
                    const float4 cv = rows[cur][r][k];
                    const float a = q[k].x - cv.x, bq = q[k].y - cv.y, cq = q[k].z - cv.z,
                                dq = q[k].w - cv.w;
                    da = fmaf(a, a, da);
                    db = fmaf(bq, bq, db);
                    dc = fmaf(cq, cq, dc);
                    dd = fmaf(dq, dq, dd);
                }
                const float d2 = (da + db) + (dc + dd);
                if (j < t && d2 <= best) {
                    best = d2;
                    bj = j;
                }
            }
            if (c + 1 < nch)
                lstore(cur ^ 1);   // every wave left that buffer at the last barrier
            __syncthreads();
        }
    }
    bd[wv][lane] = best;
    bjs[wv][lane] = bj;
    __syncthreads();
    if (wv == 0 && p_out && !act && t < pf.N)
        p_out[row3(pf, s.Hq, b, t, h)] = -1;   // rows of no token
    if (wv != 0 || !act)
        return;
#pragma unroll
    for (int w = 1; w < PFM_WAVES; ++w) {
        const float d2 = bd[w][lane];
        const int j2 = bjs[w][lane];
        if (j2 >= 0 && (d2 < best || (d2 == best && j2 > bj))) {
            best = d2;
            bj = j2;
        }
    }
    float qn2 = 0.f;
#pragma unroll
    for (int k = 0; k < D / 4; ++k) {
        qn2 = fmaf(q[k].x, q[k].x, qn2);
        qn2 = fmaf(q[k].y, q[k].y, qn2);
        qn2 = fmaf(q[k].z, q[k].z, qn2);
        qn2 = fmaf(q[k].w, q[k].w, qn2);
    }
    int p = -1;
    if (s.reuse) {
        if (bj >= 0 && s.tau >= 0.f && best <= s.tau * s.tau * qn2)
            p = bj;
        const int ov = ovr ? ovr[row3(pf, s.Hq, b, t, h)] : -2;
        if (ov != -2) {
            p = -1;
            if (ov >= 0 && ov < t)
                p = ov;
            else if (ov >= 0)
                atomicAdd(&st.stats[ST_PF_OVR_INVALID], 1ULL);
        }
    }
    const long r = row3(pf, s.Hq, b, t, h);
    pf.p[r] = p;
    pf.lo[r] = p >= 0 ? max(p - st.band[h] + 1, 0) : 0;
    if (p_out)
        p_out[r] = p;
}

// ================================================================== attend
// Head g of the group attends [hs[g], he[g]] of this page (rows past the
// token itself read as zero values, as in compute_page).
template <typename T, int G>
__device__ __forceinline__ void compute_range(const PageRegs<T> &r, int tok0, int t,
                                              const int (&hs)[G], const int (&he)[G],
                                              const float (&q)[G][Kv<T>::E],
                                              WaveAcc<G, Kv<T>::E> &acc)
{
    using K = Kv<T>;
    constexpr int E = K::E;
    const int row = lane_id() / K::LPR;
    float lg[K::LPP][G];
#pragma unroll
    for (int s = 0; s < K::LPP; ++s) {
        float kf[E];
        to_f32(r.k[s], kf);
        const int tk = tok0 + s * K::RPL + row;
#pragma unroll
        for (int g = 0; g < G; ++g) {
            float a = 0.f;
#pragma unroll
            for (int e = 0; e < E; ++e)
                a = fmaf(q[g][e], kf[e], a);
            a = row_sum<T>(a);
            lg[s][g] = (tk < hs[g] || tk > he[g]) ? NEG_INF : a;
        }
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
        float mx = lg[0][g];
#pragma unroll
        for (int s = 1; s < K::LPP; ++s)
            mx = fmaxf(mx, lg[s][g]);
        const float mn = fmaxf(acc.M[g], mx);
        const float base = mn == NEG_INF ? 0.f : mn;
        const float alpha = exp2f(acc.M[g] - base);
        acc.M[g] = mn;
        acc.L[g] *= alpha;
#pragma unroll
        for (int e = 0; e < E; ++e)
            acc.acc[g][e] *= alpha;
#pragma unroll
        for (int s = 0; s < K::LPP; ++s)
            lg[s][g] = exp2f(lg[s][g] - base);
    }
#pragma unroll
    for (int s = 0; s < K::LPP; ++s) {
        float vf[E];
        to_f32(r.v[s], vf);
        if (tok0 + s * K::RPL + row > t) {
#pragma unroll
            for (int e = 0; e < E; ++e)
                vf[e] = 0.f;
        }
#pragma unroll
        for (int g = 0; g < G; ++g) {
            acc.L[g] += lg[s][g];
#pragma unroll
            for (int e = 0; e < E; ++e)
                acc.acc[g][e] = fmaf(lg[s][g], vf[e], acc.acc[g][e]);
        }
    }
}

// Grid (N, Hkv, B), one wave per (request, KV head, token).  Piece 0 of head
// g is [lo_g, t - r_g], piece 1 is [max(lo_g, t - r_g + 1), t]; each piece is
// stored unnormalised (acc, M, L) at part[b][t][piece][head].
template <typename T, int G>
__global__ __launch_bounds__(64) void prefill_attend_kernel(Shape s, State st, KvView kv, Pf pf,
                                                            const int32_t *__restrict__ seq_lens)
{
    using K = Kv<T>;
    const int t = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
    bool bad;
    if (t >= prompt_len(kv, seq_lens[b], pf.N, bad))
        return;
    int lo[G], cut[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        const int h = kvh * G + g;
        lo[g] = pf.lo[row3(pf, s.Hq, b, t, h)];
        cut[g] = t - st.band[h] + 1;
    }
    float q[G][K::E];
    {
        const int col = lane_id() % K::LPR;
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const float *src = pf.qrot + row3(pf, s.Hq, b, t, kvh * G + g) * D + col * K::E;
#pragma unroll
            for (int e = 0; e < K::E; e += 4) {
                const float4 x = *reinterpret_cast<const float4 *>(src + e);
                q[g][e + 0] = x.x * s.scale_log2;
                q[g][e + 1] = x.y * s.scale_log2;
                q[g][e + 2] = x.z * s.scale_log2;
                q[g][e + 3] = x.w * s.scale_log2;
            }
        }
    }
    unsigned long long *badc = &st.stats[ST_BAD_INPUT];
#pragma unroll
    for (int piece = 0; piece < 2; ++piece) {
        int hs[G], he[G];
        int a = INT_MAX, z = -1;
#pragma unroll
        for (int g = 0; g < G; ++g) {
            hs[g] = piece == 0 ? lo[g] : max(lo[g], cut[g]);
            he[g] = piece == 0 ? cut[g] - 1 : t;
            if (hs[g] <= he[g]) {
                a = min(a, hs[g]);
                z = max(z, he[g]);
            }
        }
        WaveAcc<G, K::E> acc;
        acc.init();
        if (a <= z) {
            PageRegs<T> r;
            for (int page = a / PAGE; page <= z / PAGE; ++page) {
                load_page<T>(r, kv_page<T>(kv, kv.k, b, kvh, s.Hkv, page, badc),
                             kv_page<T>(kv, kv.v, b, kvh, s.Hkv, page, badc));
                compute_range<T, G>(r, page * PAGE, t, hs, he, q, acc);
            }
        }
        store_wave_summary<T, G>(
            acc, pf.part + ((((long)b * pf.N + t) * 2 + piece) * s.Hq + kvh * G) * SUMM);
    }
}

// =================================================================== count
// Grid (Hkv, B), 256 threads (4 waves): the group's prompt tokens, decisions,
// hits and keys attended (t - min_g lo_g + 1 per token), then one atomic each.
__global__ __launch_bounds__(256) void prefill_count_kernel(Shape s, State st, KvView kv, Pf pf,
                                                            const int32_t *__restrict__ seq_lens)
{
    __shared__ unsigned long long red[2][4];   // hits, keys per wave
    const int kvh = blockIdx.x, b = blockIdx.y;
    bool bad;
    const int n = prompt_len(kv, seq_lens[b], pf.N, bad);
    unsigned long long hits = 0, keys = 0;
    for (int t = threadIdx.x; t < n; t += blockDim.x) {
        int lo = t;
        for (int g = 0; g < s.G; ++g) {
            const long r = row3(pf, s.Hq, b, t, kvh * s.G + g);
            hits += pf.p[r] >= 0;
            lo = min(lo, pf.lo[r]);
        }
        keys += (unsigned long long)(t - lo + 1);
    }
    for (int off = 32; off > 0; off >>= 1) {
        hits += __shfl_xor(hits, off, 64);
        keys += __shfl_xor(keys, off, 64);
    }
    const int wv = threadIdx.x >> 6;
    if (lane_id() == 0) {
        red[0][wv] = hits;
        red[1][wv] = keys;
    }
    __syncthreads();
    if (threadIdx.x == 0 && n > 0) {
        unsigned long long H = 0, Kt = 0;
        for (int w = 0; w < 4; ++w) {
            H += red[0][w];
            Kt += red[1][w];
        }
        if (kvh == 0)
            atomicAdd(&st.stats[ST_PF_TOKENS], (unsigned long long)n);
        atomicAdd(&st.stats[ST_PF_DECISIONS], (unsigned long long)n * s.G);
        atomicAdd(&st.stats[ST_PF_HITS], H);
        atomicAdd(&st.stats[ST_PF_KV], Kt);
    }
}

// ==================================================================== chain
// A normalised summary as one wave holds it: lane l has output columns 2l,
// 2l+1; M (log2 units) and L are wave-uniform.  EMPTY is L = 0.
struct Sum2 {
    float2 o;
    float M, L;
};

__device__ __forceinline__ Sum2 merge2(const Sum2 &x, const Sum2 &y)
{
    if (!(y.L > 0.f))
        return x;
    if (!(x.L > 0.f))
        return y;
    const float Mn = fmaxf(x.M, y.M);
    const float ca = x.L * exp2f(x.M - Mn), cb = y.L * exp2f(y.M - Mn);
    const float Ln = ca + cb;
    Sum2 r;
    r.o.x = (ca * x.o.x + cb * y.o.x) / Ln;
    r.o.y = (ca * x.o.y + cb * y.o.y) / Ln;
    r.M = Mn;
    r.L = Ln;
    return r;
}

__device__ __forceinline__ Sum2 load_unnorm(const float *p)
{
    Sum2 r;
    const float L = p[D + 1];
    const float2 a = *reinterpret_cast<const float2 *>(p + 2 * lane_id());
    r.L = L;
    r.M = p[D];
    r.o = L > 0.f ? make_float2(a.x / L, a.y / L) : make_float2(0.f, 0.f);
    return r;
}

__device__ __forceinline__ Sum2 load_norm(const float *p)
{
    Sum2 r;
    r.o = *reinterpret_cast<const float2 *>(p + 2 * lane_id());
    r.M = p[D];
    r.L = p[D + 1];
    return r;
}

__device__ __forceinline__ void store_norm(float *p, const Sum2 &x)
{
    *reinterpret_cast<float2 *>(p + 2 * lane_id()) = x.o;
    if (lane_id() == 0) {
        p[D] = x.M;
        p[D + 1] = x.L;
    }
}

// S = piece 0, parent = the matched position (-1: a miss or no token).
__global__ __launch_bounds__(64 * ROW_WAVES) void prefill_chain_init_kernel(
    Shape s, KvView kv, Pf pf, const int32_t *__restrict__ seq_lens)
{
    const RowId rid = row_id(s, pf);
    if (!rid.valid)
        return;
    const int h = rid.h, t = rid.t, b = rid.b;
    bool bad;
    const bool act = t < prompt_len(kv, seq_lens[b], pf.N, bad);
    const long r = row3(pf, s.Hq, b, t, h);
    Sum2 x;
    x.o = make_float2(0.f, 0.f);
    x.M = NEG_INF;
    x.L = 0.f;
    if (act)
        x = load_unnorm(pf.part + ((((long)b * pf.N + t) * 2 + 0) * s.Hq + h) * SUMM);
    store_norm(pf.sa + r * SUMM, x);
    if (lane_id() == 0)
        pf.pa[r] = act ? pf.p[r] : -1;
}

// One round of pointer jumping: S_t <- S_parent (+) S_t, parent <- parent of
// parent; reads (si, pi), writes (so, po).
__global__ __launch_bounds__(64 * ROW_WAVES) void prefill_chain_step_kernel(
    Shape s, Pf pf, const float *__restrict__ si, const int32_t *__restrict__ pi,
    float *__restrict__ so, int32_t *__restrict__ po)
{
    const RowId rid = row_id(s, pf);
    if (!rid.valid)
        return;
    const int h = rid.h, b = rid.b;
    const long r = rid.r;
    const int par = pi[r];
    Sum2 x = load_norm(si + r * SUMM);
    int np = -1;
    if (par >= 0) {
        const long rp = row3(pf, s.Hq, b, par, h);
        x = merge2(load_norm(si + rp * SUMM), x);
        np = pi[rp];
    }
    store_norm(so + r * SUMM, x);
    if (lane_id() == 0)
        po[r] = np;
}

// O_t = S_t (+) piece 1, normalised, into out; rows of no token get zeros.
__global__ __launch_bounds__(64 * ROW_WAVES) void prefill_out_kernel(
    Shape s, KvView kv, Pf pf, const int32_t *__restrict__ seq_lens,
    const float *__restrict__ sf, float *__restrict__ out)
{
    const RowId rid = row_id(s, pf);
    if (!rid.valid)
        return;
    const int h = rid.h, t = rid.t, b = rid.b, lane = lane_id();
    bool bad;
    const long r = row3(pf, s.Hq, b, t, h);
    float2 o = make_float2(0.f, 0.f);
    if (t < prompt_len(kv, seq_lens[b], pf.N, bad)) {
        const Sum2 x = merge2(
            load_norm(sf + r * SUMM),
            load_unnorm(pf.part + ((((long)b * pf.N + t) * 2 + 1) * s.Hq + h) * SUMM));
        o = x.o;
    }
    *reinterpret_cast<float2 *>(out + r * D + 2 * lane) = o;
}

}  // namespace

size_t prefill_scratch_bytes(const Shape &s, int N)
{
    const size_t rows = (size_t)s.B * N * s.Hq;
    auto r256 = [](size_t x) { return (x + 255) / 256 * 256; };
    return r256(rows * D * 4) + 4 * r256(rows * 4) + r256(rows * 2 * SUMM * 4) +
           2 * r256(rows * SUMM * 4);
}

hipError_t launch_prefill(const Shape &s, const State &st, const KvView &kv, bool kv_fp32,
                          const int32_t *seq_lens, int N, const float *q_pre, float *out,
                          const int32_t *override_pos, int32_t *p_out, void *scratch,
                          hipStream_t stream)
{
    if (!supported_group(s.G) || N < 1)
        return hipErrorInvalidValue;
    const size_t rows = (size_t)s.B * N * s.Hq;
    auto r256 = [](size_t x) { return (x + 255) / 256 * 256; };
    char *p = static_cast<char *>(scratch);
    auto take = [&](size_t bytes) {
        void *q = p;
        p += r256(bytes);
        return q;
    };
    Pf pf;
    pf.N = N;
    pf.qrot = static_cast<float *>(take(rows * D * 4));
    pf.p = static_cast<int32_t *>(take(rows * 4));
    pf.lo = static_cast<int32_t *>(take(rows * 4));
    pf.pa = static_cast<int32_t *>(take(rows * 4));
    pf.pb = static_cast<int32_t *>(take(rows * 4));
    pf.part = static_cast<float *>(take(rows * 2 * SUMM * 4));
    pf.sa = static_cast<float *>(take(rows * SUMM * 4));
    pf.sb = static_cast<float *>(take(rows * SUMM * 4));

    const dim3 per_row((unsigned)((rows + ROW_WAVES - 1) / ROW_WAVES));
    const dim3 row_block(64 * ROW_WAVES);
    hipLaunchKernelGGL(prefill_rope_kernel, per_row, row_block, 0, stream, s, st, kv, pf,
                       seq_lens, q_pre);
    if (s.ring_bf16)
        hipLaunchKernelGGL(prefill_match_kernel<true>, dim3((N + 63) / 64, s.Hq, s.B),
                           dim3(64 * PFM_WAVES), 0, stream, s, st, kv, pf, seq_lens, q_pre,
                           override_pos, p_out);
    else
        hipLaunchKernelGGL(prefill_match_kernel<false>, dim3((N + 63) / 64, s.Hq, s.B),
                           dim3(64 * PFM_WAVES), 0, stream, s, st, kv, pf, seq_lens, q_pre,
                           override_pos, p_out);
    const dim3 per_tok(N, s.Hkv, s.B);
#define MAC_PF_CASE(TT, GG)                                                                    \
    hipLaunchKernelGGL((prefill_attend_kernel<TT, GG>), per_tok, dim3(64), 0, stream, s, st, kv, \
                       pf, seq_lens)
    if (kv_fp32) {
        switch (s.G) {
        case 1: MAC_PF_CASE(float, 1); break;
        case 2: MAC_PF_CASE(float, 2); break;
        case 4: MAC_PF_CASE(float, 4); break;
        default: MAC_PF_CASE(float, 8); break;
        }
    } else {
        switch (s.G) {
        case 1: MAC_PF_CASE(uint16_t, 1); break;
        case 2: MAC_PF_CASE(uint16_t, 2); break;
        case 4: MAC_PF_CASE(uint16_t, 4); break;
        default: MAC_PF_CASE(uint16_t, 8); break;
        }
    }
#undef MAC_PF_CASE
    hipLaunchKernelGGL(prefill_count_kernel, dim3(s.Hkv, s.B), dim3(256), 0, stream, s, st, kv, pf,
                       seq_lens);
    hipLaunchKernelGGL(prefill_chain_init_kernel, per_row, row_block, 0, stream, s, kv, pf,
                       seq_lens);
    float *si = pf.sa, *so = pf.sb;
    int32_t *pi = pf.pa, *po = pf.pb;
    // ceil(log2 N) rounds; none with reuse off, where no token has a parent
    for (int span = 1; s.reuse && span < N; span *= 2) {
        hipLaunchKernelGGL(prefill_chain_step_kernel, per_row, row_block, 0, stream, s, pf, si,
                           pi, so, po);
        float *ts = si;
        si = so;
        so = ts;
        int32_t *tp = pi;
        pi = po;
        po = tp;
    }
    hipLaunchKernelGGL(prefill_out_kernel, per_row, row_block, 0, stream, s, kv, pf, seq_lens,
                       si, out);
    return hipGetLastError();
}

}  // namespace mac
