// mac_runtime.cpp -- host side of the C ABI declared in include/mac.h.
//
// Owns a layer's device state, the amend stream and the events that order
// match(t) after amend(t-1), or after amend(t-2) with the stale-by-one ring
// (the pages' "async cache update", MAC-Attention Figure 2 (c)).  No host
// synchronisation happens inside a decode step or a prefill: the hit/miss
// decisions, the work plan and the merge all stay on the device.
#include <hip/hip_runtime.h>

#include <cmath>
#include <condition_variable>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <thread>
#include <vector>

#include "mac.h"
#include "mac_internal.h"

struct mac_ctx {
    mac_config cfg{};
    mac::Shape shape{};
    mac::State st{};
    mac::State st_odd{};     // odd calls with the stale-by-one ring: own step buffers
    int device = 0;
    int n_blocks = 0;
    bool kv_fp32 = false;
    hipStream_t main_stream = nullptr;
    hipStream_t amend_stream = nullptr;
    bool own_amend = false;
    hipEvent_t ev_attn = nullptr, ev_drain = nullptr;
    hipEvent_t ev_amend[2] = {};     // after the amend of calls of even / odd index
    bool amend_pending[2] = {};
    // an amend run on the decode stream records no event: a later call on the
    // same stream is ordered after it anyway, one on another stream records
    // the event on this stream first (amend_on: that stream, or null)
    hipStream_t amend_on[2] = {};
    hipEvent_t tm[6] = {};
    // The default form on an amend stream the handle owns: a worker thread
    // of the handle waits on the host until the call's reduce has run
    // (ev_attn), then launches the amend and records its end event, so the
    // call returns once its reduce is enqueued and no cross-stream wait is
    // enqueued at all (one costs 11-16 us of host time, and the HIP runtime
    // serialises it against the caller's launches).  Every later call on the
    // handle first waits until the worker has enqueued the posted amend
    // (wk_posted false), and takes over any error it met.  When a decode call
    // finds the worker still busy, the GPU is behind the host (calls of this
    // handle back to back, nothing else between them): the next WK_BACKOFF
    // calls run their amend on the decode stream, where it needs no hand-off
    // between queues, and the period is renewed for as long as the previous
    // call has not finished when it ends.  Measured, 8 layers back to back, us
    // per layer and step: 62 -> 37-39 at 32K x 1, 56 -> 30-35 at 4096 x 1;
    // one layer in a tight loop: 59-61 -> 43 at 32K x 1, 62-64 -> 48-49 at
    // 128K x 16 (every head hitting), 54-56 -> 37 at 4096 x 1.
    struct Job {
        mac::State S;
        mac::KvView v;
        int cur;
        bool timing;
    };
    bool wk_on = false;
    std::thread wk;
    std::mutex wk_mu;
    std::condition_variable wk_cv;
    bool wk_posted = false, wk_stop = false;
    Job wk_job{};
    hipError_t wk_err = hipSuccess;
    const char *wk_what = "";
    int wk_backoff = 0;   // decode calls left to hand off on their own
    // Calls on different streams: the stream of the last call that enqueued
    // work on the handle's state, and ev_done, recorded on it after that work
    // (not recorded while the stream was being captured into a graph: then
    // done_valid is false and the caller orders the streams).
    hipStream_t last_stream = nullptr;
    hipEvent_t ev_done = nullptr;
    hipEvent_t done_ev = nullptr;   // ev_done, or an event the call already recorded at its end
    bool done_valid = false;
    // A HIP call failed part-way through a decode or prefill call: device and
    // host state may disagree (the ring slot counter), so such calls return
    // MAC_ESTATE until mac_reset succeeds.
    bool broken = false;
    bool timed_step = false;
    long long calls = 0;   // host-side call count: parity and hidden slot of the stale-by-one ring
    size_t aux_bytes = 0;
    void *blocks[16] = {};
    int n_alloc = 0;
    std::string err;
};

namespace {

thread_local std::string g_err;

mac_status fail(mac_handle h, mac_status s, const std::string &msg)
{
    if (h)
        h->err = msg;
    else
        g_err = msg;
    return s;
}

mac_status fail_hip(mac_handle h, const char *what, hipError_t e)
{
    return fail(h, MAC_EHIP, std::string(what) + ": " + hipGetErrorString(e));
}

#define MAC_HIP(h, call)                                                                    \
    do {                                                                                    \
        hipError_t e_ = (call);                                                             \
        if (e_ != hipSuccess)                                                               \
            return fail_hip((h), #call, e_);                                                \
    } while (0)

// Wait for the handle's amend hand-off worker; an error it met breaks the handle.
#define MAC_JOIN(h)                                                                         \
    do {                                                                                    \
        const char *w_ = "";                                                                \
        hipError_t e_ = join_worker((h), &w_);                                              \
        if (e_ != hipSuccess) {                                                             \
            (h)->broken = true;                                                             \
            return fail_hip((h), w_, e_);                                                   \
        }                                                                                   \
    } while (0)

struct Sizes {
    size_t ring_q, ring_s, ring_pos, qvec, m_buf, dec_i, dec_f, grp_parts, partials, as_full,
        stats, inv_freq, band, tiles;
    size_t step_copies;   // copies of the buffers amend reads: 2 with the stale-by-one ring
                          // (m_buf's size also holds the step's ring slot, one int)
    size_t total() const
    {
        return ring_q + ring_s + ring_pos + step_copies * (2 * qvec + 2 * m_buf + as_full) +
               3 * dec_i + dec_f + grp_parts + partials + stats + inv_freq + band + tiles;
    }
};

size_t round256(size_t x) { return (x + 255) / 256 * 256; }

// Work-list segments per group (two when amend is fused into the step).
int segments_per_group(const mac_config &c)
{
    const bool reuse = !(c.flags & MAC_F_DISABLE_REUSE) && c.tau >= 0.f;
    return (reuse && (c.flags & MAC_F_FUSED_AMEND)) ? 2 : 1;
}

Sizes sizes_for(const mac_config &c, int n_workers)
{
    const size_t B = c.batch, Hq = c.num_q_heads, Hkv = c.num_kv_heads, W = c.ring_size;
    const size_t G = Hq / Hkv, nseg = segments_per_group(c);
    Sizes s;
    s.ring_q = round256(B * Hq * W * mac::D * ((c.flags & MAC_F_RING_BF16) ? 2 : 4));
    s.ring_s = round256(B * Hq * W * mac::SUMM * sizeof(float));
    s.ring_pos = round256(B * W * sizeof(int32_t));
    s.qvec = round256(B * Hq * mac::D * sizeof(float));
    s.m_buf = round256(B * sizeof(int32_t));
    s.dec_i = round256(B * Hq * sizeof(int32_t));
    s.dec_f = round256(B * Hq * sizeof(float));
    s.grp_parts = round256(B * Hkv * nseg * 2 * sizeof(int32_t));
    s.partials = round256(((size_t)n_workers + B * Hkv * nseg) * G * mac::SUMM * sizeof(float));
    s.as_full = round256(B * Hq * mac::SUMM * sizeof(float));
    s.stats = round256(mac::stats_count((long)(B * Hq), (long)(B * Hkv)) *
                       sizeof(unsigned long long));
    s.inv_freq = round256(mac::D / 2 * sizeof(double));
    s.band = round256(Hq * sizeof(int32_t));
    const size_t ntiles = (W + mac::TILE_W - 1) / mac::TILE_W;
    s.tiles = W > (size_t)mac::TILE_W ? round256(B * Hq * ntiles * 3 * sizeof(float)) : 0;
    s.step_copies = (c.flags & MAC_F_STALE_RING) ? 2 : 1;
    return s;
}

mac_status validate(const mac_config *c, std::string &why)
{
    if (!c) {
        why = "cfg is NULL";
        return MAC_EINVAL;
    }
    if (c->batch < 1 || c->num_q_heads < 1 || c->num_kv_heads < 1) {
        why = "batch, num_q_heads and num_kv_heads must be >= 1";
        return MAC_EINVAL;
    }
    if (c->num_q_heads % c->num_kv_heads != 0) {
        why = "num_q_heads must be a multiple of num_kv_heads";
        return MAC_EINVAL;
    }
    if (c->head_dim != mac::D) {
        why = "head_dim must be 128";
        return c->head_dim > 0 ? MAC_EUNSUPPORTED : MAC_EINVAL;
    }
    if (!mac::supported_group(c->num_q_heads / c->num_kv_heads)) {
        why = "query heads per KV head must be 1, 2, 4 or 8";
        return MAC_EUNSUPPORTED;
    }
    if (c->ring_size < 1 || c->ring_size > mac::MAX_W) {
        why = "ring_size must be in [1, 2048]";
        return MAC_EINVAL;
    }
    if (!c->band_per_head && c->band < 1) {
        why = "band must be >= 1";
        return MAC_EINVAL;
    }
    if (!std::isfinite(c->tau)) {
        why = "tau must be finite";
        return MAC_EINVAL;
    }
    if (!(c->rope_theta > 0.f) || !std::isfinite(c->rope_theta)) {
        why = "rope_theta must be a positive finite number";
        return MAC_EINVAL;
    }
    if (!(c->sm_scale >= 0.f) || !std::isfinite(c->sm_scale)) {
        why = "sm_scale must be finite and >= 0";
        return MAC_EINVAL;
    }
    if (c->layout != MAC_KV_CONTIGUOUS && c->layout != MAC_KV_PAGED) {
        why = "unknown layout";
        return MAC_EINVAL;
    }
    if (c->kv_dtype != MAC_BF16 && c->kv_dtype != MAC_FP32) {
        why = "unknown kv_dtype";
        return MAC_EINVAL;
    }
    if (c->page_size != mac::PAGE) {
        why = "page_size must be 16";
        return c->page_size > 0 ? MAC_EUNSUPPORTED : MAC_EINVAL;
    }
    if (c->max_seq_len < mac::PAGE || c->max_seq_len % mac::PAGE != 0) {
        why = "max_seq_len must be a positive multiple of page_size";
        return MAC_EINVAL;
    }
    if ((long long)c->batch * c->num_kv_heads > mac::MAX_GROUPS) {
        why = "batch * num_kv_heads must be <= 4096";
        return MAC_EUNSUPPORTED;
    }
    const uint32_t known = MAC_F_DISABLE_REUSE | MAC_F_SYNC_AMEND | MAC_F_TIMING |
                           MAC_F_RECORD_DEBUG | MAC_F_FUSED_AMEND | MAC_F_RING_BF16 |
                           MAC_F_STALE_RING | MAC_F_UNBALANCED_PLAN;
    if (c->flags & ~known) {
        why = "unknown flag bits";
        return MAC_EINVAL;
    }
    if ((c->flags & MAC_F_STALE_RING) && (c->flags & MAC_F_FUSED_AMEND)) {
        why = "MAC_F_STALE_RING needs the separate amend; it excludes MAC_F_FUSED_AMEND";
        return MAC_EINVAL;
    }
    if (c->band_per_head) {
        const int G = c->num_q_heads / c->num_kv_heads;
        for (int h = 0; h < c->num_q_heads; ++h) {
            if (c->band_per_head[h] < 1) {
                why = "every entry of band_per_head must be >= 1";
                return MAC_EINVAL;
            }
            if ((c->flags & MAC_F_FUSED_AMEND) && c->band_per_head[h] != c->band_per_head[h / G * G]) {
                why = "MAC_F_FUSED_AMEND needs one band per KV group";
                return MAC_EUNSUPPORTED;
            }
        }
    }
    return MAC_OK;
}

// Kernels move key/value rows, queries and outputs as 16-byte vectors.
bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

mac_status check_view(mac_handle h, const mac_kv_view *kv)
{
    if (!kv)
        return fail(h, MAC_EINVAL, "kv view is NULL");
    if (!kv->k || !kv->v)
        return fail(h, MAC_EINVAL, "kv view has a NULL key or value pointer");
    if (!aligned16(kv->k) || !aligned16(kv->v))
        return fail(h, MAC_EINVAL, "kv view key and value pointers must be 16-byte aligned");
    if (!kv->seq_lens)
        return fail(h, MAC_EINVAL, "kv view has NULL seq_lens");
    if (h->cfg.layout == MAC_KV_PAGED &&
        (!kv->page_table || kv->max_pages_per_req < 1 || kv->num_pages < 1))
        return fail(h, MAC_EINVAL, "paged kv view needs page_table, max_pages_per_req and num_pages");
    return MAC_OK;
}

// Order `st` after the amend of calls of parity i (when one is pending).
hipError_t wait_amend(mac_ctx *h, int i, hipStream_t st)
{
    if (!h->amend_pending[i])
        return hipSuccess;
    if (h->amend_on[i]) {   // ran on a decode stream, no event recorded yet
        if (h->amend_on[i] == st)
            return hipSuccess;
        const hipError_t e = hipEventRecord(h->ev_amend[i], h->amend_on[i]);
        if (e != hipSuccess)
            return e;
        h->amend_on[i] = nullptr;
    }
    // an amend already finished needs no wait (a stream wait costs ~10 us of
    // host time; the query ~1 us)
    const hipError_t q = hipEventQuery(h->ev_amend[i]);
    if (q == hipSuccess) {
        h->amend_pending[i] = false;
        return hipSuccess;
    }
    if (q != hipErrorNotReady)
        return q;
    return hipStreamWaitEvent(st, h->ev_amend[i], 0);
}

// Order a call on stream st after the handle's last call when that one ran
// on another stream (its kernels read and write the same state).
hipError_t follow(mac_ctx *h, hipStream_t st)
{
    if (h->last_stream && h->last_stream != st && h->done_valid)
        return hipStreamWaitEvent(st, h->done_ev, 0);
    return hipSuccess;
}

// Mark the end of a call's work on st (skipped while st is being captured).
// `recorded`: an event the call has just recorded on st after its last work
// (the hand-off to the amend stream), which then serves as the end mark.
// `known`: st's capture status when the caller has already queried it.
hipError_t mark_done(mac_ctx *h, hipStream_t st, hipEvent_t recorded = nullptr,
                     const hipStreamCaptureStatus *known = nullptr)
{
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (known) {
        cs = *known;
    } else {
        const hipError_t e = hipStreamIsCapturing(st, &cs);
        if (e != hipSuccess)
            return e;
    }
    h->last_stream = st;
    h->done_valid = cs == hipStreamCaptureStatusNone;
    if (!h->done_valid)
        return hipSuccess;
    if (recorded) {
        h->done_ev = recorded;
        return hipSuccess;
    }
    h->done_ev = h->ev_done;
    return hipEventRecord(h->ev_done, st);
}

// The amend of the call whose reduce ev_attn follows (recorded on the decode
// stream), on the amend stream, then ev_amend[cur] after it.  host_wait: wait
// on the host until ev_attn has been reached instead of enqueueing a
// cross-stream wait (the worker thread's way).
hipError_t enqueue_amend(mac_ctx *h, const mac::State &S, const mac::KvView &v, int cur,
                         bool timing, bool host_wait, const char **what)
{
#define MAC_TRY(call)                                                                       \
    do {                                                                                    \
        hipError_t e_ = (call);                                                             \
        if (e_ != hipSuccess) {                                                             \
            *what = #call;                                                                  \
            return e_;                                                                      \
        }                                                                                   \
    } while (0)
    hipStream_t as = h->amend_stream;
    if (host_wait)
        MAC_TRY(hipEventSynchronize(h->ev_attn));
    else
        MAC_TRY(hipStreamWaitEvent(as, h->ev_attn, 0));
    if (timing)
        MAC_TRY(hipEventRecord(h->tm[4], as));
    MAC_TRY(mac::launch_amend(h->shape, S, v, h->kv_fp32, as));
    if (timing)
        MAC_TRY(hipEventRecord(h->tm[5], as));
    MAC_TRY(hipEventRecord(h->ev_amend[cur], as));
    return hipSuccess;
#undef MAC_TRY
}

void worker_main(mac_ctx *h)
{
    (void)hipSetDevice(h->device);
    // a graph capture that another thread of the process runs in global mode
    // must not turn this thread's host wait into an error: its calls touch
    // only streams and events of the handle, none of them captured
    hipStreamCaptureMode mode = hipStreamCaptureModeRelaxed;
    (void)hipThreadExchangeStreamCaptureMode(&mode);
    std::unique_lock<std::mutex> lk(h->wk_mu);
    for (;;) {
        h->wk_cv.wait(lk, [h] { return h->wk_posted || h->wk_stop; });
        if (!h->wk_posted)
            return;
        const mac_ctx::Job j = h->wk_job;
        lk.unlock();
        const char *what = "";
        const hipError_t e = enqueue_amend(h, j.S, j.v, j.cur, j.timing, true, &what);
        lk.lock();
        if (e != hipSuccess && h->wk_err == hipSuccess) {
            h->wk_err = e;
            h->wk_what = what;
        }
        h->wk_posted = false;
        h->wk_cv.notify_all();
    }
}

void post_amend(mac_ctx *h, const mac::State &S, const mac::KvView &v, int cur, bool timing)
{
    {
        std::lock_guard<std::mutex> lk(h->wk_mu);
        h->wk_job = mac_ctx::Job{S, v, cur, timing};
        h->wk_posted = true;
    }
    h->wk_cv.notify_all();
}

constexpr int WK_BACKOFF = 16;

// Wait until the worker has enqueued the hand-off posted last; returns (and
// clears) the first error it met since the last call.  *waited: it was still
// busy.
hipError_t join_worker(mac_ctx *h, const char **what, bool *waited = nullptr)
{
    if (!h->wk_on)
        return hipSuccess;
    std::unique_lock<std::mutex> lk(h->wk_mu);
    if (waited)
        *waited = h->wk_posted;
    h->wk_cv.wait(lk, [h] { return !h->wk_posted; });
    const hipError_t e = h->wk_err;
    if (e != hipSuccess) {
        *what = h->wk_what;
        h->wk_err = hipSuccess;
    }
    return e;
}

mac::KvView to_view(const mac_ctx *h, const mac_kv_view *kv)
{
    mac::KvView v{};
    v.k = kv->k;
    v.v = kv->v;
    v.paged = h->cfg.layout == MAC_KV_PAGED;
    v.page_table = v.paged ? kv->page_table : nullptr;
    v.max_pages = v.paged ? kv->max_pages_per_req : 0;
    v.num_pages = v.paged ? kv->num_pages : 0;
    v.max_seq_len = h->cfg.max_seq_len;
    return v;
}

void stop_worker(mac_ctx *h)
{
    if (!h->wk.joinable())
        return;
    {
        std::lock_guard<std::mutex> lk(h->wk_mu);
        h->wk_stop = true;
    }
    h->wk_cv.notify_all();
    h->wk.join();
}

void release(mac_ctx *h)
{
    stop_worker(h);   // it finishes a posted hand-off first
    // the last call may have run on a stream of the caller's: its end mark
    // follows all its work there (an amend on that stream included)
    if (h->done_valid && h->done_ev)
        (void)hipEventSynchronize(h->done_ev);
    if (h->main_stream || h->amend_stream) {
        if (h->amend_stream)
            (void)hipStreamSynchronize(h->amend_stream);
        (void)hipStreamSynchronize(h->main_stream);
    }
    for (int i = 0; i < h->n_alloc; ++i)
        (void)hipFree(h->blocks[i]);
    h->n_alloc = 0;
    if (h->ev_attn) (void)hipEventDestroy(h->ev_attn);
    for (auto &e : h->ev_amend)
        if (e) (void)hipEventDestroy(e);
    if (h->ev_drain) (void)hipEventDestroy(h->ev_drain);
    if (h->ev_done) (void)hipEventDestroy(h->ev_done);
    for (auto &e : h->tm)
        if (e) (void)hipEventDestroy(e);
    if (h->own_amend && h->amend_stream)
        (void)hipStreamDestroy(h->amend_stream);
}

}  // namespace

extern "C" {

const char *mac_status_string(mac_status s)
{
    switch (s) {
    case MAC_OK: return "MAC_OK";
    case MAC_EINVAL: return "MAC_EINVAL";
    case MAC_ENOMEM: return "MAC_ENOMEM";
    case MAC_EHIP: return "MAC_EHIP";
    case MAC_ESTATE: return "MAC_ESTATE";
    case MAC_EUNSUPPORTED: return "MAC_EUNSUPPORTED";
    }
    return "unknown mac_status";
}

const char *mac_last_error(mac_handle h) { return h ? h->err.c_str() : g_err.c_str(); }

mac_status mac_config_validate(const mac_config *cfg)
{
    std::string why;
    mac_status s = validate(cfg, why);
    if (s != MAC_OK)
        return fail(nullptr, s, why);
    return MAC_OK;
}

size_t mac_aux_bytes(const mac_config *cfg, int32_t num_cu)
{
    std::string why;
    if (validate(cfg, why) != MAC_OK || num_cu < 1)
        return 0;
    // the complete grid is num_cu * (resident blocks per CU) blocks of 4 waves;
    // count a generous 8 resident blocks per CU here
    return sizes_for(*cfg, num_cu * 8 * mac::WAVES).total();
}

mac_status mac_init(const mac_config *cfg, void *main_stream, void *amend_stream, mac_handle *out)
{
    std::string why;
    if (!out)
        return fail(nullptr, MAC_EINVAL, "out is NULL");
    *out = nullptr;
    mac_status vs = validate(cfg, why);
    if (vs != MAC_OK)
        return fail(nullptr, vs, why);

    mac_ctx *h = new (std::nothrow) mac_ctx();
    if (!h)
        return fail(nullptr, MAC_ENOMEM, "host allocation failed");
    h->cfg = *cfg;
    h->kv_fp32 = cfg->kv_dtype == MAC_FP32;
    h->main_stream = (hipStream_t)main_stream;

    auto bail = [&](mac_status s, const std::string &msg) {
        release(h);
        delete h;
        return fail(nullptr, s, msg);
    };
    hipError_t e = hipGetDevice(&h->device);
    if (e != hipSuccess)
        return bail(MAC_EHIP, std::string("hipGetDevice: ") + hipGetErrorString(e));
    e = mac::prefill_static_scratch_init(h->device);
    if (e != hipSuccess)
        return bail(MAC_EHIP, std::string("static prefill scratch: ") + hipGetErrorString(e));
    int n_cu = 0;
    e = hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, h->device);
    if (e != hipSuccess || n_cu < 1)
        return bail(MAC_EHIP, "cannot query the compute-unit count");

    const int G = cfg->num_q_heads / cfg->num_kv_heads;
    // The complete kernel's LDS plan: one offset per work-list segment, and
    // for short lists each segment's first key and each request's position
    // too (while that keeps the plan within 3 KB, so three blocks of the
    // kernel still fit a CU's 160 KB of LDS).
    const long n_plan = (long)cfg->batch * cfg->num_kv_heads * segments_per_group(*cfg);
    const bool plan_bounds = (2 * n_plan + 1 + cfg->batch) * (long)sizeof(int) <= 3072;
    const size_t plan_lds =
        (size_t)(plan_bounds ? 2 * n_plan + 1 + cfg->batch : n_plan + 1) * sizeof(int);
    h->st.slots = mac::complete_blocks_per_cu(h->kv_fp32, G, plan_lds);
    h->n_blocks = n_cu * h->st.slots;
    h->st.n_workers = h->n_blocks * mac::WAVES;
    const long n_seg = (long)cfg->batch * cfg->num_kv_heads * segments_per_group(*cfg);
    if ((cfg->flags & MAC_F_UNBALANCED_PLAN) && n_seg > h->st.n_workers)
        return bail(MAC_EUNSUPPORTED, "MAC_F_UNBALANCED_PLAN needs at least one wave of the "
                                      "complete grid per work-list segment");

    Sizes sz = sizes_for(*cfg, h->st.n_workers);
    h->aux_bytes = sz.total();
    auto grab = [&](size_t bytes) -> void * {
        void *p = nullptr;
        if (hipMalloc(&p, bytes) != hipSuccess)
            return nullptr;
        h->blocks[h->n_alloc++] = p;
        return p;
    };
    void *base = grab(sz.total());
    if (!base)
        return bail(MAC_ENOMEM, "device allocation of the handle state failed");
    char *p = (char *)base;
    auto take = [&](size_t bytes) {
        void *r = p;
        p += bytes;
        return r;
    };
    h->st.ring_q = take(sz.ring_q);
    h->st.ring_s = (float *)take(sz.ring_s);
    h->st.ring_pos = (int32_t *)take(sz.ring_pos);
    h->st.q_copy = (float *)take(sz.qvec);
    h->st.q_rot = (float *)take(sz.qvec);
    h->st.m_buf = (int32_t *)take(sz.m_buf);
    h->st.step_slot = (int32_t *)take(sz.m_buf);
    h->st.dec_slot = (int32_t *)take(sz.dec_i);
    h->st.dec_p = (int32_t *)take(sz.dec_i);
    h->st.dec_start = (int32_t *)take(sz.dec_i);
    h->st.dec_rel = (float *)take(sz.dec_f);
    h->st.grp_parts = (int32_t *)take(sz.grp_parts);
    h->st.partials = (float *)take(sz.partials);
    h->st.as_full = (float *)take(sz.as_full);
    h->st.stats = (unsigned long long *)take(sz.stats);
    h->st.head_stats = h->st.stats + mac::MAC_NSTAT;
    h->st.grp_stats = h->st.head_stats + (long)cfg->batch * cfg->num_q_heads * mac::HEAD_NSTAT;
    h->st.inv_freq = (const double *)take(sz.inv_freq);
    h->st.band = (const int32_t *)take(sz.band);
    h->st.tile_best = sz.tiles ? (float *)take(sz.tiles) : nullptr;
    h->st_odd = h->st;
    if (sz.step_copies == 2) {
        h->st_odd.q_copy = (float *)take(sz.qvec);
        h->st_odd.q_rot = (float *)take(sz.qvec);
        h->st_odd.m_buf = (int32_t *)take(sz.m_buf);
        h->st_odd.step_slot = (int32_t *)take(sz.m_buf);
        h->st_odd.as_full = (float *)take(sz.as_full);
    }

    e = hipMemset(base, 0, sz.total());
    if (e != hipSuccess)
        return bail(MAC_EHIP, std::string("hipMemset: ") + hipGetErrorString(e));
    double inv[mac::D / 2];
    for (int i = 0; i < mac::D / 2; ++i)
        inv[i] = std::pow((double)cfg->rope_theta, -2.0 * i / (double)mac::D);
    e = hipMemcpy((void *)h->st.inv_freq, inv, sizeof inv, hipMemcpyHostToDevice);
    if (e != hipSuccess)
        return bail(MAC_EHIP, std::string("hipMemcpy: ") + hipGetErrorString(e));
    std::vector<int32_t> bands(cfg->num_q_heads, cfg->band);
    if (cfg->band_per_head)
        bands.assign(cfg->band_per_head, cfg->band_per_head + cfg->num_q_heads);
    h->cfg.band_per_head = nullptr;   // borrowed for this call only
    e = hipMemcpy((void *)h->st.band, bands.data(), bands.size() * sizeof(int32_t),
                  hipMemcpyHostToDevice);
    if (e != hipSuccess)
        return bail(MAC_EHIP, std::string("hipMemcpy: ") + hipGetErrorString(e));

    h->shape.B = cfg->batch;
    h->shape.Hq = cfg->num_q_heads;
    h->shape.Hkv = cfg->num_kv_heads;
    h->shape.G = G;
    h->shape.W = cfg->ring_size;
    h->shape.tau = cfg->tau;
    const double scale = cfg->sm_scale > 0.f ? (double)cfg->sm_scale : 1.0 / std::sqrt((double)mac::D);
    h->shape.scale_log2 = (float)(scale * 1.4426950408889634);
    h->shape.reuse = !(cfg->flags & MAC_F_DISABLE_REUSE) && cfg->tau >= 0.f;
    h->shape.nseg = segments_per_group(*cfg);
    h->shape.ring_bf16 = (cfg->flags & MAC_F_RING_BF16) ? 1 : 0;
    h->shape.unbalanced = (cfg->flags & MAC_F_UNBALANCED_PLAN) ? 1 : 0;
    h->shape.plan_bounds = plan_bounds ? 1 : 0;

    if (amend_stream) {
        h->amend_stream = (hipStream_t)amend_stream;
    } else {
        e = hipStreamCreateWithFlags(&h->amend_stream, hipStreamNonBlocking);
        if (e != hipSuccess)
            return bail(MAC_EHIP, std::string("hipStreamCreate: ") + hipGetErrorString(e));
        h->own_amend = true;
    }
    // These events only order streams of this device, and the host only asks
    // whether one has completed; HIP documents that an event without the
    // system-scope fence (a cache write-back and invalidate when it is
    // reached) leaves device memory possibly invisible to the host and to
    // other devices only.  Measured: 1.5 to 3 us less per call on short
    // steps, the same on long ones.
    constexpr unsigned ORDER_EVENT = hipEventDisableTiming | hipEventDisableSystemFence;
    // ev_attn is also what the amend worker waits for on the host: blocking,
    // so a handle's thread sleeps instead of spinning a core
    if (hipEventCreateWithFlags(&h->ev_attn, ORDER_EVENT | hipEventBlockingSync) != hipSuccess ||
        hipEventCreateWithFlags(&h->ev_amend[0], ORDER_EVENT) != hipSuccess ||
        hipEventCreateWithFlags(&h->ev_amend[1], ORDER_EVENT) != hipSuccess ||
        hipEventCreateWithFlags(&h->ev_drain, ORDER_EVENT) != hipSuccess ||
        hipEventCreateWithFlags(&h->ev_done, ORDER_EVENT) != hipSuccess)
        return bail(MAC_EHIP, "hipEventCreate failed");
    // the timing events (MAC_F_TIMING) skip the fence too: a write-back at
    // each would land inside the kernel times they bracket
    for (auto &ev : h->tm)
        if (hipEventCreateWithFlags(&ev, hipEventDisableSystemFence) != hipSuccess)
            return bail(MAC_EHIP, "hipEventCreate failed");

    e = mac::launch_reset(h->shape, h->st, h->main_stream);
    if (e == hipSuccess)
        e = hipStreamSynchronize(h->main_stream);
    if (e != hipSuccess)
        return bail(MAC_EHIP, std::string("ring reset: ") + hipGetErrorString(e));
    if (h->own_amend && h->shape.reuse && h->shape.nseg == 1 &&
        !(cfg->flags & MAC_F_SYNC_AMEND)) {
        try {
            h->wk = std::thread(worker_main, h);
        } catch (...) {
            return bail(MAC_EUNSUPPORTED, "cannot start the amend hand-off thread");
        }
        h->wk_on = true;
    }
    *out = h;
    return MAC_OK;
}

mac_status mac_destroy(mac_handle h)
{
    if (!h)
        return fail(nullptr, MAC_EINVAL, "handle is NULL");
    release(h);
    delete h;
    return MAC_OK;
}

mac_status mac_reset(mac_handle h)
{
    if (!h)
        return fail(nullptr, MAC_EINVAL, "handle is NULL");
    const char *what = "";
    (void)join_worker(h, &what);   // the state is rebuilt below whatever the worker met
    MAC_HIP(h, follow(h, h->main_stream));
    for (int i = 0; i < 2; ++i)
        MAC_HIP(h, wait_amend(h, i, h->main_stream));
    MAC_HIP(h, mac::launch_reset(h->shape, h->st, h->main_stream));
    MAC_HIP(h, mark_done(h, h->main_stream));
    h->calls = 0;
    h->timed_step = false;
    h->broken = false;
    return MAC_OK;
}

mac_status mac_append_kv(mac_handle h, const mac_kv_view *kv, const void *k_new, const void *v_new,
                         const int32_t *positions, void *stream)
{
    if (!h)
        return fail(nullptr, MAC_EINVAL, "handle is NULL");
    mac_status s = check_view(h, kv);
    if (s != MAC_OK)
        return s;
    if (!k_new || !v_new || !positions)
        return fail(h, MAC_EINVAL, "k_new, v_new and positions must be non-NULL");
    if (!aligned16(k_new) || !aligned16(v_new))
        return fail(h, MAC_EINVAL, "k_new and v_new must be 16-byte aligned");
    hipStream_t st = stream ? (hipStream_t)stream : h->main_stream;
    MAC_HIP(h, mac::launch_append(h->shape, h->st, to_view(h, kv), h->kv_fp32, k_new, v_new,
                                  positions, st));
    return MAC_OK;
}

namespace {

// Decode calls that enqueue the same work with the same arguments every call,
// so that a graph captured from one replays the step: no amend on another
// stream (its events are chosen per call on the host), no alternating
// buffers (stale-by-one ring), no per-kernel timing events.
bool capturable(const mac_ctx *h, hipStream_t st)
{
    const unsigned f = h->cfg.flags;
    if (f & (MAC_F_STALE_RING | MAC_F_TIMING))
        return false;
    const bool amend_elsewhere = h->shape.reuse && h->shape.nseg == 1 &&
                                 !(f & MAC_F_SYNC_AMEND) && h->amend_stream != st;
    return !amend_elsewhere;
}

// The enqueue sequence of one decode call on stream st; `what` names the HIP
// call that failed.
hipError_t decode_enqueue(mac_ctx *h, const mac_kv_view *kv, const float *q_pre_rope, float *out,
                          const int32_t *override_pos, hipStream_t st,
                          hipStreamCaptureStatus capture, const char **what)
{
#define MAC_TRY(call)                                                                       \
    do {                                                                                    \
        hipError_t e_ = (call);                                                             \
        if (e_ != hipSuccess) {                                                             \
            *what = #call;                                                                  \
            return e_;                                                                      \
        }                                                                                   \
    } while (0)
    const mac::KvView v = to_view(h, kv);
    const bool timing = h->cfg.flags & MAC_F_TIMING;
    const int cur = (int)(h->calls & 1);

    {
        bool waited = false;
        const hipError_t e = join_worker(h, what, &waited);   // *what names the worker's call
        if (e != hipSuccess)
            return e;
        if (waited)
            h->wk_backoff = WK_BACKOFF;
    }
    MAC_TRY(follow(h, st));
    // match(t) reads the ring amend(t-1) writes.  The stale-by-one ring hides
    // that slot from match(t), which then waits only for amend(t-2); the two
    // calls also work on separate copies of the buffers amend reads.
    const bool stale = h->cfg.flags & MAC_F_STALE_RING;
    const mac::State &S = (stale && cur) ? h->st_odd : h->st;
    MAC_TRY(wait_amend(h, stale ? cur : cur ^ 1, st));
    const int hidden = (stale && h->calls > 0) ? (int)((h->calls - 1) % h->cfg.ring_size) : -1;
    if (timing)
        MAC_TRY(hipEventRecord(h->tm[0], st));
    MAC_TRY(mac::launch_match(h->shape, S, v, kv->seq_lens, q_pre_rope, override_pos, out,
                              hidden, st));
    // The complete kernel is a persistent grid with equal static shares per
    // wave: a kernel still holding CU slots when it launches delays some of
    // its waves and with them the whole launch (measured: +35 % when an amend
    // of another layer overlapped its first microsecond).  So on an amend
    // stream the caller supplied (which other layers may share), complete
    // waits for every amend already queued there; amend still overlaps append
    // and match.  A stream the handle owns holds only this handle's amend,
    // which match already waited for (the extra cross-queue wait costs ~10 us).
    const bool fused = h->shape.nseg == 2;
    if (!h->own_amend && h->amend_stream != st && !(h->cfg.flags & MAC_F_SYNC_AMEND) &&
        h->shape.reuse && !fused) {
        MAC_TRY(hipEventRecord(h->ev_drain, h->amend_stream));
        MAC_TRY(hipStreamWaitEvent(st, h->ev_drain, 0));
    }
    if (timing)
        MAC_TRY(hipEventRecord(h->tm[1], st));
    MAC_TRY(mac::launch_complete(h->shape, S, v, h->kv_fp32, h->n_blocks, st));
    if (timing)
        MAC_TRY(hipEventRecord(h->tm[2], st));
    MAC_TRY(mac::launch_reduce(h->shape, S, out, st));
    if (timing)
        MAC_TRY(hipEventRecord(h->tm[3], st));

    hipEvent_t end_mark = nullptr;   // an event recorded on st after this call's last work
    const bool backing_off = h->wk_on && h->wk_backoff > 0;
    if (backing_off && --h->wk_backoff == 0 && h->done_valid && h->last_stream == st) {
        // the period ends only once the GPU has caught up with the previous
        // call: handing off to the thread while it is behind would stall the
        // next call until the GPU drains
        const hipError_t q = hipEventQuery(h->done_ev);
        if (q == hipErrorNotReady)
            h->wk_backoff = WK_BACKOFF;
        else if (q != hipSuccess) {
            *what = "hipEventQuery";
            return q;
        }
    }
    const bool via_worker = h->wk_on && h->amend_stream != st && !backing_off;
    if (h->shape.reuse && !fused && via_worker) {
        MAC_TRY(hipEventRecord(h->ev_attn, st));
        end_mark = h->ev_attn;
        post_amend(h, S, v, cur, timing);
        h->amend_on[cur] = nullptr;
        h->amend_pending[cur] = true;
    } else if (h->shape.reuse && !fused) {
        // backing off, the GPU is behind the host: amend on the decode stream
        // costs it no hand-off between queues, and the host no stream wait
        hipStream_t as = ((h->cfg.flags & MAC_F_SYNC_AMEND) || backing_off) ? st : h->amend_stream;
        if (as != st) {
            MAC_TRY(hipEventRecord(h->ev_attn, st));
            MAC_TRY(hipStreamWaitEvent(as, h->ev_attn, 0));
            end_mark = h->ev_attn;
        }
        if (timing)
            MAC_TRY(hipEventRecord(h->tm[4], as));
        MAC_TRY(mac::launch_amend(h->shape, S, v, h->kv_fp32, as));
        if (timing)
            MAC_TRY(hipEventRecord(h->tm[5], as));
        if (as != st) {
            MAC_TRY(hipEventRecord(h->ev_amend[cur], as));
            h->amend_on[cur] = nullptr;
        } else {
            h->amend_on[cur] = st;
        }
        h->amend_pending[cur] = true;
    }
    MAC_TRY(mark_done(h, st, end_mark, &capture));
    h->timed_step = timing;
    h->calls += 1;
    return hipSuccess;
#undef MAC_TRY
}

}  // namespace

mac_status mac_decode_step(mac_handle h, const mac_kv_view *kv, const float *q_pre_rope, float *out,
                           const int32_t *override_pos, void *stream)
{
    if (!h)
        return fail(nullptr, MAC_EINVAL, "handle is NULL");
    if (h->broken)
        return fail(h, MAC_ESTATE, "an earlier call failed part-way; call mac_reset first");
    mac_status s = check_view(h, kv);
    if (s != MAC_OK)
        return s;
    if (!q_pre_rope || !out)
        return fail(h, MAC_EINVAL, "q_pre_rope and out must be non-NULL");
    if (!aligned16(q_pre_rope) || !aligned16(out))
        return fail(h, MAC_EINVAL, "q_pre_rope and out must be 16-byte aligned");
    hipStream_t st = stream ? (hipStream_t)stream : h->main_stream;
    hipStreamCaptureStatus capture = hipStreamCaptureStatusNone;
    MAC_HIP(h, hipStreamIsCapturing(st, &capture));
    if (capture != hipStreamCaptureStatusNone && !capturable(h, st))
        return fail(h, MAC_EUNSUPPORTED,
                    "this form chooses its events or buffers per call on the host and cannot be "
                    "captured into a graph (capturable: fused amend or amend on the decode "
                    "stream, or reuse disabled; without the stale ring or per-kernel timing)");
    const char *what = "";
    const hipError_t e = decode_enqueue(h, kv, q_pre_rope, out, override_pos, st, capture, &what);
    if (e != hipSuccess) {
        h->broken = true;
        return fail_hip(h, what, e);
    }
    return MAC_OK;
}

mac_status mac_prefill(mac_handle h, const mac_kv_view *kv, int32_t num_tokens,
                       const float *q_pre, float *out, const int32_t *override_pos,
                       int32_t *p_out, void *stream)
{
    if (!h)
        return fail(nullptr, MAC_EINVAL, "handle is NULL");
    if (h->broken)
        return fail(h, MAC_ESTATE, "an earlier call failed part-way; call mac_reset first");
    MAC_JOIN(h);
    mac_status s = check_view(h, kv);
    if (s != MAC_OK)
        return s;
    if (num_tokens < 1 || num_tokens > 32768)
        return fail(h, MAC_EINVAL, "num_tokens must be in [1, 32768]");
    if (!q_pre || !out)
        return fail(h, MAC_EINVAL, "q_pre and out must be non-NULL");
    if (!aligned16(q_pre) || !aligned16(out))
        return fail(h, MAC_EINVAL, "q_pre and out must be 16-byte aligned");
    hipStream_t st = stream ? (hipStream_t)stream : h->main_stream;
    hipError_t e = follow(h, st);
    if (e != hipSuccess) {
        h->broken = true;
        return fail_hip(h, "follow", e);
    }
    const size_t bytes = mac::prefill_scratch_bytes(h->shape, num_tokens);
    void *scratch = nullptr;
    if (hipMallocAsync(&scratch, bytes, st) != hipSuccess || !scratch) {
        (void)hipGetLastError();
        return fail(h, MAC_ENOMEM, "stream-ordered allocation of the prefill scratch failed");
    }
    e = mac::launch_prefill(h->shape, h->st, to_view(h, kv), h->kv_fp32, kv->seq_lens, num_tokens,
                            q_pre, out, override_pos, p_out, scratch, st);
    const hipError_t ef = hipFreeAsync(scratch, st);
    const hipError_t ed = e == hipSuccess && ef == hipSuccess ? mark_done(h, st) : hipSuccess;
    if (e != hipSuccess || ef != hipSuccess || ed != hipSuccess) {
        h->broken = true;
        return e != hipSuccess ? fail_hip(h, "launch_prefill", e)
               : ef != hipSuccess ? fail_hip(h, "hipFreeAsync", ef) : fail_hip(h, "mark_done", ed);
    }
    return MAC_OK;
}

mac_status mac_prefill_noalloc(mac_handle h, const mac_kv_view *kv, int32_t num_tokens,
                               const float *q_pre, float *out, const int32_t *override_pos,
                               int32_t *p_out, void *stream)
{
    if (!h)
        return fail(nullptr, MAC_EINVAL, "handle is NULL");
    if (h->broken)
        return fail(h, MAC_ESTATE, "an earlier call failed part-way; call mac_reset first");
    MAC_JOIN(h);
    mac_status s = check_view(h, kv);
    if (s != MAC_OK)
        return s;
    if (num_tokens < 1 || num_tokens > 32768)
        return fail(h, MAC_EINVAL, "num_tokens must be in [1, 32768]");
    if (!q_pre || !out)
        return fail(h, MAC_EINVAL, "q_pre and out must be non-NULL");
    if (!aligned16(q_pre) || !aligned16(out))
        return fail(h, MAC_EINVAL, "q_pre and out must be 16-byte aligned");
    const size_t bytes = mac::prefill_scratch_bytes(h->shape, num_tokens);
    if (bytes > mac::PREFILL_STATIC_BYTES)
        return fail(h, MAC_EINVAL, "mac_prefill_noalloc: batch * num_tokens * num_q_heads needs " +
                                       std::to_string(bytes) + " bytes of scratch, over the " +
                                       std::to_string(mac::PREFILL_STATIC_BYTES) +
                                       "-byte static array (use mac_prefill)");
    void *scratch = mac::prefill_static_scratch(h->device);
    if (!scratch)
        return fail(h, MAC_ESTATE, "static prefill scratch not set up on this device");
    hipStream_t st = stream ? (hipStream_t)stream : h->main_stream;
    hipError_t e = follow(h, st);
    if (e == hipSuccess)
        e = mac::launch_prefill(h->shape, h->st, to_view(h, kv), h->kv_fp32, kv->seq_lens,
                                num_tokens, q_pre, out, override_pos, p_out, scratch, st);
    if (e == hipSuccess)
        e = mark_done(h, st);
    if (e != hipSuccess) {
        h->broken = true;
        return fail_hip(h, "mac_prefill_noalloc", e);
    }
    return MAC_OK;
}

mac_status mac_stats(mac_handle h, mac_stats_t *out)
{
    if (!h || !out)
        return fail(h, MAC_EINVAL, "handle and out must be non-NULL");
    MAC_JOIN(h);
    MAC_HIP(h, hipStreamSynchronize(h->main_stream));
    if (h->amend_stream)
        MAC_HIP(h, hipStreamSynchronize(h->amend_stream));
    MAC_HIP(h, hipDeviceSynchronize());
    const long n_heads = (long)h->cfg.batch * h->cfg.num_q_heads;
    const long n_groups = (long)h->cfg.batch * h->cfg.num_kv_heads;
    std::vector<unsigned long long> raw(mac::stats_count(n_heads, n_groups));
    MAC_HIP(h, hipMemcpy(raw.data(), h->st.stats, raw.size() * sizeof(unsigned long long),
                         hipMemcpyDeviceToHost));
    unsigned long long hs[mac::HEAD_NSTAT] = {}, gs[mac::GRP_NSTAT] = {};
    const unsigned long long *hp = raw.data() + mac::MAC_NSTAT;
    const unsigned long long *gp = hp + n_heads * mac::HEAD_NSTAT;
    for (long i = 0; i < n_heads; ++i)
        for (int k = 0; k < mac::HEAD_NSTAT; ++k)
            hs[k] += hp[i * mac::HEAD_NSTAT + k];
    for (long g = 0; g < n_groups; ++g)
        for (int k = 0; k < mac::GRP_NSTAT; ++k)
            gs[k] += gp[g * mac::GRP_NSTAT + k];
    std::memset(out, 0, sizeof *out);
    const uint64_t row = 2ull * mac::D * (h->kv_fp32 ? 4 : 2);   // one key row + one value row
    out->steps = raw[mac::ST_STEPS];   // counted on the device (graph replays included)
    out->hits = hs[mac::HS_HITS];
    out->misses = hs[mac::HS_MISSES];
    out->decisions = out->hits + out->misses;
    out->near_tau = hs[mac::HS_NEAR_TAU];
    out->override_invalid = hs[mac::HS_OVR_INVALID];
    out->kv_tokens_critical = gs[mac::GS_TOK_CRIT];
    out->kv_tokens_amend = gs[mac::GS_TOK_AMEND];
    out->kv_bytes_critical = gs[mac::GS_TOK_CRIT] * row;
    out->kv_bytes_amend = gs[mac::GS_TOK_AMEND] * row;
    out->aux_bytes = h->aux_bytes;
    out->complete_waves = (uint64_t)h->st.n_workers;
    out->bad_input = raw[mac::ST_BAD_INPUT];
    out->prefill_tokens = raw[mac::ST_PF_TOKENS];
    out->prefill_decisions = raw[mac::ST_PF_DECISIONS];
    out->prefill_hits = raw[mac::ST_PF_HITS];
    out->prefill_kv_tokens = raw[mac::ST_PF_KV];
    out->prefill_override_invalid = raw[mac::ST_PF_OVR_INVALID];
    if (h->timed_step) {
        float t = 0.f;
        if (hipEventElapsedTime(&t, h->tm[0], h->tm[1]) == hipSuccess) out->last_us_match = t * 1e3f;
        if (hipEventElapsedTime(&t, h->tm[1], h->tm[2]) == hipSuccess) out->last_us_complete = t * 1e3f;
        if (hipEventElapsedTime(&t, h->tm[2], h->tm[3]) == hipSuccess) out->last_us_reduce = t * 1e3f;
        if (hipEventElapsedTime(&t, h->tm[0], h->tm[3]) == hipSuccess) out->last_us_attention = t * 1e3f;
        if (h->shape.reuse && h->shape.nseg == 1 &&
            hipEventElapsedTime(&t, h->tm[4], h->tm[5]) == hipSuccess)
            out->last_us_amend = t * 1e3f;
    }
    return MAC_OK;
}

mac_status mac_debug_last(mac_handle h, int32_t *p, uint8_t *hit, float *rel)
{
    if (!h)
        return fail(nullptr, MAC_EINVAL, "handle is NULL");
    if (!(h->cfg.flags & MAC_F_RECORD_DEBUG))
        return fail(h, MAC_ESTATE, "mac_debug_last needs MAC_F_RECORD_DEBUG");
    MAC_JOIN(h);
    MAC_HIP(h, hipStreamSynchronize(h->main_stream));
    MAC_HIP(h, hipDeviceSynchronize());
    const size_t n = (size_t)h->cfg.batch * h->cfg.num_q_heads;
    if (p)
        MAC_HIP(h, hipMemcpy(p, h->st.dec_p, n * sizeof(int32_t), hipMemcpyDeviceToHost));
    if (hit) {
        int32_t *tmp = new (std::nothrow) int32_t[n];
        if (!tmp)
            return fail(h, MAC_ENOMEM, "host allocation failed");
        hipError_t e = hipMemcpy(tmp, h->st.dec_slot, n * sizeof(int32_t), hipMemcpyDeviceToHost);
        if (e != hipSuccess) {
            delete[] tmp;
            return fail_hip(h, "hipMemcpy", e);
        }
        for (size_t i = 0; i < n; ++i)
            hit[i] = tmp[i] >= 0;
        delete[] tmp;
    }
    if (rel)
        MAC_HIP(h, hipMemcpy(rel, h->st.dec_rel, n * sizeof(float), hipMemcpyDeviceToHost));
    return MAC_OK;
}

}  // extern "C"
