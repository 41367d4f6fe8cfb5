"""Benchmark of the MAC-Attention decode step on one MI355X.

Workload (default): batch 16 x 131072-token context, 32 query / 8 KV heads,
d = 128, paged bf16 KV (16-token pages, permuted table), ring 32, r = 256,
tau = 0.3, per-request AR(1) rho ~ U[0.8, 0.99] -- synthetic inputs of that
shape (no dataset, no model weights).

A step is one pass of the whole hot path over the batch: append this token's
K/V rows, match, complete, reduce/merge (the attention phase) and amend on its
own stream.  The timed region runs K steps after W warm-up steps; inputs are
resident in HBM before it starts.  The attention phase (match -> reduce, amend
excluded, as the pages split it in Table 5) is timed per step by two events on
the decode stream around the decode call, each step launched onto an idle GPU
(the counters are read between steps), so the span includes the call's launch
latency but no wait for an amend.  The same steps enqueued back to back give
`attention_us_pipelined`.  A further pass over the same steps, from a fresh
ring, records the library's HIP events around every kernel (MAC_F_TIMING) for
the per-kernel durations and the roofline of the complete kernel.

Prints one JSON line.  `value` is the attention-phase microseconds per decode
step (lower is better); the line also carries achieved HBM GB/s, tokens/s, the
roofline of the dominant kernel (complete), the in-house full-attention kernel
on the same cache (timed the same way) and the fp64 oracle timed on a bounded
sample.  `loop_us_per_step` gives back-to-back figures with amend included.  With the default workload the line also carries
`workloads`: compact records of the other shapes (the CPU-sized 4K workload
over all 256 steps, the 32q/4kv MoE shape at r = 64, 256 and 1024, continuous
generation over 32 layers), each MAC against full attention on its own cache.
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
CPU_WARM, CPU_STEPS = 8, 16      # oracle sample at the headline shape: warm-up, timed steps
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "complete_kernel_b16_128k_traffic.json")
# sources the complete kernel is built from: the counters are void once they change
KERNEL_SRCS = [os.path.join(ROOT, "kv_reuse_amd", "csrc", f)
               for f in ("complete.hip", "mfma_page.h", "mac_device.h", "mac_internal.h")]


def kernel_sha16():
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SRCS:
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def measured_traffic(workload):
    """HBM bytes per complete launch from the committed rocprofv3 counter
    summary, valid only while the kernel source is the one it was taken on."""
    if workload != "b16_128k" or not os.path.exists(TRAFFIC_FILE):
        return None
    rec = json.load(open(TRAFFIC_FILE))
    return rec["traffic_bytes_per_launch"] if rec.get("kernel_sha16") == kernel_sha16() else None


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=48)
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--config", default="b16_128k")
    ap.add_argument("--r", type=int, default=0, help="override the band width")
    ap.add_argument("--set", action="append", default=[], metavar="FIELD=VALUE",
                    help="override a workload field (B, Hq, Hkv, C, W, r, tau, ...)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-baseline-kernel", action="store_true")
    ap.add_argument("--no-32k", action="store_true", help="skip the 32K speedup point")
    ap.add_argument("--no-workloads", action="store_true",
                    help="skip the other workloads' sub-records (CPU-sized 4K, MoE 122K at "
                         "r = 64/256/1024, continuous generation)")
    ap.add_argument("--figures", nargs="?", const="fig4,fig5,fig8a,fig8b", default=None,
                    help="synthetic analogs of the pages' Figures 4, 5 and 8 (one JSON line); "
                         "optionally a comma list of fig4, fig5, fig8a, fig8b")
    ap.add_argument("--fused-amend", action="store_true",
                    help="MAC passes with MAC_F_FUSED_AMEND (the reduce updates the ring)")
    ap.add_argument("--ring-bf16", action="store_true",
                    help="MAC passes with MAC_F_RING_BF16 (ring queries kept as bfloat16)")
    ap.add_argument("--stale-ring", action="store_true",
                    help="MAC passes with MAC_F_STALE_RING (match skips the previous call's entry)")
    ap.add_argument("--table5", action="store_true",
                    help="Table 5 analog: match / complete / reduce / attention-phase us at a "
                         "1024-entry window, batch 1, 32K and 60K context, KV 1-20 %% (one JSON line)")
    ap.add_argument("--prefill", action="store_true",
                    help="Table 8 analog: MAC over a prompt (mac_prefill, unbounded window) vs "
                         "the same engine with reuse off (one JSON line)")
    ap.add_argument("--band-per-head", default="",
                    help="comma list of bands r_h, cycled over the query heads of the MAC passes")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a 2 GiB device copy (reference for HBM counters)")
    return ap.parse_args()


class Bench:
    def __init__(self, w, flags, K, V, paged, table, bands=None):
        import torch
        import kv_reuse_amd as mac
        self.w = w
        self.torch = torch
        self.mac = mac
        dev = "cuda"
        self.kc, self.vc, self.table = K, V, table
        self.seq = torch.zeros(w.B, dtype=torch.int32, device=dev)
        self.pos = torch.zeros(w.B, dtype=torch.int32, device=dev)
        self.cfg = mac.make_config(
            batch=w.B, num_q_heads=w.Hq, num_kv_heads=w.Hkv, ring_size=w.W, band=w.r, tau=w.tau,
            rope_theta=w.theta, layout=mac.MAC_KV_PAGED if paged else mac.MAC_KV_CONTIGUOUS,
            kv_dtype=mac.MAC_FP32 if w.kv == "fp32" else mac.MAC_BF16, max_seq_len=w.n_cap,
            flags=flags, band_per_head=bands)
        self.stream = torch.cuda.current_stream()
        self.layer = mac.MacLayer(self.cfg, main_stream=self.stream)
        self.view = mac.make_kv_view(self.kc, self.vc, self.seq, self.table,
                                     num_pages=self.kc.shape[0] if paged else 0)
        self.out = torch.empty((w.B, w.Hq, w.d), dtype=torch.float32, device=dev)

    def step(self, t, q, k_new, v_new, scrub=None, override=None):
        """One decode step.  Returns the counters (synchronises) with the last
        step's kernel times (MAC_F_TIMING) and "span_us": the decode call's work
        on the main stream (match -> reduce) between two stream events, with
        nothing recorded between its kernels."""
        w = self.w
        torch = self.torch
        if scrub is not None:
            # read 1 GiB: evicts the KV cache from L2 and the Infinity Cache
            # without leaving dirty lines for the timed kernels to write back
            scrub[1].copy_(scrub[0].sum())
        self.pos.fill_(w.C + t)
        self.seq.fill_(w.C + t + 1)
        self.layer.append_kv(self.view, k_new, v_new, self.pos, self.stream)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(self.stream)
        self.layer.decode_step(self.view, q, self.out, override, self.stream)
        e1.record(self.stream)
        st = self.layer.stats()            # synchronises; last step's kernel times
        st["span_us"] = e0.elapsed_time(e1) * 1e3
        return st

    def enqueue(self, t, q, k_new, v_new):
        """One decode step enqueued without any host synchronisation."""
        w = self.w
        self.pos.fill_(w.C + t)
        self.seq.fill_(w.C + t + 1)
        self.layer.append_kv(self.view, k_new, v_new, self.pos, self.stream)
        self.layer.decode_step(self.view, q, self.out, None, self.stream)


def pipelined_us(w, flags, cache, q_dev, k_rows, v_rows, warmup, steps, scrub=None):
    """Attention phase with the launches queued ahead, as a serving loop
    issues them: after `warmup` synchronised steps from a fresh ring, `steps`
    steps are enqueued back to back (the optional scrub read, append, then
    the decode call between two stream events) and the host synchronises once
    at the end.  The mean of the event spans is the decode call's device time
    without the host's launch latency; it includes any wait for the previous
    step's amend."""
    import torch
    bn = Bench(w, flags, *cache)
    for t in range(warmup):
        bn.step(t, q_dev[t], k_rows[t], v_rows[t], scrub)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    for i, t in enumerate(range(warmup, warmup + steps)):
        if scrub is not None:
            scrub[1].copy_(scrub[0].sum())
        bn.pos.fill_(w.C + t)
        bn.seq.fill_(w.C + t + 1)
        bn.layer.append_kv(bn.view, k_rows[t], v_rows[t], bn.pos, bn.stream)
        ev[i][0].record(bn.stream)
        bn.layer.decode_step(bn.view, q_dev[t], bn.out, None, bn.stream)
        ev[i][1].record(bn.stream)
    bn.layer.stats()                        # synchronises every stream of the handle
    bn.layer.close()
    return float(np.mean([a.elapsed_time(b) * 1e3 for a, b in ev]))


def loop_us(w, flags, cache, q_dev, k_rows, v_rows, warmup, steps, hit_rate=None):
    """Microseconds per step of a decode loop run back to back (append and
    decode enqueued with no host synchronisation, as a serving loop runs):
    each step's match waits for the previous step's amend (the one before it
    with the stale-by-one ring), so this is the step's whole cost, amend
    included.  Events on the decode stream around the timed steps; a fresh
    ring, then `warmup` synchronised steps first.  `hit_rate`, a dict, gets
    the timed steps' share of heads that hit, under the same key."""
    import torch
    bn = Bench(w, flags, *cache)
    for t in range(warmup):
        bn.step(t, q_dev[t], k_rows[t], v_rows[t])
    h0 = bn.layer.stats()["hits"]
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(bn.stream)
    for t in range(warmup, warmup + steps):
        bn.enqueue(t, q_dev[t], k_rows[t], v_rows[t])
    e1.record(bn.stream)
    h1 = bn.layer.stats()["hits"]          # synchronises every stream of the handle
    us = e0.elapsed_time(e1) * 1e3 / steps
    bn.layer.close()
    if hit_rate is not None:
        hit_rate[flags] = (h1 - h0) / (steps * w.B * w.Hq)
    return us


def speedup_point(name, steps=24, warmup=40):
    """MAC attention phase (async, fused and decode-stream amend) vs the in-house
    full-attention kernel on one workload, with a 1 GiB scrub read before every
    step (the KV of small contexts fits in the 256 MB Infinity Cache).  The
    attention phase is timed by stream events around the decode call, so the
    scrub is not in it."""
    import torch
    import kv_reuse_amd as mac
    from workloads import get_config, kv_logical, page_table, queries, to_paged
    w = get_config(name)
    total = warmup + steps
    K, V = kv_logical(w, "cuda")
    idx = torch.arange(w.C, w.C + total, device="cuda")
    k_rows = K[:, :, idx].permute(2, 0, 1, 3).contiguous()
    v_rows = V[:, :, idx].permute(2, 0, 1, 3).contiguous()
    q_dev = torch.as_tensor(queries(w, steps=total), device="cuda")
    paged = w.layout == "paged"
    if paged:
        tab = page_table(w)
        kc, vc, table = to_paged(K, tab), to_paged(V, tab), torch.as_tensor(tab, device="cuda")
    else:
        kc, vc, table = K, V, None
    scrub = [torch.ones(1 << 28, dtype=torch.float32, device="cuda"),
             torch.zeros((), dtype=torch.float32, device="cuda")]
    res = {}
    for label, flags in (("mac", 0), ("mac_fused_amend", mac.MAC_F_FUSED_AMEND),
                         ("mac_sync_amend", mac.MAC_F_SYNC_AMEND),
                         ("full", mac.MAC_F_DISABLE_REUSE)):
        bn = Bench(w, flags, kc, vc, paged, table)
        att, hits = [], []
        prev = None
        for t in range(total):
            st = bn.step(t, q_dev[t], k_rows[t], v_rows[t], scrub)
            if t >= warmup:
                att.append(st["span_us"])
                hits.append(st["hits"] - prev["hits"])
            prev = st
        bn.layer.close()
        res[label] = (float(np.mean(att)), float(np.sum(hits)) / (len(hits) * w.B * w.Hq))
    # per-kernel HIP events (MAC_F_TIMING), the same steps and scrub
    kernels = {}
    for label, flags in (("mac", 0), ("full", mac.MAC_F_DISABLE_REUSE)):
        bn = Bench(w, flags | mac.MAC_F_TIMING, kc, vc, paged, table)
        kern, toks, prev = {}, 0, None
        for t in range(total):
            st = bn.step(t, q_dev[t], k_rows[t], v_rows[t], scrub)
            if t >= warmup:
                for k in ("match", "complete", "reduce", "amend"):
                    kern.setdefault(k, []).append(st["last_us_" + k])
                toks += st["kv_tokens_critical"] - prev["kv_tokens_critical"]
            prev = st
        bn.layer.close()
        kv = toks * 2 * w.d * w.kv_elem_bytes / steps
        kernels[label] = kernel_rates(w, {k: float(np.mean(v)) for k, v in kern.items()}, kv)
        kernels[label]["kv_bytes_per_step"] = kv
    cache = (kc, vc, paged, table)
    piped = {label: pipelined_us(w, flags, cache, q_dev, k_rows, v_rows, warmup, steps, scrub)
             for label, flags in (("mac", 0), ("mac_fused_amend", mac.MAC_F_FUSED_AMEND),
                                  ("full", mac.MAC_F_DISABLE_REUSE))}
    graph = fused_graph_loops(w, kc, vc, paged, table, k_rows, v_rows, q_dev, warmup)
    return {"workload": name, "context": w.C, "batch": w.B,
            "mac_attention_us": res["mac"][0], "full_attention_us": res["full"][0],
            "fused_amend_loop_us_per_step": graph,
            "head_hit_rate": res["mac"][1], "speedup": res["full"][0] / res["mac"][0],
            # the other amend forms: no second stream, so no cross-queue event
            # after the reduce (sync: amend runs inside the span)
            "mac_fused_amend_attention_us": res["mac_fused_amend"][0],
            "mac_sync_amend_attention_us": res["mac_sync_amend"][0],
            "speedup_fused_amend": res["full"][0] / res["mac_fused_amend"][0],
            "kernels": kernels, "attention_us_pipelined": piped,
            "speedup_pipelined": piped["full"] / piped["mac"],
            "steps": steps, "warmup": warmup}


def fused_graph_loops(w, kc, vc, paged, table, k_rows, v_rows, q_dev, start, steps=16):
    """Back-to-back fused-amend decode loops (append + decode per step, each
    step's inputs written in place first, no host synchronisation): the
    library called eagerly, and the same step captured once into a HIP graph
    and replayed.  Microseconds per step between two stream events."""
    import torch
    import kv_reuse_amd as mac
    out = {}
    for label in ("eager", "graph"):
        bn = Bench(w, mac.MAC_F_FUSED_AMEND, kc, vc, paged, table)
        s = torch.cuda.Stream()
        k_in, v_in, q_in = k_rows[0].clone(), v_rows[0].clone(), q_dev[0].clone()

        def inputs(t):
            bn.pos.fill_(w.C + t)
            bn.seq.fill_(w.C + t + 1)
            k_in.copy_(k_rows[t])
            v_in.copy_(v_rows[t])
            q_in.copy_(q_dev[t])

        def step():
            bn.layer.append_kv(bn.view, k_in, v_in, bn.pos, s)
            bn.layer.decode_step(bn.view, q_in, bn.out, None, s)

        torch.cuda.synchronize()
        with torch.cuda.stream(s):
            for t in range(start - 2):          # warm-up on the loop's stream
                inputs(t)
                step()
            g = None
            if label == "graph":
                torch.cuda.synchronize()
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=s):
                    step()
            torch.cuda.synchronize()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(s)
            for t in range(start - 2, start - 2 + steps):
                inputs(t)
                if g is None:
                    step()
                else:
                    g.replay()
            e1.record(s)
        torch.cuda.synchronize()
        out[label] = e0.elapsed_time(e1) * 1e3 / steps
        bn.layer.close()
    return out


def workload_cache(w, total):
    """K/V of a workload in HBM (paged or contiguous) and the rows appended
    during `total` steps, and its queries, all on the GPU."""
    import torch
    from workloads import kv_logical, page_table, queries, to_paged
    K, V = kv_logical(w, "cuda")
    idx = torch.arange(w.C, w.C + total, device="cuda")
    k_rows = K[:, :, idx].permute(2, 0, 1, 3).contiguous()
    v_rows = V[:, :, idx].permute(2, 0, 1, 3).contiguous()
    q_dev = torch.as_tensor(queries(w, steps=total), device="cuda")
    paged = w.layout == "paged"
    if paged:
        tab = page_table(w)
        cache = (to_paged(K, tab), to_paged(V, tab), True, torch.as_tensor(tab, device="cuda"))
        del K, V
    else:
        cache = (K, V, False, None)
    return cache, k_rows, v_rows, q_dev


def measure(w, flags, cache, k_rows, v_rows, q_dev, warm, steps, scrub=None):
    """Two passes over the same steps from a fresh ring: the attention phase
    between two stream events per step (with the per-head decisions read
    after each step), then the library's per-kernel HIP events."""
    import kv_reuse_amd as mac
    G = w.Hq // w.Hkv
    out = {}
    for timing in (False, True):
        fl = flags | (mac.MAC_F_TIMING if timing else mac.MAC_F_RECORD_DEBUG)
        bn = Bench(w, fl, *cache)
        span, hits, toks, grp, kern, prev = [], 0, 0, 0, {}, None
        for t in range(warm + steps):
            st = bn.step(t, q_dev[t], k_rows[t], v_rows[t], scrub)
            if t >= warm:
                if timing:
                    for k in ("match", "complete", "reduce", "amend"):
                        kern.setdefault(k, []).append(st["last_us_" + k])
                else:
                    span.append(st["span_us"])
                    hit = bn.layer.debug_last()[1].reshape(w.B, w.Hkv, G)
                    grp += int(hit.all(axis=-1).sum())
                hits += st["hits"] - (prev["hits"] if prev else 0)
                toks += st["kv_tokens_critical"] - (prev["kv_tokens_critical"] if prev else 0)
            prev = st
        bn.layer.close()
        if timing:
            assert toks == out["kv_tokens"], "the instrumented pass streamed different bytes"
            out["kernel_us"] = {k: float(np.mean(v)) for k, v in kern.items()}
        else:
            out.update({"attention_us": float(np.mean(span)), "kv_tokens": toks,
                        "head_hit_rate": hits / (steps * w.B * w.Hq),
                        "groups_all_hit_rate": grp / (steps * w.B * w.Hkv)})
    return out


def kernel_rates(w, kernel_us, kv_bytes, ring_bytes_per_elem=4):
    """Achieved GB/s (and fraction of 8 TB/s) of the two streaming kernels from
    their HIP-event durations: match on the ring queries it scans (plus this
    step's queries in and the two query copies out), complete on the K/V rows
    of the union spans plus the post-RoPE queries."""
    q = w.B * w.Hq * w.d * 4
    match_bytes = w.B * w.Hq * w.W * w.d * ring_bytes_per_elem + w.B * w.W * 4 + 3 * q
    out = {}
    for k, nbytes in (("match", match_bytes), ("complete", kv_bytes + q)):
        us = kernel_us[k]
        gbps = nbytes / (us * 1e-6) / 1e9 if us > 0 else None
        out[k] = {"us": us, "bytes": nbytes, "gbps": gbps,
                  "frac": gbps / PEAK_HBM_GBS if gbps else None}
    for k in ("reduce", "amend"):
        if k in kernel_us:
            out[k] = {"us": kernel_us[k]}
    return out


def workload_record(name, warm, steps, bands=(None,), loop=True):
    """Compact record of one workload: MAC (async amend) against the in-house
    full-attention kernel on the same cache, `steps` steps after `warm`
    warm-up steps from a fresh ring.  With several bands, one MAC record per
    band (full attention does not depend on it).  Per record: attention-phase
    µs/step (synchronised step), tokens/s, KV bytes per step, the complete
    kernel's achieved GB/s and fraction of 8 TB/s, head-hit and all-hit-group
    shares, the back-to-back loop µs/step (amend included) and MAC vs full;
    and the same MAC step with fused amend (no second stream)."""
    import torch
    import kv_reuse_amd as mac
    from workloads import get_config, scaled
    w0 = get_config(name)
    total = warm + steps
    assert total <= w0.steps
    cache, k_rows, v_rows, q_dev = workload_cache(w0, total)
    row_bytes = 2 * w0.d * w0.kv_elem_bytes
    q_bytes = w0.B * w0.Hq * w0.d * 4

    def summarise(w, flags):
        m = measure(w, flags, cache, k_rows, v_rows, q_dev, warm, steps)
        kv = m.pop("kv_tokens") * row_bytes / steps
        gbps = (kv + q_bytes) / (m["kernel_us"]["complete"] * 1e-6) / 1e9
        m.update({"tokens_per_s": w.B / (m["attention_us"] * 1e-6), "kv_bytes_per_step": kv,
                  "complete_gbps": gbps, "complete_frac": gbps / PEAK_HBM_GBS})
        if loop:
            m["loop_us_per_step"] = loop_us(w, flags, cache, q_dev, k_rows, v_rows, min(warm, 8),
                                            min(steps, 16))
        return m

    full = summarise(w0, mac.MAC_F_DISABLE_REUSE)
    recs = []
    for r in bands:
        w = w0 if r is None else scaled(w0, r=r)
        m = summarise(w, 0)
        m["band"] = w.r
        m["speedup_vs_full"] = full["attention_us"] / m["attention_us"]
        if loop:
            m["loop_speedup_vs_full"] = full["loop_us_per_step"] / m["loop_us_per_step"]
        # the fused amend form (no second stream): attention phase and loop only
        f = measure(w, mac.MAC_F_FUSED_AMEND, cache, k_rows, v_rows, q_dev, warm, steps)
        m["fused_amend"] = {"attention_us": f["attention_us"],
                            "speedup_vs_full": full["attention_us"] / f["attention_us"]}
        if loop:
            fl = loop_us(w, mac.MAC_F_FUSED_AMEND, cache, q_dev, k_rows, v_rows, min(warm, 8),
                         min(steps, 16))
            m["fused_amend"].update({"loop_us_per_step": fl,
                                     "loop_speedup_vs_full": full["loop_us_per_step"] / fl})
        recs.append(m)
    del cache, k_rows, v_rows, q_dev
    torch.cuda.empty_cache()
    rec = {"workload": name, "batch": w0.B, "context": w0.C, "q_heads": w0.Hq,
           "kv_heads": w0.Hkv, "kv_dtype": w0.kv, "kv_layout": w0.layout, "ring": w0.W,
           "tau": w0.tau, "rho": list(w0.rho), "warmup": warm, "steps": steps,
           "full_attention": full}
    if len(recs) == 1:
        rec["mac"] = recs[0]
    else:
        rec["mac_by_band"] = recs
    return rec


def multilayer_record(name="llama32k", layers=8, warm=16, steps=32):
    """Several layers of one small-batch workload decoded back to back, each
    layer its own handle, cache and (library-created) amend stream, all on one
    decode stream with no host synchronisation: µs per layer and step for MAC
    with async amend, with fused amend, and for full attention.  Between two
    calls of a layer the other layers' calls run, as in a model's decode."""
    import torch
    import kv_reuse_amd as mac
    from workloads import get_config
    w = get_config(name)
    total = warm + steps
    caches = [workload_cache(w, total) for _ in range(layers)]
    k_rows, v_rows, q_dev = caches[0][1], caches[0][2], caches[0][3]
    res = {}
    for label, flags in (("mac", 0), ("mac_sync_amend", mac.MAC_F_SYNC_AMEND),
                         ("mac_fused_amend", mac.MAC_F_FUSED_AMEND),
                         ("full_attention", mac.MAC_F_DISABLE_REUSE)):
        bns = [Bench(w, flags, *c[0]) for c in caches]
        for t in range(warm):
            for bn in bns:
                bn.enqueue(t, q_dev[t], k_rows[t], v_rows[t])
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(bns[0].stream)
        for t in range(warm, total):
            for bn in bns:
                bn.enqueue(t, q_dev[t], k_rows[t], v_rows[t])
        e1.record(bns[0].stream)
        torch.cuda.synchronize()
        hits = sum(bn.layer.stats()["hits"] for bn in bns)
        for bn in bns:
            bn.layer.close()
        us = e0.elapsed_time(e1) * 1e3 / (steps * layers)
        res[label] = {"us_per_layer_step": us, "tokens_per_s": w.B / (us * 1e-6 * layers),
                      "head_hit_rate": hits / (total * layers * w.B * w.Hq)}
    del caches, k_rows, v_rows, q_dev
    torch.cuda.empty_cache()
    return {"workload": name, "layers": layers, "batch": w.B, "context": w.C, "warmup": warm,
            "steps": steps, **res,
            "speedup_vs_full": res["full_attention"]["us_per_layer_step"] / res["mac"]["us_per_layer_step"],
            "speedup_vs_full_sync_amend": (res["full_attention"]["us_per_layer_step"] /
                                           res["mac_sync_amend"]["us_per_layer_step"]),
            "speedup_vs_full_fused_amend": (res["full_attention"]["us_per_layer_step"] /
                                            res["mac_fused_amend"]["us_per_layer_step"]),
            "note": "layers decoded back to back on one stream, no host synchronisation; "
                    "attention path only (append, match, complete, reduce, amend)"}


def contgen_run(warm, steps, decisions=True):
    """Continuous generation: 32 layers x batch 32, 16384-token prompt then
    generated tokens, K/V appended every step and amend overlapping the next
    layers on a shared stream.  Steady state is measured at the mid-run context
    (position 16384 + 8192): the ring remembers only its last W steps, so the
    window starts there with a fresh ring, warms up, then times the steps.
    With `decisions`, one more untimed MAC pass over the same steps reads
    every layer's per-head decisions (share of all-hit KV groups)."""
    import torch
    import kv_reuse_amd as mac
    from workloads import get_config, kv_logical, page_table, queries, scaled, to_paged
    base = get_config("contgen")
    total = warm + steps
    ctx0 = base.C + base.steps // 2
    w = scaled(base, C=ctx0, steps=total)
    L = w.layers
    G = w.Hq // w.Hkv
    t0 = time.perf_counter()
    tab_np = page_table(w)
    table = torch.as_tensor(tab_np, device="cuda")
    kcs, vcs, krows, vrows, qs = [], [], [], [], []
    idx = torch.arange(w.C, w.C + total, device="cuda")
    for layer in range(L):
        K, V = kv_logical(w, "cuda", layer=layer)
        krows.append(K[:, :, idx].permute(2, 0, 1, 3).contiguous())
        vrows.append(V[:, :, idx].permute(2, 0, 1, 3).contiguous())
        kcs.append(to_paged(K, tab_np))
        vcs.append(to_paged(V, tab_np))
        del K, V
        qs.append(torch.as_tensor(queries(w, steps=total, layer=layer), device="cuda"))
    torch.cuda.synchronize()
    setup = time.perf_counter() - t0
    seq = torch.zeros(w.B, dtype=torch.int32, device="cuda")
    pos = torch.zeros(w.B, dtype=torch.int32, device="cuda")
    out = torch.empty((w.B, w.Hq, w.d), dtype=torch.float32, device="cuda")
    main = torch.cuda.current_stream()
    amend = torch.cuda.Stream()
    res = {}
    passes = [("mac", 0), ("mac_sync_amend", mac.MAC_F_SYNC_AMEND),
              ("mac_fused_amend", mac.MAC_F_FUSED_AMEND),
              ("mac_fused_amend_ring_bf16", mac.MAC_F_FUSED_AMEND | mac.MAC_F_RING_BF16),
              ("full", mac.MAC_F_DISABLE_REUSE)]
    if decisions:
        passes.append(("decisions", mac.MAC_F_RECORD_DEBUG))
    for label, flags in passes:
        cfg = mac.make_config(batch=w.B, num_q_heads=w.Hq, num_kv_heads=w.Hkv, ring_size=w.W,
                              band=w.r, tau=w.tau, rope_theta=w.theta, layout=mac.MAC_KV_PAGED,
                              kv_dtype=mac.MAC_BF16, max_seq_len=w.n_cap, flags=flags)
        layers = [mac.MacLayer(cfg, main_stream=main, amend_stream=amend) for _ in range(L)]
        views = [mac.make_kv_view(kcs[i], vcs[i], seq, table, num_pages=kcs[i].shape[0])
                 for i in range(L)]
        all_hit = []

        def run(t):
            pos.fill_(w.C + t)
            seq.fill_(w.C + t + 1)
            for i in range(L):
                layers[i].append_kv(views[i], krows[i][t], vrows[i][t], pos, main)
                layers[i].decode_step(views[i], qs[i][t], out, None, main)
                if label == "decisions" and t >= warm:
                    hit = layers[i].debug_last()[1].reshape(w.B, w.Hkv, G)
                    all_hit.append(float(hit.all(axis=-1).mean()))

        for t in range(warm):
            run(t)
        torch.cuda.synchronize()
        h0 = sum(l.stats()["hits"] for l in layers)
        k0 = sum(l.stats()["kv_tokens_critical"] for l in layers)
        wall0 = time.perf_counter()
        for t in range(warm, total):
            run(t)
        torch.cuda.synchronize()
        wall = time.perf_counter() - wall0
        st = [l.stats() for l in layers]
        hits = sum(x["hits"] for x in st) - h0
        toks = sum(x["kv_tokens_critical"] for x in st) - k0
        for l in layers:
            l.close()
        if label == "decisions":
            res["mac"]["groups_all_hit_rate"] = float(np.mean(all_hit))
            continue
        res[label] = {"tokens_per_s": w.B * steps / wall, "ms_per_step": wall * 1e3 / steps,
                      "head_hit_rate": hits / (steps * L * w.B * w.Hq),
                      "kv_bytes_per_step": toks * 2 * w.d * 2 / steps,
                      "hbm_gbps": toks * 2 * w.d * 2 / wall / 1e9}
        res[label]["hbm_frac"] = res[label]["hbm_gbps"] / PEAK_HBM_GBS
    del kcs, vcs, krows, vrows, qs
    torch.cuda.empty_cache()
    return {"workload": "contgen", "batch": w.B, "layers": L, "context_at_window": ctx0,
            "q_heads": w.Hq, "kv_heads": w.Hkv, "ring": w.W, "band": w.r, "tau": w.tau,
            "rho": list(base.rho), "jump_every": base.jump_every, "warmup": warm,
            "steps": steps, "mac": res["mac"], "mac_sync_amend": res["mac_sync_amend"],
            "mac_fused_amend": res["mac_fused_amend"],
            "mac_fused_amend_ring_bf16": res["mac_fused_amend_ring_bf16"],
            "full_attention": res["full"],
            "speedup_vs_full": res["mac"]["tokens_per_s"] / res["full"]["tokens_per_s"],
            "speedup_vs_full_sync_amend": (res["mac_sync_amend"]["tokens_per_s"] /
                                           res["full"]["tokens_per_s"]),
            "speedup_vs_full_fused_amend": (res["mac_fused_amend"]["tokens_per_s"] /
                                            res["full"]["tokens_per_s"]),
            "speedup_vs_full_fused_amend_ring_bf16": (
                res["mac_fused_amend_ring_bf16"]["tokens_per_s"] / res["full"]["tokens_per_s"]),
            "setup_s": setup,
            "note": "attention path only (append, match, complete, reduce, amend on a second "
                    "stream shared by the layers); wall clock over the timed steps, no FFN"}


def contgen(args):
    """`--config contgen`: the continuous-generation record as its own line."""
    from workloads import get_config
    W = get_config("contgen").W
    rec = contgen_run(max(args.warmup, W + 8), args.steps)
    line = {
        "metric": "steady-state tokens/s, continuous generation (32 layers, batch 32, GQA 32q/8kv)",
        "value": rec["mac"]["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1,
        "steps": rec["steps"], "warmup": rec["warmup"], "ms_per_step": rec["mac"]["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {k: rec[k] for k in ("workload", "batch", "layers", "context_at_window",
                                       "q_heads", "kv_heads", "ring", "band", "tau", "rho",
                                       "jump_every", "note")},
    }
    line.update({k: v for k, v in rec.items() if k not in line["config"]})
    print(json.dumps(line), flush=True)


def table5(args):
    """Synthetic analog of the pages' Table 5: the attention path at a fixed
    1024-entry match window, batch 1, 32q/8kv, contiguous bf16 K/V at 32K and
    60K context.  The queries (AR(1), rho = 0.99) make every head hit its
    previous step, so each group reads its band plus the tail; the band r
    sets the share of the context read, KV % = (r + 1) / context, at the
    pages' 1, 5, 10 and 20 %.  Each step follows a 1 GiB read scrub (the
    cache fits the 256 MB Infinity Cache); per-kernel HIP events (match;
    complete, whose plan is the load balancer; reduce) and the attention-phase
    span, against the in-house full-attention kernel on the same cache.
    Prints one JSON line."""
    import torch
    import kv_reuse_amd as mac
    from workloads import get_config, scaled
    warm, steps = 8, 16
    scrub = [torch.ones(1 << 28, dtype=torch.float32, device="cuda"),
             torch.zeros((), dtype=torch.float32, device="cuda")]
    rows = []
    for C in (32768, 61440):
        w0 = scaled(get_config("llama32k"), C=C, W=1024, rho=("const", 0.99), steps=warm + steps)
        cache, k_rows, v_rows, q_dev = workload_cache(w0, warm + steps)
        full_tok = sum(w0.B * w0.Hkv * (C + t + 1) for t in range(warm, warm + steps))
        f = measure(w0, mac.MAC_F_DISABLE_REUSE, cache, k_rows, v_rows, q_dev, warm, steps, scrub)
        for kvp in (1, 5, 10, 20):
            r = max(1, int(round(kvp / 100.0 * C)) - 1)
            w = scaled(w0, r=r)
            m = measure(w, 0, cache, k_rows, v_rows, q_dev, warm, steps, scrub)
            rows.append({"context": C, "kv_pct_target": kvp, "band": r,
                         "kv_pct": 100.0 * m["kv_tokens"] / full_tok,
                         "head_hit_rate": m["head_hit_rate"],
                         "full_attention_us": f["attention_us"],
                         "full_attention_complete_us": f["kernel_us"]["complete"],
                         "match_us": m["kernel_us"]["match"],
                         "complete_us": m["kernel_us"]["complete"],
                         "reduce_us": m["kernel_us"]["reduce"],
                         "amend_us_second_stream": m["kernel_us"]["amend"],
                         "attention_us": m["attention_us"],
                         "speedup_vs_full": f["attention_us"] / m["attention_us"]})
        del cache, k_rows, v_rows, q_dev
        torch.cuda.empty_cache()
    print(json.dumps({"table5": rows,
                      "config": {"workload": "llama32k-shaped, batch 1", "q_heads": 32,
                                 "kv_heads": 8, "ring": 1024, "tau": 0.3, "rho": 0.99,
                                 "kv_layout": "contiguous", "warmup": warm, "steps": steps,
                                 "data": "synthetic"}}), flush=True)


def figures(args):
    """Synthetic analogs of the pages' Figures 5, 4 and 8 (no datasets, no
    model queries; the AR(1) recipes of the workloads):
      fig5: head hit rate and skipped-key share vs tau and window W, and vs the
            query correlation rho (128K x 16 paged cache);
      fig4: MAC-vs-full relative output error vs the reuse gap m - p (hits
            forced through the override input) and the band r;
      fig8a: match latency vs query heads per KV head G and window W;
      fig8b: complete kernel time with the balanced plan, with an unbalanced
            one (the same number of waves per KV group), and the ideal
            (bytes at the full-attention kernel's bandwidth).
    Prints one JSON line."""
    import torch
    import kv_reuse_amd as mac
    from workloads import get_config, kv_logical, page_table, queries, scaled, to_paged
    base = scaled(get_config("b16_128k"), steps=40)
    total = base.steps
    K, V = kv_logical(base, "cuda")
    idx = torch.arange(base.C, base.C + total, device="cuda")
    k_rows = K[:, :, idx].permute(2, 0, 1, 3).contiguous()
    v_rows = V[:, :, idx].permute(2, 0, 1, 3).contiguous()
    tab = page_table(base)
    cache = (to_paged(K, tab), to_paged(V, tab), True, torch.as_tensor(tab, device="cuda"))
    del K, V
    B, Hq, Hkv = base.B, base.Hq, base.Hkv

    def rates(w, warm=4, steps=8):
        qd = torch.as_tensor(queries(w, steps=warm + steps), device="cuda")
        bn = Bench(w, 0, *cache)
        hits = toks = full = 0
        att, prev = [], None
        for t in range(warm + steps):
            st = bn.step(t, qd[t], k_rows[t], v_rows[t])
            if t >= warm:
                hits += st["hits"] - prev["hits"]
                toks += st["kv_tokens_critical"] - prev["kv_tokens_critical"]
                full += (w.C + t + 1) * B * Hkv
                att.append(st["span_us"])
            prev = st
        bn.layer.close()
        return {"head_hit_rate": hits / (steps * B * Hq), "skipped_keys": 1.0 - toks / full,
                "attention_us": float(np.mean(att))}

    parts = set(args.figures.split(","))
    fig5, fig5_rho, fig4, fig8, fig8b, full_us = [], [], [], [], [], None
    row_bytes = 2 * base.d * 2

    def complete_us(w, flags, warm=4, steps=8):
        qd = torch.as_tensor(queries(w, steps=warm + steps), device="cuda")
        bn = Bench(w, flags | mac.MAC_F_TIMING, *cache)
        us, toks, prev = [], 0, None
        for t in range(warm + steps):
            st = bn.step(t, qd[t], k_rows[t], v_rows[t])
            if t >= warm:
                us.append(st["last_us_complete"])
                toks += st["kv_tokens_critical"] - prev["kv_tokens_critical"]
            prev = st
        bn.layer.close()
        return float(np.mean(us)), toks * row_bytes / steps

    if "fig8b" in parts:
        # Figure 8 (b): the plan against an unbalanced split and the ideal
        f_us, f_bytes = complete_us(scaled(base, tau=-1.0), 0)
        bw = f_bytes / (f_us * 1e-6)
        for label, w in (("headline queries", base),
                         ("rho 0.96", scaled(base, rho=("const", 0.96))),
                         ("rho 0.97", scaled(base, rho=("const", 0.97))),
                         ("rho 0.99", scaled(base, rho=("const", 0.99)))):
            bal, nb = complete_us(w, 0)
            unb, nb2 = complete_us(w, mac.MAC_F_UNBALANCED_PLAN)
            assert nb == nb2, "the two plans streamed different bytes"
            fig8b.append({"queries": label, "kv_bytes_per_step": nb, "balanced_us": bal,
                          "unbalanced_us": unb, "ideal_us": nb / bw * 1e6,
                          "full_attention_complete_us": f_us})

    for tau in ((0.1, 0.2, 0.3, 0.45, 0.6) if "fig5" in parts else ()):
        for W in (16, 32, 256, 1024):
            r = rates(scaled(base, tau=tau, W=W))
            r.update({"tau": tau, "W": W})
            fig5.append(r)
    if "fig5" in parts:
        full_us = rates(scaled(base, tau=-1.0))["attention_us"]
    for rho in ((0.9, 0.95, 0.96, 0.97, 0.98, 0.99) if "fig5" in parts else ()):
        r = rates(scaled(base, rho=("const", rho)))
        r.update({"rho": rho, "speedup_vs_full": full_us / r["attention_us"]})
        fig5_rho.append(r)

    # fig4: every head forced to reuse the entry from gap steps back.  With
    # fresh summaries the warm-up steps are forced misses, so each stored
    # AS_{1:p-r} is exact attention of q_p; with natural decisions hits chain
    # (a hit's stored summary inherits the prefix it reused), so the prefix a
    # late step reuses was computed for a query many steps older.
    wq = scaled(base, rho=("const", 0.97))
    qd = torch.as_tensor(queries(wq, steps=total), device="cuda")
    warm, steps = 33, 4

    def outputs(w, flags, gap=0, fresh=False):
        bn = Bench(w, flags, *cache)
        res = []
        for t in range(warm + steps):
            ov = None
            if gap and t >= warm:
                ov = torch.full((B, Hq), w.C + t - gap, dtype=torch.int32, device="cuda")
            elif fresh and t < warm:
                ov = torch.full((B, Hq), -1, dtype=torch.int32, device="cuda")
            st = bn.step(t, qd[t], k_rows[t], v_rows[t], override=ov)
            if t >= warm:
                res.append(bn.out.clone())
                if gap:
                    assert st["override_invalid"] == 0, "forced position not in the ring"
        bn.layer.close()
        return res

    def rel_err(got, ref):
        e = torch.stack([(g - f).norm(dim=-1) / f.norm(dim=-1) for g, f in zip(got, ref)])
        return float(e.mean()), float(e.max())

    ref = outputs(wq, mac.MAC_F_DISABLE_REUSE) if "fig4" in parts else None
    for r in ((64, 256, 1024) if "fig4" in parts else ()):
        for gap in (1, 2, 4, 8, 16, 32):
            mean_e, max_e = rel_err(outputs(scaled(wq, r=r), 0, gap, fresh=True), ref)
            fig4.append({"r": r, "gap": gap, "summaries": "fresh", "mean_rel_err": mean_e,
                         "max_rel_err": max_e})
        mean_e, max_e = rel_err(outputs(scaled(wq, r=r), 0), ref)
        fig4.append({"r": r, "gap": None, "summaries": "natural chains (33 steps)",
                     "mean_rel_err": mean_e, "max_rel_err": max_e})
    del cache, k_rows, v_rows
    torch.cuda.empty_cache()

    # fig8a: match latency (library HIP events) vs G and W at a short context
    for G in ((1, 2, 4, 8) if "fig8a" in parts else ()):
        w8 = scaled(base, Hkv=Hq // G, C=4096, steps=12, rho=("const", 0.97))
        K, V = kv_logical(w8, "cuda")
        idx = torch.arange(w8.C, w8.C + 12, device="cuda")
        kr = K[:, :, idx].permute(2, 0, 1, 3).contiguous()
        vr = V[:, :, idx].permute(2, 0, 1, 3).contiguous()
        t8 = page_table(w8)
        c8 = (to_paged(K, t8), to_paged(V, t8), True, torch.as_tensor(t8, device="cuda"))
        del K, V
        q8 = torch.as_tensor(queries(w8, steps=12), device="cuda")
        for W in (16, 32, 64, 256, 1024, 2048):
            for ring, rflag, qbytes in (("fp32", 0, 4), ("bf16", mac.MAC_F_RING_BF16, 2)):
                bn = Bench(scaled(w8, W=W), mac.MAC_F_TIMING | rflag, *c8)
                us = []
                for t in range(12):
                    st = bn.step(t, q8[t], kr[t], vr[t])
                    if t >= 4:
                        us.append(st["last_us_match"])
                bn.layer.close()
                fig8.append({"G": G, "W": W, "ring": ring, "match_us": float(np.mean(us)),
                             "ring_bytes": B * Hq * W * w8.d * qbytes})
        del c8, kr, vr
        torch.cuda.empty_cache()

    print(json.dumps({"figures": {"fig5_tau_window": fig5, "fig5_rho": fig5_rho,
                                  "full_attention_us": full_us, "fig4_gap_band": fig4,
                                  "fig8_match": fig8, "fig8b_plan": fig8b},
                      "config": {"workload": "b16_128k", "batch": B, "context": base.C,
                                 "q_heads": Hq, "kv_heads": Hkv, "data": "synthetic"}}),
          flush=True)


def prefill_table8(args):
    """MAC-Attention in prefill (mac_prefill; window unbounded over the prompt)
    on a 4096-token prompt, batch 4, 32q/8kv paged bf16, AR(1) queries at rho
    0.97: hit and skipped-key rates and time per call at the (tau, r) pairs of
    the pages' Table 8, against the same engine with reuse off (plain causal
    attention).  Time: HIP events around the call, median of 5 after 1."""
    import torch
    import kv_reuse_amd as mac
    from workloads import get_config, kv_logical, page_table, queries, scaled, to_paged
    N = 4096
    w = scaled(get_config("b16_128k"), B=4, C=0, steps=N, rho=("const", 0.97))
    K, V = kv_logical(w, "cuda")
    tab = page_table(w)
    kc, vc, table = to_paged(K, tab), to_paged(V, tab), torch.as_tensor(tab, device="cuda")
    del K, V
    qd = torch.as_tensor(np.ascontiguousarray(queries(w, steps=N).transpose(1, 0, 2, 3)),
                         device="cuda")
    seq = torch.full((w.B,), N, dtype=torch.int32, device="cuda")
    out = torch.empty((w.B, N, w.Hq, w.d), device="cuda")
    view = mac.make_kv_view(kc, vc, seq, table, num_pages=kc.shape[0])
    causal_keys = w.B * w.Hkv * N * (N + 1) // 2

    def run(tau, r, flags):
        cfg = mac.make_config(batch=w.B, num_q_heads=w.Hq, num_kv_heads=w.Hkv, ring_size=w.W,
                              band=r, tau=tau, rope_theta=w.theta, layout=mac.MAC_KV_PAGED,
                              kv_dtype=mac.MAC_BF16, max_seq_len=w.n_cap, flags=flags)
        layer = mac.MacLayer(cfg)
        ms = []
        for it in range(6):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            layer.prefill(view, N, qd, out)
            e1.record()
            torch.cuda.synchronize()
            if it:
                ms.append(e0.elapsed_time(e1))
        st = layer.stats()
        layer.close()
        calls = 6
        return {"ms": float(np.median(ms)),
                "hit_rate": st["prefill_hits"] / st["prefill_decisions"],
                "skipped_keys": 1.0 - st["prefill_kv_tokens"] / (calls * causal_keys)}

    base = run(0.3, 256, mac.MAC_F_DISABLE_REUSE)
    rows = []
    for tau, r in ((0.30, 512), (0.35, 512), (0.45, 128), (0.45, 256)):
        x = run(tau, r, 0)
        x.update({"tau": tau, "r": r, "speedup_vs_causal": base["ms"] / x["ms"]})
        rows.append(x)
    print(json.dumps({"prefill_table8": rows, "causal_ms": base["ms"],
                      "config": {"workload": "prefill_4k", "batch": w.B, "prompt": N,
                                 "q_heads": w.Hq, "kv_heads": w.Hkv, "kv_layout": "paged",
                                 "rho": 0.97, "window": "unbounded (whole prompt)",
                                 "data": "synthetic"}}), flush=True)


def host_cpu():
    """The host the oracle ran on: CPU model and logical CPUs."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"model": model, "logical_cpus": os.cpu_count()}


def oracle_baseline(w, K, V, qs, n_req, n_steps, flags=0, warm=0):
    """fp64 oracle, as it stands, on the first n_req requests: `warm` untimed
    steps, then n_steps timed ones; seconds per timed step (flags: the
    oracle's F_* bits; F_DISABLE_REUSE gives its full-attention step)."""
    import oracle
    from workloads import bf16_bits
    Kg, Vg = [], []
    for b in range(n_req):
        for g in range(w.Hkv):
            Kg.append(bf16_bits(K[b, g, :w.C + warm + n_steps]))
            Vg.append(bf16_bits(V[b, g, :w.C + warm + n_steps]))
    orc = oracle.Oracle(n_req, w.Hq, w.Hkv, w.d, w.W, w.r, w.tau, w.theta,
                        kv_fp32=(w.kv == "fp32"), flags=flags)
    for t in range(warm):
        orc.step(Kg, Vg, np.full(n_req, w.C + t + 1, np.int32), qs[t, :n_req])
    t0 = time.perf_counter()
    for t in range(warm, warm + n_steps):
        orc.step(Kg, Vg, np.full(n_req, w.C + t + 1, np.int32), qs[t, :n_req])
    dt = time.perf_counter() - t0
    return dt / n_steps


def cpu_baseline(w, host_sample):
    """The fp64 oracle on the host cores: the headline shape on a bounded
    sample (n_req requests, CPU_WARM warm-up steps so the ring holds entries,
    CPU_STEPS timed, scaled to the batch; full attention on 4 steps), and the
    CPU-sized 4K workload over all its 256 steps with every thread and with
    one."""
    import torch
    import oracle
    from workloads import get_config, kv_logical, queries
    K, V, qs = host_sample
    n_req = K.shape[0]
    # the host's threads (OMP_NUM_THREADS when set): the OpenMP runtime is
    # shared with torch, whose own setting must not decide the oracle's
    threads = int(os.environ.get("OMP_NUM_THREADS") or os.cpu_count() or 1)
    oracle.set_threads(threads)
    threads = oracle.set_threads(0)
    sec = oracle_baseline(w, K, V, qs, n_req, CPU_STEPS, warm=CPU_WARM)
    sec_full = oracle_baseline(w, K, V, qs, n_req, 4, flags=oracle.F_DISABLE_REUSE)
    w1 = get_config("cpu4k")
    K1, V1 = kv_logical(w1, "cuda")
    K1, V1 = K1.cpu(), V1.cpu()
    q1 = queries(w1)
    c4k = {"threads": threads,
           "us_per_step": oracle_baseline(w1, K1, V1, q1, w1.B, w1.steps) * 1e6}
    oracle.set_threads(1)
    try:
        c4k["single_thread_us_per_step"] = oracle_baseline(w1, K1, V1, q1, w1.B, w1.steps) * 1e6
    finally:
        oracle.set_threads(threads)
    c4k["full_attention_us_per_step"] = oracle_baseline(
        w1, K1, V1, q1, w1.B, 16, flags=oracle.F_DISABLE_REUSE) * 1e6
    c4k["sample"] = ("the whole CPU-sized workload: 1 request, 8q/2kv fp32, 4096 + 256 steps "
                     "from an empty ring (full attention: its first 16 steps)")
    return {"value": sec * 1e6 * (w.B / n_req), "unit": "us/step", "cores": threads,
            "kind": "oracle", "host": host_cpu(),
            "full_attention_value": sec_full * 1e6 * (w.B / n_req),
            "sample": "%d of %d requests (all %d heads each): %d untimed steps fill the ring, "
                      "then %d timed steps (full attention: 4 steps), scaled by %d/%d to the "
                      "batch; OpenMP over (request, head), %d threads"
                      % (n_req, w.B, w.Hq, CPU_WARM, CPU_STEPS, w.B, n_req, threads),
            "cpu4k": c4k}


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU: the decode step runs on a single MI355X and "
              "--gpus %d is not supported (requests and KV groups shard without communication "
              "inside attention, so one GPU's share is the unit measured)"
              % args.gpus, file=sys.stderr)
        sys.exit(2)
    import torch
    import kv_reuse_amd as mac
    from workloads import get_config, kv_logical, page_table, queries, scaled, to_paged
    mac.load()
    torch.cuda.set_device(0)
    if args.config == "contgen":
        contgen(args)
        return
    if args.prefill:
        prefill_table8(args)
        return
    if args.table5:
        table5(args)
        return
    if args.figures:
        figures(args)
        return
    w = get_config(args.config)
    if args.r:
        w = scaled(w, r=args.r)
    for kv_pair in args.set:
        key, val = kv_pair.split("=", 1)
        cur = getattr(w, key)
        if key == "rho":
            parts = val.split(",")
            val = (parts[0],) + tuple(float(x) for x in parts[1:])
        else:
            val = type(cur)(val)
        w = scaled(w, **{key: val})
    total = args.warmup + args.steps
    assert total <= w.steps, "at most %d steps for this workload" % w.steps
    paged = w.layout == "paged"

    t_setup = time.perf_counter()
    K, V = kv_logical(w, "cuda")
    steps_idx = torch.arange(w.C, w.C + total, device="cuda")
    k_rows = K[:, :, steps_idx].permute(2, 0, 1, 3).contiguous()     # [steps, B, Hkv, d]
    v_rows = V[:, :, steps_idx].permute(2, 0, 1, 3).contiguous()
    qs = queries(w, steps=total)
    q_dev = torch.as_tensor(qs, device="cuda")
    if paged:
        tab_np = page_table(w)
        kc, vc = to_paged(K, tab_np), to_paged(V, tab_np)
        table = torch.as_tensor(tab_np, device="cuda")
    else:
        kc, vc, table = K, V, None
    host_sample = None
    if not args.no_cpu_baseline:
        n_req = min(2, w.B)
        n_cpu = CPU_WARM + CPU_STEPS
        host_sample = (K[:n_req, :, :w.C + n_cpu].cpu(), V[:n_req, :, :w.C + n_cpu].cpu(),
                       queries(w, steps=n_cpu)[:, :n_req].copy())
    if paged:
        del K, V
    torch.cuda.synchronize()
    t_setup = time.perf_counter() - t_setup

    # pass 1 (the timed region): the attention phase between two stream events
    # per step, no events between the kernels; each step is launched onto an
    # idle GPU (the counters are read between steps), so amend, which the
    # attention phase excludes, has ended before the next step starts
    mac_flags = ((mac.MAC_F_FUSED_AMEND if args.fused_amend else 0) |
                 (mac.MAC_F_RING_BF16 if args.ring_bf16 else 0) |
                 (mac.MAC_F_STALE_RING if args.stale_ring else 0))
    bands = None
    if args.band_per_head:
        cyc = [int(x) for x in args.band_per_head.split(",")]
        bands = [cyc[h % len(cyc)] for h in range(w.Hq)]
    bench = Bench(w, mac_flags, kc, vc, paged, table, bands)
    for t in range(args.warmup):
        bench.step(t, q_dev[t], k_rows[t], v_rows[t])
    st0 = bench.layer.stats()
    torch.cuda.synchronize()
    att, hits, toks = [], [], []
    prev = st0
    wall0 = time.perf_counter()
    for t in range(args.warmup, total):
        st = bench.step(t, q_dev[t], k_rows[t], v_rows[t])
        att.append(st["span_us"])
        hits.append(st["hits"] - prev["hits"])
        toks.append(st["kv_tokens_critical"] - prev["kv_tokens_critical"])
        prev = st
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    st1 = bench.layer.stats()
    bench.layer.close()
    # the same span with the steps enqueued back to back (device time without
    # the host's launch latency, any wait for the previous amend included)
    piped = pipelined_us(w, mac_flags, (kc, vc, paged, table), q_dev, k_rows, v_rows,
                         args.warmup, args.steps)

    # pass 2: the same steps from a fresh ring (same decisions, same bytes)
    # with the library's HIP events around every kernel (MAC_F_TIMING)
    kb = Bench(w, mac_flags | mac.MAC_F_TIMING | mac.MAC_F_RECORD_DEBUG, kc, vc, paged, table,
               bands)
    comp, match, red, amend, att_ev, toks2 = [], [], [], [], [], []
    mac_out, mac_hit = {}, {}     # steps 4..19: outputs and hit flags, for the deviation
    prev = None
    for t in range(total):
        st = kb.step(t, q_dev[t], k_rows[t], v_rows[t])
        if 4 <= t < 20:
            mac_out[t] = kb.out.clone()
            mac_hit[t] = torch.as_tensor(kb.layer.debug_last()[1], device="cuda").bool()
        if t >= args.warmup:
            comp.append(st["last_us_complete"])
            match.append(st["last_us_match"])
            red.append(st["last_us_reduce"])
            amend.append(st["last_us_amend"])
            att_ev.append(st["last_us_attention"])
            toks2.append(st["kv_tokens_critical"] - prev["kv_tokens_critical"])
        prev = st
    kb.layer.close()
    assert toks2 == toks, "the instrumented pass streamed different bytes"

    row_bytes = 2 * w.d * w.kv_elem_bytes                   # one key row + one value row
    kv_bytes = np.array(toks, np.float64) * row_bytes       # per step, per complete launch
    q_bytes = w.B * w.Hq * w.d * 4
    comp_bytes = kv_bytes + q_bytes
    att_us = float(np.mean(att))
    comp_us = float(np.mean(comp))
    achieved = float(np.mean(comp_bytes)) / (comp_us * 1e-6) / 1e9
    att_bytes = float(np.mean(kv_bytes)) + (w.B * w.Hq * (w.W * w.d * 4 + 3 * w.d * 4))
    heads = w.B * w.Hq

    # in-house full-attention kernel (every head misses) on the same cache
    base = None
    if not args.no_baseline_kernel:
        fa, fc = [], []
        dev_all, dev_hit = [], []
        for fl in (mac.MAC_F_DISABLE_REUSE, mac.MAC_F_DISABLE_REUSE | mac.MAC_F_TIMING):
            fb = Bench(w, fl, kc, vc, paged, table)
            for t in range(min(total, 4 + 16)):
                st = fb.step(t, q_dev[t], k_rows[t], v_rows[t])
                if t >= 4:
                    if fl & mac.MAC_F_TIMING:
                        fc.append(st["last_us_complete"])
                    else:
                        fa.append(st["span_us"])
                        if bands is None and t in mac_out:
                            # MAC vs full attention on the same step (information)
                            f = fb.out
                            rel = (mac_out[t] - f).norm(dim=-1) / f.norm(dim=-1)
                            dev_all.append(rel.flatten())
                            dev_hit.append(rel[mac_hit[t]])
            fb.layer.close()
        full_tok = (w.C + total) * w.B * w.Hkv
        deviation = None
        if dev_all:
            da, dh = torch.cat(dev_all), torch.cat(dev_hit)
            deviation = {"what": "||O_mac - O_full|| / ||O_full|| per (request, head), steps 4-19",
                         "mean_all_heads": float(da.mean()),
                         "mean_hit_heads": float(dh.mean()) if dh.numel() else None,
                         "max_hit_heads": float(dh.max()) if dh.numel() else None,
                         "hit_heads": int(dh.numel()), "heads": int(da.numel())}
        full_piped = pipelined_us(w, mac.MAC_F_DISABLE_REUSE, (kc, vc, paged, table), q_dev,
                                  k_rows, v_rows, min(args.warmup, 4), min(args.steps, 16))
        base = {"attention_us": float(np.mean(fa)), "complete_us": float(np.mean(fc)),
                "attention_us_pipelined": full_piped,
                "mac_vs_full_deviation": deviation,
                "hbm_gbps": full_tok * row_bytes / (float(np.mean(fc)) * 1e-6) / 1e9,
                "speedup_vs_full": float(np.mean(fa)) / att_us,
                "speedup_vs_full_pipelined": full_piped / piped}

    # the reuse path's own speedup at this context: the same cache, queries
    # with rho = 0.97 (nearly every head hits its previous step)
    allhit = loops = None
    if (not args.no_baseline_kernel and args.config == "b16_128k" and not args.set and not args.r
            and not args.band_per_head):
        cache = (kc, vc, paged, table)
        row_bytes_ = 2 * w.d * w.kv_elem_bytes

        def reuse_point(rho):
            wa = scaled(w, rho=("const", rho))
            qa = torch.as_tensor(queries(wa, steps=total), device="cuda")
            m = measure(wa, mac_flags, cache, k_rows, v_rows, qa, 4, 16)
            kv = m.pop("kv_tokens") * row_bytes_ / 16
            m["attention_us_pipelined"] = {
                "mac": pipelined_us(wa, mac_flags, cache, qa, k_rows, v_rows, 4, 16),
                "mac_fused_amend": pipelined_us(wa, mac_flags | mac.MAC_F_FUSED_AMEND, cache, qa,
                                                k_rows, v_rows, 4, 16)}
            m.update({"rho": rho, "kv_bytes_per_step": kv,
                      "speedup_vs_full": (base["attention_us"] / m["attention_us"])
                      if base else None,
                      "speedup_vs_full_pipelined": (base["attention_us"] /
                                                    m["attention_us_pipelined"]["mac"])
                      if base else None,
                      "kernels": kernel_rates(wa, m["kernel_us"], kv,
                                              2 if args.ring_bf16 else 4)})
            return wa, qa, m

        wa, qa, allhit = reuse_point(0.97)
        allhit["loop_us_per_step"] = {
            "mac": loop_us(wa, 0, cache, qa, k_rows, v_rows, 4, 16),
            "mac_fused_amend": loop_us(wa, mac.MAC_F_FUSED_AMEND, cache, qa, k_rows, v_rows, 4, 16),
            "mac_sync_amend": loop_us(wa, mac.MAC_F_SYNC_AMEND, cache, qa, k_rows, v_rows, 4, 16)}
        # the mixed workload's decode loop, amend included, for every amend form
        lh = {}
        loops = {"mac": loop_us(w, 0, cache, q_dev, k_rows, v_rows, 4, 16, lh),
                 "mac_fused_amend": loop_us(w, mac.MAC_F_FUSED_AMEND, cache, q_dev, k_rows,
                                            v_rows, 4, 16, lh),
                 "mac_stale_ring": loop_us(w, mac.MAC_F_STALE_RING, cache, q_dev, k_rows,
                                           v_rows, 4, 16, lh),
                 "mac_sync_amend": loop_us(w, mac.MAC_F_SYNC_AMEND, cache, q_dev, k_rows,
                                           v_rows, 4, 16),
                 "full_attention": loop_us(w, mac.MAC_F_DISABLE_REUSE, cache, q_dev, k_rows,
                                           v_rows, 4, 16),
                 "head_hit_rate": {"mac": lh[0], "mac_stale_ring": lh[mac.MAC_F_STALE_RING]}}
        # the stale-by-one ring matches two calls back: at rho = 0.99 the
        # queries of the previous-but-one step are still within tau, so both
        # ring forms hit everywhere and the loops differ by the overlap
        ws, qsd, stale = reuse_point(0.99)
        sh = {}
        stale.update({
            "loop_us_per_step": {
                "mac": loop_us(ws, 0, cache, qsd, k_rows, v_rows, 4, 16, sh),
                "mac_stale_ring": loop_us(ws, mac.MAC_F_STALE_RING, cache, qsd, k_rows, v_rows,
                                          4, 16, sh),
                "mac_fused_amend": loop_us(ws, mac.MAC_F_FUSED_AMEND, cache, qsd, k_rows, v_rows,
                                           4, 16),
                "mac_sync_amend": loop_us(ws, mac.MAC_F_SYNC_AMEND, cache, qsd, k_rows, v_rows,
                                          4, 16)},
            "loop_head_hit_rate": {"mac": sh[0], "mac_stale_ring": sh[mac.MAC_F_STALE_RING]}})
        allhit["rho99_point"] = stale

    point_32k = None
    if not args.no_32k and args.config == "b16_128k" and not args.set and not args.r:
        bench = None
        point_32k = speedup_point("llama32k")

    sub = None
    if (not args.no_workloads and args.config == "b16_128k" and not args.set and not args.r
            and not args.band_per_head):
        bench = kc = vc = table = k_rows = v_rows = q_dev = None
        torch.cuda.empty_cache()
        from workloads import get_config as _gc
        sub = {
            # the CPU-sized workload: all 256 steps from an empty ring
            "cpu4k": workload_record("cpu4k", 0, 256),
            # the MoE shape, band swept; W + 8 warm-up steps
            "moe_122k": workload_record("moe_122k", _gc("moe_122k").W + 8, 16,
                                        bands=(64, 256, 1024)),
            # continuous generation at mid-run context, W + 8 warm-up steps
            "contgen": contgen_run(_gc("contgen").W + 8, 16),
            # small-batch layers back to back, each with its own amend stream
            "multilayer_32k": multilayer_record("llama32k", 8, 16, 32),
        }

    cpu = None
    if host_sample is not None:
        cpu = cpu_baseline(w, host_sample)

    # a measured HBM rate beside the published peak: a plain device copy of
    # 2 GiB (2 GiB read + 2 GiB written)
    n = 1 << 30
    a = torch.empty(n, dtype=torch.int16, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1)
    for _ in range(2 if args.copy_calibration else 1):
        b.copy_(a)
    torch.cuda.synchronize()
    hbm_measured = {}
    for name, fn, nbytes in (("copy_gbps", lambda: b.copy_(a), 4 * n),):
        fn()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(5):
            fn()
        e1.record()
        torch.cuda.synchronize()
        hbm_measured[name] = nbytes * 5 / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del a, b

    line = {
        "metric": "attention-phase µs/decode step + HBM GB/s at 128K ctx, batch 16, GQA 32q/8kv",
        "value": att_us,
        "unit": "us/step",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall * 1e3 / args.steps,
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.kv == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.B, "context": w.C, "q_heads": w.Hq,
                   "kv_heads": w.Hkv, "head_dim": w.d, "kv_layout": w.layout,
                   "ring": w.W, "band": w.r, "tau": w.tau, "rho": list(w.rho),
                   "amend": ("fused" if args.fused_amend else
                             "async, stale-by-one ring" if args.stale_ring else "async"),
                   "ring_queries": "bf16" if args.ring_bf16 else "fp32",
                   "band_per_head": bands},
        "hbm_gbps": float(np.mean(kv_bytes)) / (att_us * 1e-6) / 1e9,
        "tokens_per_s": w.B / (att_us * 1e-6),
        "kv_bytes_per_step": float(np.mean(kv_bytes)),
        "head_hit_rate": float(np.sum(hits)) / (heads * len(hits)),
        "kernel_us": {"match": float(np.mean(match)), "complete": comp_us,
                      "reduce": float(np.mean(red)), "amend": float(np.mean(amend)),
                      "attention_with_kernel_events": float(np.mean(att_ev))},
        "hbm_measured": hbm_measured,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBS, "traffic": measured_traffic(w.name),
                     "kernel": "complete_mfma_kernel" if w.kv == "bf16" else "complete_kernel",
                     "kernel_sha16": kernel_sha16(), "bytes_per_launch": float(np.mean(comp_bytes))},
        "attention_phase_bytes_per_step": att_bytes,
        "full_attention_kernel": base,
        "loop_us_per_step": loops,
        "attention_us_pipelined": piped,
        "allhit_128k": allhit,
        "speedup_32k": point_32k,
        "cpu_baseline": cpu,
        "workloads": sub,
        "setup_s": t_setup,
        "timing_note": ("value: mean over the K timed steps of the decode call's span on the "
                        "decode stream (two stream events), each step launched onto an idle "
                        "GPU (host launch latency included; amend, which the attention phase "
                        "excludes, ends before the next step); attention_us_pipelined: the "
                        "same span with the K steps enqueued back to back (no launch latency, "
                        "any wait for the previous step's amend included); warm-up steps as "
                        "given by --warmup (the AR(1) queries' nearest ring entry is the "
                        "newest, so a few steps fill what matches)"),
        "bad_input": int(st1["bad_input"]),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
