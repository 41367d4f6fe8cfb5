"""Lockstep runner: the HIP library (through the C ABI) beside the fp64 oracle.

Per decode step the oracle decides first; heads whose relative distance lies
within 1e-4 of tau, or whose two nearest ring entries are within a relative
1e-5, are forced to the oracle's decision through the override array (both
decisions are correct there).  The GPU then runs and must reproduce every
decision bit for bit and every output within max-abs 2e-3 and per-row
relative 1e-2.  Cache rows that have not been appended yet hold NaN (per
request, for ragged prefill lengths), so a kernel that reads past a request's
query position fails loudly.
"""
import numpy as np
import torch

import kv_reuse_amd as mac
import oracle
from workloads import bf16_bits, kv_logical, page_table, queries, to_paged

MAX_ABS = 2e-3
ROW_REL = 1e-2


def _kv_nan(dtype):
    return torch.tensor(float("nan"), dtype=dtype)


class Lockstep:
    def __init__(self, w, flags=0, track=None, device="cuda", oracle_flags=0, tau=None, r=None,
                 W=None, sync_amend=False, layer=0, amend_stream=None, prefill=None,
                 bands=None):
        self.w = w
        # per-request prefill length (ragged batches); request b decodes
        # position prefill[b] + t at step t
        self.prefill = (np.full(w.B, w.C, np.int32) if prefill is None
                        else np.asarray(prefill, np.int32))
        assert self.prefill.shape == (w.B,) and self.prefill.max() <= w.C
        self.tau = w.tau if tau is None else tau
        self.r = w.r if r is None else r
        # per-head bands: the config's band_per_head and the oracle's r_h
        self.bands = None if bands is None else [int(x) for x in bands]
        self.W = w.W if W is None else W
        self.dev = device
        B, Hkv, d = w.B, w.Hkv, w.d
        K, V = kv_logical(w, device, layer=layer)
        self.K, self.V = K, V
        self.paged = w.layout == "paged"
        # oracle views: logical rows per (request, KV head); only tracked groups copied
        if track is None:
            groups = [(b, g) for b in range(B) for g in range(Hkv)]
        else:
            tr = np.asarray(track).reshape(B, w.Hq)
            groups = sorted({(b, h // w.G) for b in range(B) for h in range(w.Hq) if tr[b, h]})
        self.track = None if track is None else np.asarray(track, np.uint8).reshape(B, w.Hq)
        self.Kg = [None] * (B * Hkv)
        self.Vg = [None] * (B * Hkv)
        for b, g in groups:
            self.Kg[b * Hkv + g] = bf16_bits(K[b, g])
            self.Vg[b * Hkv + g] = bf16_bits(V[b, g])
        # device cache: prefill rows present, the rest NaN until appended
        logical_k = K.clone()
        logical_v = V.clone()
        for b in range(B):
            logical_k[b, :, int(self.prefill[b]):] = _kv_nan(K.dtype)
            logical_v[b, :, int(self.prefill[b]):] = _kv_nan(V.dtype)
        if self.paged:
            self.table_np = page_table(w)
            self.kc = to_paged(logical_k, self.table_np)
            self.vc = to_paged(logical_v, self.table_np)
            self.table = torch.as_tensor(self.table_np, device=device)
            del logical_k, logical_v
        else:
            self.table_np = None
            self.kc, self.vc = logical_k, logical_v
            self.table = None
        self.q = queries(w, layer=layer)
        self.seq = torch.zeros(B, dtype=torch.int32, device=device)
        self.pos = torch.zeros(B, dtype=torch.int32, device=device)
        fl = flags | mac.MAC_F_RECORD_DEBUG | (mac.MAC_F_SYNC_AMEND if sync_amend else 0)
        self.cfg = mac.make_config(
            batch=B, num_q_heads=w.Hq, num_kv_heads=Hkv, head_dim=d, ring_size=self.W,
            band=self.r, tau=self.tau, rope_theta=w.theta,
            layout=mac.MAC_KV_PAGED if self.paged else mac.MAC_KV_CONTIGUOUS,
            kv_dtype=mac.MAC_FP32 if w.kv == "fp32" else mac.MAC_BF16,
            max_seq_len=w.n_cap, flags=fl, band_per_head=self.bands)
        self.layer = mac.MacLayer(self.cfg, amend_stream=amend_stream)
        self.view = mac.make_kv_view(self.kc, self.vc, self.seq, self.table,
                                     num_pages=self.kc.shape[0] if self.paged else 0)
        self.orc = oracle.Oracle(B, w.Hq, Hkv, d, self.W,
                                 self.r if self.bands is None else self.bands, self.tau, w.theta,
                                 kv_fp32=(w.kv == "fp32"), flags=oracle_flags)
        self.out = torch.empty((B, w.Hq, d), dtype=torch.float32, device=device)
        self.stats = []

    def step(self, t, seq_lens=None, override=None, compare=True, q=None):
        return self.finish(self.launch(t, seq_lens, override, q), compare)

    def launch(self, t, seq_lens=None, override=None, q=None):
        """Append, run the oracle, enqueue the GPU decode step (no synchronisation)."""
        w = self.w
        B = w.B
        seq_h = (self.prefill + t + 1).astype(np.int32) if seq_lens is None else np.asarray(
            seq_lens, np.int32)
        q_h = self.q[t] if q is None else q
        # KV manager: row prefill[b]+t of the workload enters request b's cache
        # at step t, whether or not the request decodes this step
        pos_h = (self.prefill + t).astype(np.int32)
        self.pos.copy_(torch.as_tensor(pos_h))
        m_idx = torch.as_tensor(pos_h, device=self.dev, dtype=torch.long)
        bi = torch.arange(B, device=self.dev)
        k_new = self.K[bi, :, m_idx].contiguous()
        v_new = self.V[bi, :, m_idx].contiguous()
        self.layer.append_kv(self.view, k_new, v_new, self.pos)
        self.seq.copy_(torch.as_tensor(seq_h))
        res = self.orc.step(self.Kg, self.Vg, seq_h, q_h, override=override, track=self.track)
        forced = np.full((B, w.Hq), -2, np.int32) if override is None else override.copy()
        flag = (res["near_tau"] | res["near_tie"]).astype(bool) & (forced == -2)
        forced[flag] = np.where(res["hit"][flag] != 0, res["p"][flag], -1)
        ov = torch.as_tensor(forced, device=self.dev)
        qd = torch.as_tensor(q_h, device=self.dev)
        self.layer.decode_step(self.view, qd, self.out, ov)
        # keep the step's device inputs alive until it has run
        return {"t": t, "res": res, "flag": flag, "keep": (k_new, v_new, ov, qd)}

    def finish(self, pending, compare=True):
        """Synchronise and compare the step launched by launch()."""
        torch.cuda.synchronize()
        res, t = pending["res"], pending["t"]
        p_g, hit_g, rel_g = self.layer.debug_last()
        out_g = self.out.cpu().numpy().astype(np.float64)
        info = {"t": t, "forced": int(pending["flag"].sum()), "hits": int(res["hit"].sum()),
                "p_gpu": p_g, "hit_gpu": hit_g, "res": res, "out_gpu": out_g}
        if compare:
            self.check(res, p_g, hit_g, out_g, t)
        return info

    def check(self, res, p_g, hit_g, out_g, t):
        assert np.array_equal(hit_g, res["hit"]), ("decision mismatch", t,
                                                   np.argwhere(hit_g != res["hit"]))
        assert np.array_equal(p_g, res["p"]), ("position mismatch", t,
                                               np.argwhere(p_g != res["p"]))
        mask = np.ones(p_g.shape, bool) if self.track is None else self.track.astype(bool)
        o = res["out"][mask]
        g = out_g[mask]
        err = np.abs(g - o)
        assert np.all(np.isfinite(g)), ("non-finite output", t)
        assert err.max() <= MAX_ABS, ("max-abs", t, float(err.max()))
        rel = np.linalg.norm(g - o, axis=-1) / np.maximum(np.linalg.norm(o, axis=-1), 1e-30)
        assert rel.max() <= ROW_REL, ("row-rel", t, float(rel.max()))
        self.stats.append((float(err.max()), float(rel.max())))

    def close(self):
        self.layer.close()
