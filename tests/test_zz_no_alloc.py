"""mac_prefill_noalloc (the allocation-free form of mac_prefill, its scratch in
a static device array) against mac_prefill, through the C ABI: two calls in a
row, the second smaller than the first, so the second runs on scratch the
first left behind.  Matched positions bit-exact, outputs within max-abs 2e-3
and per-row relative 1e-2 of mac_prefill's; a call whose scratch would exceed
the array is refused before any GPU work."""
import numpy as np
import pytest
import torch

from gpu_harness import MAX_ABS, ROW_REL
from workloads import get_config, kv_logical, page_table, queries, scaled, to_paged

pytestmark = pytest.mark.gpu


def test_prefill_noalloc_matches_prefill(gpu_lib):
    import kv_reuse_amd as mac
    w = scaled(get_config("b16_128k"), B=2, C=0, steps=300,
               rho=("per_request_uniform", 0.95, 0.995))
    K, V = kv_logical(w, "cuda")
    tab = page_table(w)
    kc, vc, table = to_paged(K, tab), to_paged(V, tab), torch.as_tensor(tab, device="cuda")
    cfg = mac.make_config(batch=w.B, num_q_heads=w.Hq, num_kv_heads=w.Hkv, ring_size=w.W,
                          band=w.r, tau=w.tau, rope_theta=w.theta, layout=mac.MAC_KV_PAGED,
                          kv_dtype=mac.MAC_BF16, max_seq_len=w.n_cap)
    layer = mac.MacLayer(cfg)
    q_all = queries(w, steps=w.steps)                        # [N][B][Hq][d]
    try:
        for N, lens in ((300, [300, 300]), (120, [120, 77])):
            print("call N", N, "lens", lens, flush=True)
            seq = torch.tensor(lens, dtype=torch.int32, device="cuda")
            view = mac.make_kv_view(kc, vc, seq, table, num_pages=kc.shape[0])
            qd = torch.as_tensor(np.ascontiguousarray(q_all[:N].transpose(1, 0, 2, 3)),
                                 device="cuda")
            res = {}
            for label in ("prefill", "noalloc"):
                out = torch.full((w.B, N, w.Hq, w.d), float("nan"), device="cuda")
                pout = torch.full((w.B, N, w.Hq), -7, dtype=torch.int32, device="cuda")
                if label == "prefill":
                    layer.prefill(view, N, qd, out, None, pout)
                else:
                    layer.prefill_noalloc(view, N, qd, out, None, pout)
                torch.cuda.synchronize()
                res[label] = (out.cpu().numpy().astype(np.float64), pout.cpu().numpy())
            (oa, pa), (ob, pb) = res["prefill"], res["noalloc"]
            assert np.array_equal(pa, pb), np.argwhere(pa != pb)[:8]
            assert (pa >= 0).sum() > 0
            live = np.arange(N)[None, :] < np.asarray(lens)[:, None]
            assert not ob[~live].any(), "rows past a prompt must be zero"
            g, o = ob[live], oa[live]
            assert np.all(np.isfinite(g))
            err = np.abs(g - o)
            rel = np.linalg.norm(g - o, axis=-1) / np.maximum(np.linalg.norm(o, axis=-1), 1e-30)
            print("  hits", int((pa >= 0).sum()), "max-abs %.2e row-rel %.2e bit-identical %s"
                  % (err.max(), rel.max(), bool(np.array_equal(g, o))), flush=True)
            assert err.max() <= MAX_ABS and rel.max() <= ROW_REL
        # over the static array: refused on the host, before any GPU work
        N = 4096
        seq = torch.tensor([N, N], dtype=torch.int32, device="cuda")
        view = mac.make_kv_view(kc, vc, seq, table, num_pages=kc.shape[0])
        qd = torch.zeros((w.B, N, w.Hq, w.d), device="cuda")
        out = torch.zeros_like(qd)
        with pytest.raises(mac.MacError) as ei:
            layer.prefill_noalloc(view, N, qd, out)
        assert ei.value.status == mac.MAC_EINVAL
        assert "static array" in mac.mac_last_error(layer.h)
    finally:
        torch.cuda.synchronize()
        layer.close()
