"""HIP-graph replay of the decode step (fused amend, and amend on the decode
stream): the ring slot comes from the device's call counter, so a captured
append + decode, replayed with its input buffers updated in place, gives
the same bits as the same steps run eagerly on a second handle.  Every
replay is checked, with eager work and synchronisations between replays."""
import numpy as np
import pytest
import torch

from workloads import get_config, kv_logical, page_table, queries, scaled, to_paged

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("form", ["fused", "sync"])
def test_graph_replay_equals_eager(gpu_lib, form):
    import kv_reuse_amd as mac
    flags = mac.MAC_F_FUSED_AMEND if form == "fused" else mac.MAC_F_SYNC_AMEND
    w = scaled(get_config("b16_128k"), B=2, C=600, steps=16, r=64, rho=("const", 0.97))
    warm, total = 2, 12
    print("graph case", form, "B", w.B, "C", w.C, "steps", total, flush=True)
    K, V = kv_logical(w, "cuda")
    idx = torch.arange(w.C, w.C + total, device="cuda")
    k_rows = K[:, :, idx].permute(2, 0, 1, 3).contiguous()
    v_rows = V[:, :, idx].permute(2, 0, 1, 3).contiguous()
    q = torch.as_tensor(queries(w, steps=total), device="cuda")
    tab = page_table(w)
    table = torch.as_tensor(tab, device="cuda")

    def make():
        kc, vc = to_paged(K, tab), to_paged(V, tab)
        seq = torch.zeros(w.B, dtype=torch.int32, device="cuda")
        cfg = mac.make_config(batch=w.B, num_q_heads=w.Hq, num_kv_heads=w.Hkv, ring_size=w.W,
                              band=w.r, tau=w.tau, rope_theta=w.theta, layout=mac.MAC_KV_PAGED,
                              kv_dtype=mac.MAC_BF16, max_seq_len=w.n_cap, flags=flags)
        layer = mac.MacLayer(cfg)
        view = mac.make_kv_view(kc, vc, seq, table, num_pages=kc.shape[0])
        return layer, view, seq, (kc, vc)

    eager, view_e, seq_e, keep_e = make()
    graphed, view_g, seq_g, keep_g = make()
    pos_e = torch.zeros(w.B, dtype=torch.int32, device="cuda")
    out_e = torch.empty((w.B, w.Hq, w.d), dtype=torch.float32, device="cuda")
    # the graphed handle's static inputs
    pos_g = torch.zeros(w.B, dtype=torch.int32, device="cuda")
    k_g, v_g, q_g = k_rows[0].clone(), v_rows[0].clone(), q[0].clone()
    out_g = torch.empty_like(out_e)

    def fill(t):
        pos_g.fill_(w.C + t)
        seq_g.fill_(w.C + t + 1)
        k_g.copy_(k_rows[t])
        v_g.copy_(v_rows[t])
        q_g.copy_(q[t])

    def step_g(stream):
        graphed.append_kv(view_g, k_g, v_g, pos_g, stream)
        graphed.decode_step(view_g, q_g, out_g, None, stream)

    def step_e(t):
        pos_e.fill_(w.C + t)
        seq_e.fill_(w.C + t + 1)
        eager.append_kv(view_e, k_rows[t], v_rows[t], pos_e)
        eager.decode_step(view_e, q[t], out_e)
        torch.cuda.synchronize()

    try:
        s = torch.cuda.Stream()
        for t in range(warm):                    # warm-up, eager, on the capture stream
            step_e(t)
            fill(t)
            torch.cuda.synchronize()
            with torch.cuda.stream(s):
                step_g(s)
            torch.cuda.synchronize()
            assert torch.equal(out_g, out_e), ("warm-up", t)
        g = torch.cuda.CUDAGraph()
        fill(warm)
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            step_g(s)                            # recorded, not run
        torch.cuda.synchronize()
        for t in range(warm, total):
            step_e(t)
            fill(t)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(out_g, out_e), ("replay", t)
        st_e, st_g = eager.stats(), graphed.stats()
        print("  steps", st_g["steps"], "hits eager", st_e["hits"], "graph", st_g["hits"], flush=True)
        assert st_g["steps"] == st_e["steps"] == total
        assert st_g["hits"] == st_e["hits"] and st_g["misses"] == st_e["misses"]
        assert st_e["hits"] > 0
    finally:
        eager.close()
        graphed.close()


@pytest.mark.parametrize("form", ["async", "stale", "timing"])
def test_capture_of_per_call_forms_is_rejected(gpu_lib, form):
    """The forms whose calls choose events or buffers on the host refuse a
    stream being captured with MAC_EUNSUPPORTED, enqueue nothing and stay
    usable: the steps after the refused call are bit-equal to a twin handle
    that never saw it.  The async form's amend thread then waits while
    another stream is being captured (global mode) and must not fail."""
    import kv_reuse_amd as mac
    flags = {"async": 0, "stale": mac.MAC_F_STALE_RING, "timing": mac.MAC_F_TIMING}[form]
    w = scaled(get_config("b16_128k"), B=2, C=600, steps=12, r=64, rho=("const", 0.97))
    total = 8
    print("capture refusal case", form, "B", w.B, "C", w.C, "steps", total, flush=True)
    K, V = kv_logical(w, "cuda")
    idx = torch.arange(w.C, w.C + total, device="cuda")
    k_rows = K[:, :, idx].permute(2, 0, 1, 3).contiguous()
    v_rows = V[:, :, idx].permute(2, 0, 1, 3).contiguous()
    q = torch.as_tensor(queries(w, steps=total), device="cuda")
    tab = page_table(w)
    table = torch.as_tensor(tab, device="cuda")

    def make():
        kc, vc = to_paged(K, tab), to_paged(V, tab)
        seq = torch.zeros(w.B, dtype=torch.int32, device="cuda")
        pos = torch.zeros(w.B, dtype=torch.int32, device="cuda")
        cfg = mac.make_config(batch=w.B, num_q_heads=w.Hq, num_kv_heads=w.Hkv, ring_size=w.W,
                              band=w.r, tau=w.tau, rope_theta=w.theta, layout=mac.MAC_KV_PAGED,
                              kv_dtype=mac.MAC_BF16, max_seq_len=w.n_cap, flags=flags)
        layer = mac.MacLayer(cfg)
        view = mac.make_kv_view(kc, vc, seq, table, num_pages=kc.shape[0])
        out = torch.empty((w.B, w.Hq, w.d), dtype=torch.float32, device="cuda")
        return layer, view, seq, pos, out, (kc, vc)

    a, b = make(), make()
    s = torch.cuda.Stream()
    other = torch.cuda.Stream()
    x = torch.ones(1 << 20, device="cuda")

    def step(h, t, stream=None):
        layer, view, seq, pos, out, _ = h
        with torch.cuda.stream(stream or torch.cuda.current_stream()):
            pos.fill_(w.C + t)
            seq.fill_(w.C + t + 1)
            layer.append_kv(view, k_rows[t], v_rows[t], pos, stream)
            layer.decode_step(view, q[t], out, None, stream)

    try:
        refused = 0
        for t in range(total):
            torch.cuda.synchronize()
            step(b, t)
            step(a, t, s)
            if form == "async":
                # a capture on another stream while a's amend thread waits
                g2 = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g2, stream=other):
                    x.mul_(1.0)
            if t == 2:
                g = torch.cuda.CUDAGraph()
                layer, view, seq, pos, out, _ = a
                with torch.cuda.graph(g, stream=s):
                    with pytest.raises(mac.MacError) as err:
                        layer.decode_step(view, q[t], out, None, s)
                    refused += 1
                assert err.value.status == mac.MAC_EUNSUPPORTED, err.value
            torch.cuda.synchronize()
            assert torch.equal(a[4], b[4]), ("step", t)
        st_a, st_b = a[0].stats(), b[0].stats()
        print("  steps", st_a["steps"], "hits", st_a["hits"], "refused", refused, flush=True)
        assert refused == 1
        assert st_a["steps"] == st_b["steps"] == total
        assert st_a["hits"] == st_b["hits"] > 0
    finally:
        a[0].close()
        b[0].close()
