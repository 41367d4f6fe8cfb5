"""Host-side checks of the C-ABI library: it loads, exports every entry point the
header declares, and validates configurations without touching a GPU."""
import ctypes
import os
import re

import pytest

import kv_reuse_amd as mac

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GOLDEN = os.path.join(ROOT, "tests", "golden")


def _declared():
    src = open(os.path.join(ROOT, "include", "mac.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(mac_[a-z_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    lib = mac.load()
    names = _declared()
    assert set(names) == set(mac.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n
        assert ctypes.cast(getattr(lib, n), ctypes.c_void_p).value


def _cfg(**kw):
    base = dict(batch=2, num_q_heads=8, num_kv_heads=2, ring_size=16, band=64, tau=0.3,
                max_seq_len=4096)
    base.update(kw)
    return mac.make_config(**base)


def test_valid_config_passes():
    mac.mac_config_validate(_cfg())
    mac.mac_config_validate(_cfg(layout=mac.MAC_KV_PAGED, kv_dtype=mac.MAC_FP32, ring_size=64,
                                 num_q_heads=32, num_kv_heads=4, tau=-1.0))
    mac.mac_config_validate(_cfg(ring_size=2048))     # the pages' largest window (Table 7)
    mac.mac_config_validate(_cfg(flags=mac.MAC_F_STALE_RING | mac.MAC_F_RING_BF16))
    # per-head bands; with fused amend one band per KV group (4 heads here)
    mac.mac_config_validate(_cfg(band=0, band_per_head=[1, 2, 3, 4, 5, 6, 7, 8]))
    mac.mac_config_validate(_cfg(band_per_head=[9, 9, 9, 9, 2, 2, 2, 2],
                                 flags=mac.MAC_F_FUSED_AMEND))


def test_stale_ring_doubles_only_the_step_buffers():
    """The stale-by-one ring holds a second copy of the per-call buffers the
    amend reads (two query vectors, a position and AS_{1:m} per head); the
    rings themselves are not duplicated."""
    B, Hq = 16, 32
    base = mac.mac_aux_bytes(_cfg(batch=B, num_q_heads=Hq, num_kv_heads=8), 256)
    st = mac.mac_aux_bytes(_cfg(batch=B, num_q_heads=Hq, num_kv_heads=8,
                                flags=mac.MAC_F_STALE_RING), 256)
    per_head = (2 * 128 + 132) * 4
    assert st - base == pytest.approx(B * Hq * per_head + B * 4, abs=3 * 256)


@pytest.mark.parametrize("kw,status", [
    (dict(batch=0), mac.MAC_EINVAL),
    (dict(num_q_heads=6, num_kv_heads=4), mac.MAC_EINVAL),
    (dict(head_dim=64), mac.MAC_EUNSUPPORTED),
    (dict(head_dim=0), mac.MAC_EINVAL),
    (dict(num_q_heads=32, num_kv_heads=2), mac.MAC_EUNSUPPORTED),   # 16 q heads per KV head
    (dict(ring_size=0), mac.MAC_EINVAL),
    (dict(ring_size=2049), mac.MAC_EINVAL),
    (dict(band=0), mac.MAC_EINVAL),
    (dict(tau=float("nan")), mac.MAC_EINVAL),
    (dict(rope_theta=0.0), mac.MAC_EINVAL),
    (dict(sm_scale=-1.0), mac.MAC_EINVAL),
    (dict(layout=7), mac.MAC_EINVAL),
    (dict(kv_dtype=3), mac.MAC_EINVAL),
    (dict(page_size=32), mac.MAC_EUNSUPPORTED),
    (dict(max_seq_len=100), mac.MAC_EINVAL),
    (dict(batch=1024, num_q_heads=8, num_kv_heads=8), mac.MAC_EUNSUPPORTED),
    (dict(flags=1 << 9), mac.MAC_EINVAL),
    (dict(flags=mac.MAC_F_STALE_RING | mac.MAC_F_FUSED_AMEND), mac.MAC_EINVAL),
    (dict(band_per_head=[64, 64, 0, 64, 64, 64, 64, 64]), mac.MAC_EINVAL),
    (dict(band_per_head=[64, 32, 64, 64, 64, 64, 64, 64], flags=mac.MAC_F_FUSED_AMEND),
     mac.MAC_EUNSUPPORTED),
])
def test_invalid_configs_rejected(kw, status):
    with pytest.raises(mac.MacError) as ei:
        mac.mac_config_validate(_cfg(**kw))
    assert ei.value.status == status
    assert mac.mac_last_error()


def test_status_strings():
    assert mac.mac_status_string(mac.MAC_OK) == "MAC_OK"
    assert mac.mac_status_string(mac.MAC_EHIP) == "MAC_EHIP"


def _table7():
    rows = []
    for line in open(os.path.join(GOLDEN, "table7_aux_overhead.txt")):
        line = line.strip()
        if line and not line.startswith("#"):
            k, pct = line.split()
            rows.append((int(k), float(pct)))
    return rows


def test_aux_memory_is_linear_in_window_like_table7():
    """Table 7 of the pages: aux HBM overhead doubles with the search window.
    Our ring memory (the part that depends on W) must scale the same way."""
    rows = _table7()
    ks = [k for k, _ in rows]
    pcts = [p for _, p in rows]
    for (k0, p0), (k1, p1) in zip(rows, rows[1:]):
        assert k1 == 2 * k0
        assert abs(p1 / p0 - 2.0) < 0.1       # printed to one decimal
    base = mac.mac_aux_bytes(_cfg(ring_size=1), 256)
    per_slot = mac.mac_aux_bytes(_cfg(ring_size=2), 256) - base
    assert per_slot > 0
    for w in (4, 8, 16, 32, 64):
        assert mac.mac_aux_bytes(_cfg(ring_size=w), 256) == pytest.approx(base + (w - 1) * per_slot,
                                                                           rel=1e-3)
    assert ks == [256, 512, 1024, 2048] and pcts[0] == 1.2


def test_aux_bytes_rejects_bad_config():
    assert mac.mac_aux_bytes(_cfg(batch=0), 256) == 0


def test_init_rejects_bad_config_before_any_device_work():
    with pytest.raises(mac.MacError) as ei:
        mac.mac_init(_cfg(band=0))
    assert ei.value.status == mac.MAC_EINVAL


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU's share: --gpus N > 1 exits with status 2 and
    a message, before any import of the library or the GPU runtime."""
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "--gpus 2 is not supported" in r.stderr
    assert r.stdout == ""
