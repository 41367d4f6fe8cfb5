"""ctypes binding of include/mac.h: the same entry points, argument marshalling only.

Every step of the decode path runs in the HIP library kv_reuse_amd/libmac.so;
this module only converts Python/torch arguments to the C ABI and raises
MacError on a non-OK status.  There is no fallback: without the built library
every call raises.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmac.so")

MAC_OK, MAC_EINVAL, MAC_ENOMEM, MAC_EHIP, MAC_ESTATE, MAC_EUNSUPPORTED = range(6)
MAC_KV_CONTIGUOUS, MAC_KV_PAGED = 0, 1
MAC_BF16, MAC_FP32 = 0, 1
MAC_F_DISABLE_REUSE, MAC_F_SYNC_AMEND, MAC_F_TIMING, MAC_F_RECORD_DEBUG = 1, 2, 4, 8
MAC_F_FUSED_AMEND = 16
MAC_F_RING_BF16 = 32
MAC_F_STALE_RING = 64
MAC_F_UNBALANCED_PLAN = 128

EXPORTS = ["mac_config_validate", "mac_aux_bytes", "mac_init", "mac_destroy", "mac_reset",
           "mac_append_kv", "mac_decode_step", "mac_stats", "mac_debug_last", "mac_last_error",
           "mac_status_string", "mac_prefill", "mac_prefill_noalloc"]


class MacError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__("%s: %s" % (_STATUS.get(status, status), msg))
        self.status = status


_STATUS = {0: "MAC_OK", 1: "MAC_EINVAL", 2: "MAC_ENOMEM", 3: "MAC_EHIP", 4: "MAC_ESTATE",
           5: "MAC_EUNSUPPORTED"}


class MacConfig(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("ring_size", ctypes.c_int32), ("band", ctypes.c_int32),
                ("tau", ctypes.c_float), ("rope_theta", ctypes.c_float),
                ("sm_scale", ctypes.c_float), ("layout", ctypes.c_int32),
                ("kv_dtype", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("max_seq_len", ctypes.c_int32), ("flags", ctypes.c_uint32),
                ("band_per_head", ctypes.c_void_p)]


class MacKvView(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("page_table", ctypes.c_void_p), ("max_pages_per_req", ctypes.c_int32),
                ("num_pages", ctypes.c_int32), ("seq_lens", ctypes.c_void_p)]


class MacStats(ctypes.Structure):
    _fields_ = [(n, ctypes.c_uint64) for n in
                ("steps", "decisions", "hits", "misses", "near_tau", "override_invalid",
                 "kv_tokens_critical", "kv_tokens_amend", "kv_bytes_critical",
                 "kv_bytes_amend", "aux_bytes", "bad_input")] + \
               [(n, ctypes.c_float) for n in
                ("last_us_match", "last_us_complete", "last_us_reduce", "last_us_amend",
                 "last_us_attention")] + \
               [(n, ctypes.c_uint64) for n in
                ("prefill_tokens", "prefill_decisions", "prefill_hits", "prefill_kv_tokens",
                 "prefill_override_invalid", "complete_waves")]


_lib = None


def load():
    """Load libmac.so; raises when it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("HIP library %s is not built (python -m kv_reuse_amd.build)" % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, st = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int
    lib.mac_config_validate.argtypes = [ctypes.POINTER(MacConfig)]
    lib.mac_config_validate.restype = st
    lib.mac_aux_bytes.argtypes = [ctypes.POINTER(MacConfig), i32]
    lib.mac_aux_bytes.restype = ctypes.c_size_t
    lib.mac_init.argtypes = [ctypes.POINTER(MacConfig), vp, vp, ctypes.POINTER(vp)]
    lib.mac_init.restype = st
    lib.mac_destroy.argtypes = [vp]
    lib.mac_destroy.restype = st
    lib.mac_reset.argtypes = [vp]
    lib.mac_reset.restype = st
    lib.mac_append_kv.argtypes = [vp, ctypes.POINTER(MacKvView), vp, vp, vp, vp]
    lib.mac_append_kv.restype = st
    lib.mac_decode_step.argtypes = [vp, ctypes.POINTER(MacKvView), vp, vp, vp, vp]
    lib.mac_decode_step.restype = st
    lib.mac_stats.argtypes = [vp, ctypes.POINTER(MacStats)]
    lib.mac_stats.restype = st
    lib.mac_prefill.argtypes = [vp, ctypes.POINTER(MacKvView), i32, vp, vp, vp, vp, vp]
    lib.mac_prefill.restype = st
    lib.mac_prefill_noalloc.argtypes = [vp, ctypes.POINTER(MacKvView), i32, vp, vp, vp, vp, vp]
    lib.mac_prefill_noalloc.restype = st
    lib.mac_debug_last.argtypes = [vp, vp, vp, vp]
    lib.mac_debug_last.restype = st
    lib.mac_last_error.argtypes = [vp]
    lib.mac_last_error.restype = ctypes.c_char_p
    lib.mac_status_string.argtypes = [st]
    lib.mac_status_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _check(status, handle=None):
    if status != MAC_OK:
        msg = load().mac_last_error(handle)
        raise MacError(status, msg.decode() if msg else "")


def _ptr(t):
    """Device (or host) address of a torch tensor / numpy array / int / None."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if isinstance(t, np.ndarray):
        return t.ctypes.data
    return t.data_ptr()


def _stream(s):
    if s is None:
        return None
    if isinstance(s, int):
        return s
    return s.cuda_stream


def make_config(batch, num_q_heads, num_kv_heads, head_dim=128, ring_size=32, band=256, tau=0.3,
                rope_theta=500000.0, sm_scale=0.0, layout=MAC_KV_CONTIGUOUS, kv_dtype=MAC_BF16,
                page_size=16, max_seq_len=0, flags=0, band_per_head=None):
    """band_per_head: None or a sequence of num_q_heads per-head bands (the
    config keeps the int32 array alive; the library copies it at init)."""
    cfg = MacConfig(batch, num_q_heads, num_kv_heads, head_dim, ring_size, band, tau, rope_theta,
                    sm_scale, layout, kv_dtype, page_size, max_seq_len, flags, None)
    if band_per_head is not None:
        arr = (ctypes.c_int32 * num_q_heads)(*[int(x) for x in band_per_head])
        if len(band_per_head) != num_q_heads:
            raise ValueError("band_per_head needs num_q_heads entries")
        cfg._bands = arr
        cfg.band_per_head = ctypes.cast(arr, ctypes.c_void_p)
    return cfg


def make_kv_view(k, v, seq_lens, page_table=None, num_pages=0):
    """View of a layer's cache.  The tensors must outlive every call that uses it."""
    if page_table is None:
        return MacKvView(_ptr(k), _ptr(v), None, 0, 0, _ptr(seq_lens))
    return MacKvView(_ptr(k), _ptr(v), _ptr(page_table), int(page_table.shape[-1]),
                     int(num_pages or k.shape[0]), _ptr(seq_lens))


def mac_config_validate(cfg):
    _check(load().mac_config_validate(ctypes.byref(cfg)))


def mac_aux_bytes(cfg, num_cu):
    return int(load().mac_aux_bytes(ctypes.byref(cfg), int(num_cu)))


def mac_init(cfg, main_stream=None, amend_stream=None):
    h = ctypes.c_void_p()
    _check(load().mac_init(ctypes.byref(cfg), _stream(main_stream), _stream(amend_stream),
                           ctypes.byref(h)))
    return h


def mac_destroy(h):
    _check(load().mac_destroy(h), h)


def mac_reset(h):
    _check(load().mac_reset(h), h)


def mac_append_kv(h, kv, k_new, v_new, positions, stream=None):
    _check(load().mac_append_kv(h, ctypes.byref(kv), _ptr(k_new), _ptr(v_new), _ptr(positions),
                                _stream(stream)), h)


def mac_decode_step(h, kv, q_pre_rope, out, override_pos=None, stream=None):
    _check(load().mac_decode_step(h, ctypes.byref(kv), _ptr(q_pre_rope), _ptr(out),
                                  _ptr(override_pos), _stream(stream)), h)


def mac_prefill(h, kv, num_tokens, q_pre, out, override_pos=None, p_out=None, stream=None):
    _check(load().mac_prefill(h, ctypes.byref(kv), int(num_tokens), _ptr(q_pre), _ptr(out),
                              _ptr(override_pos), _ptr(p_out), _stream(stream)), h)


def mac_prefill_noalloc(h, kv, num_tokens, q_pre, out, override_pos=None, p_out=None,
                        stream=None):
    _check(load().mac_prefill_noalloc(h, ctypes.byref(kv), int(num_tokens), _ptr(q_pre),
                                      _ptr(out), _ptr(override_pos), _ptr(p_out),
                                      _stream(stream)), h)


def mac_stats(h):
    s = MacStats()
    _check(load().mac_stats(h, ctypes.byref(s)), h)
    return {name: getattr(s, name) for name, _ in MacStats._fields_}


def mac_debug_last(h, batch, num_q_heads):
    n = batch * num_q_heads
    p = np.empty(n, np.int32)
    hit = np.empty(n, np.uint8)
    rel = np.empty(n, np.float32)
    _check(load().mac_debug_last(h, p.ctypes.data, hit.ctypes.data, rel.ctypes.data), h)
    return p.reshape(batch, num_q_heads), hit.reshape(batch, num_q_heads), \
        rel.reshape(batch, num_q_heads)


def mac_last_error(h=None):
    m = load().mac_last_error(h)
    return m.decode() if m else ""


def mac_status_string(status):
    return load().mac_status_string(int(status)).decode()
