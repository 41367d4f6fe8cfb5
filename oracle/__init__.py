"""fp64 CPU oracle of the MAC-Attention decode step -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It shares no code with the HIP library
in ``kv_reuse_amd/``; the C source is ``oracle/mac_oracle.c`` and this module is
argument marshalling over ctypes.

What each function follows (MAC-Attention, arXiv 2604.00235, paper card):
  rope ........ pre-/post-RoPE queries (abstract; Figure 2), RoFormer rotate-half
  attend ...... the attention summary AS over a key range (Figure 2)
  merge ....... log-domain merge (+) (Figure 2 (b))
  remove ...... log-domain removal (-) (Figure 2 (c))
  nearest ..... pre-RoPE L2 nearest neighbour over the ring (Figure 2 (a))
  round_bf16 .. ring queries kept in bfloat16 (F_RING_BF16; Table 7's memory)
  F_STALE_RING  asynchronous cache update read as one call of staleness
                (Figure 2 (c)): call t matches entries of calls <= t-2
  Oracle.step . match -> complete -> amend, one decode call (Figure 2, Figure 3 (c))

Parity pins live in tests/test_oracle_pins.py; every function here has one.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libmac_oracle.so")
_lib = None

F_DISABLE_REUSE = 1
F_RING_BF16 = 2          # the ring keeps pre-RoPE queries rounded to bfloat16
F_STALE_RING = 4         # call t matches only entries inserted up to call t-2

_dp = ctypes.POINTER(ctypes.c_double)
_fp = ctypes.POINTER(ctypes.c_float)
_i32p = ctypes.POINTER(ctypes.c_int32)
_i64p = ctypes.POINTER(ctypes.c_int64)
_u8p = ctypes.POINTER(ctypes.c_uint8)
_vp = ctypes.c_void_p


def _use_library(path):
    """Load the oracle from another build of mac_oracle.c (the mutation tests
    build copies with a planted mistake); None returns to the default build.
    Oracle objects created before the switch keep the library they had."""
    global _lib
    _lib = None
    return _load(path)


def _load(path=None):
    global _lib
    if _lib is not None:
        return _lib
    if path is None:
        path = _LIB_PATH
        if not os.path.exists(path):
            from . import build as _b
            _b.build()
    lib = ctypes.CDLL(path)
    lib.orc_rope.argtypes = [_fp, ctypes.c_int, ctypes.c_int64, ctypes.c_double, _dp]
    lib.orc_empty.argtypes = [ctypes.c_int, _dp]
    lib.orc_attend.argtypes = [_dp, _vp, _vp, ctypes.c_int, ctypes.c_int, ctypes.c_int64,
                               ctypes.c_int64, ctypes.c_double, _dp]
    lib.orc_merge.argtypes = [_dp, _dp, ctypes.c_int, _dp]
    lib.orc_remove.argtypes = [_dp, _dp, ctypes.c_int, _dp]
    lib.orc_nearest.argtypes = [_fp, _fp, _i32p, ctypes.c_int, ctypes.c_int, ctypes.c_int64,
                                _dp, _dp]
    lib.orc_nearest.restype = ctypes.c_int
    lib.orc_round_bf16.argtypes = [ctypes.c_float]
    lib.orc_round_bf16.restype = ctypes.c_float
    lib.orc_create.argtypes = [ctypes.c_int] * 6 + [ctypes.c_double] * 3 + [ctypes.c_int,
                                                                          ctypes.c_uint]
    lib.orc_create.restype = _vp
    lib.orc_destroy.argtypes = [_vp]
    lib.orc_reset.argtypes = [_vp]
    lib.orc_set_bands.argtypes = [_vp, _i32p]
    lib.orc_ring_entry.argtypes = [_vp, ctypes.c_int, ctypes.c_int, ctypes.c_int, _i32p, _fp, _dp]
    lib.orc_step.argtypes = [_vp, ctypes.POINTER(_vp), ctypes.POINTER(_vp), _i32p, _fp, _i32p,
                             _u8p, _dp, _dp, _u8p, _i32p, _dp, _u8p, _u8p, _i32p, _i64p]
    lib.orc_step.restype = ctypes.c_int
    lib.orc_set_threads.argtypes = [ctypes.c_int]
    lib.orc_set_threads.restype = ctypes.c_int
    _lib = lib
    return lib


def _ptr(a, t):
    return None if a is None else a.ctypes.data_as(t)


def _kv(a):
    """Return (array, kv_fp32) for a key/value block given as float32 or bf16 bits (uint16)."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.float32:
        return a, 1
    if a.dtype == np.uint16:
        return a, 0
    raise TypeError("key/value rows must be float32 or bf16 bits (uint16), got %s" % a.dtype)


def set_threads(n):
    """OpenMP threads of Oracle.step (timing only); returns the previous count."""
    return int(_load().orc_set_threads(int(n)))


def rope(x, m, theta):
    """Rotate-half RoPE of one fp32 vector at position m, angles in fp64."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape[0], np.float64)
    _load().orc_rope(_ptr(x, _fp), x.shape[0], int(m), float(theta), _ptr(out, _dp))
    return out


def empty(d):
    s = np.empty(d + 2, np.float64)
    _load().orc_empty(d, _ptr(s, _dp))
    return s


def attend(q, k, v, a, b, scale):
    """A(q, [a, b]) over rows of k/v ([n][d], float32 or bf16 bits) -> (o, M, l) as [d+2]."""
    q = np.ascontiguousarray(q, dtype=np.float64)
    k, fk = _kv(k)
    v, fv = _kv(v)
    assert fk == fv and k.shape == v.shape and k.shape[1] == q.shape[0]
    b = min(int(b), k.shape[0] - 1)
    out = np.empty(q.shape[0] + 2, np.float64)
    _load().orc_attend(_ptr(q, _dp), k.ctypes.data, v.ctypes.data, fk, q.shape[0], int(a), b,
                       float(scale), _ptr(out, _dp))
    return out


def merge(x, y):
    x = np.ascontiguousarray(x, dtype=np.float64)
    y = np.ascontiguousarray(y, dtype=np.float64)
    z = np.empty_like(x)
    _load().orc_merge(_ptr(x, _dp), _ptr(y, _dp), x.shape[0] - 2, _ptr(z, _dp))
    return z


def remove(z, y):
    z = np.ascontiguousarray(z, dtype=np.float64)
    y = np.ascontiguousarray(y, dtype=np.float64)
    x = np.empty_like(z)
    _load().orc_remove(_ptr(z, _dp), _ptr(y, _dp), z.shape[0] - 2, _ptr(x, _dp))
    return x


def round_bf16(x):
    """x (float32 array) rounded to the nearest bfloat16, ties to even, as float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    f = _load().orc_round_bf16
    return np.array([f(float(v)) for v in x.reshape(-1)], np.float32).reshape(x.shape)


def nearest(qt, ring_q, ring_pos, m):
    """(slot, best distance, second-best distance) over the valid ring entries."""
    qt = np.ascontiguousarray(qt, dtype=np.float32)
    ring_q = np.ascontiguousarray(ring_q, dtype=np.float32)
    ring_pos = np.ascontiguousarray(ring_pos, dtype=np.int32)
    d1 = ctypes.c_double()
    d2 = ctypes.c_double()
    j = _load().orc_nearest(_ptr(qt, _fp), _ptr(ring_q, _fp), _ptr(ring_pos, _i32p),
                            ring_pos.shape[0], qt.shape[0], int(m), ctypes.byref(d1),
                            ctypes.byref(d2))
    return j, d1.value, d2.value


class Oracle:
    """Per-(request, query head) MAC policy state and the batched decode call."""

    def __init__(self, B, Hq, Hkv, d, W, r, tau, theta, scale=None, kv_fp32=False, flags=0):
        """r: the band, one int for every head or a sequence of Hq per-head
        bands (Figure 3 (b))."""
        assert Hq % Hkv == 0
        bands = np.broadcast_to(np.asarray(r, np.int32), (Hq,)).copy()
        assert (bands >= 1).all()
        self.B, self.Hq, self.Hkv, self.d, self.W = B, Hq, Hkv, d, W
        self.r = int(bands[0]) if np.ndim(r) == 0 else bands
        self.tau = float(tau)
        scale = 1.0 / np.sqrt(d) if scale is None else float(scale)
        self._lib = _load()
        self._h = self._lib.orc_create(B, Hq, Hkv, d, W, int(bands.max()), float(tau),
                                       float(theta), scale, 1 if kv_fp32 else 0, int(flags))
        self._lib.orc_set_bands(self._h, _ptr(bands, _i32p))

    def __del__(self):
        h, self._h = getattr(self, "_h", None), None
        if h:
            self._lib.orc_destroy(h)

    def reset(self):
        self._lib.orc_reset(self._h)

    def ring_entry(self, b, h, slot):
        pos = ctypes.c_int32()
        q = np.empty(self.d, np.float32)
        s = np.empty(self.d + 2, np.float64)
        self._lib.orc_ring_entry(self._h, b, h, slot, ctypes.byref(pos), _ptr(q, _fp),
                                 _ptr(s, _dp))
        return pos.value, q, s

    def step(self, k_groups, v_groups, seq_lens, q_pre, override=None, track=None,
             want_full=False):
        """One decode call.  k_groups/v_groups: list of B*Hkv arrays [N][d] (or None
        for groups with no tracked head); returns a dict of numpy arrays."""
        B, Hq, Hkv, d = self.B, self.Hq, self.Hkv, self.d
        keep = []
        kp = (_vp * (B * Hkv))()
        vp = (_vp * (B * Hkv))()
        for i in range(B * Hkv):
            if k_groups[i] is None:
                kp[i] = vp[i] = None
                continue
            ka, _ = _kv(k_groups[i])
            va, _ = _kv(v_groups[i])
            keep += [ka, va]
            kp[i] = ka.ctypes.data
            vp[i] = va.ctypes.data
        seq = np.ascontiguousarray(seq_lens, dtype=np.int32)
        q = np.ascontiguousarray(q_pre, dtype=np.float32).reshape(B * Hq * d)
        ov = None if override is None else np.ascontiguousarray(override, np.int32).reshape(-1)
        tr = None if track is None else np.ascontiguousarray(track, np.uint8).reshape(-1)
        res = {
            "out": np.zeros((B, Hq, d)),
            "full": np.zeros((B, Hq, d)) if want_full else None,
            "hit": np.zeros((B, Hq), np.uint8),
            "p": np.zeros((B, Hq), np.int32),
            "rel": np.zeros((B, Hq)),
            "near_tau": np.zeros((B, Hq), np.uint8),
            "near_tie": np.zeros((B, Hq), np.uint8),
            "start": np.zeros((B, Hq), np.int32),
            "kv_tokens": np.zeros((B, Hkv), np.int64),
        }
        inv = self._lib.orc_step(
            self._h, kp, vp, _ptr(seq, _i32p), _ptr(q, _fp), _ptr(ov, _i32p), _ptr(tr, _u8p),
            _ptr(res["out"], _dp), _ptr(res["full"], _dp), _ptr(res["hit"], _u8p),
            _ptr(res["p"], _i32p), _ptr(res["rel"], _dp), _ptr(res["near_tau"], _u8p),
            _ptr(res["near_tie"], _u8p), _ptr(res["start"], _i32p),
            _ptr(res["kv_tokens"], _i64p))
        res["override_invalid"] = inv
        return res
