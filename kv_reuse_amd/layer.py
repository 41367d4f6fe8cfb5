"""MacLayer: one attention layer's MAC state behind the C ABI (handle ownership only)."""
from . import _lib


class MacLayer:
    """Owns a mac_handle for one layer; methods forward to the C ABI unchanged."""

    def __init__(self, cfg, main_stream=None, amend_stream=None):
        self.cfg = cfg
        self.h = _lib.mac_init(cfg, main_stream, amend_stream)

    def close(self):
        if getattr(self, "h", None) is not None:
            _lib.mac_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def reset(self):
        _lib.mac_reset(self.h)

    def append_kv(self, kv, k_new, v_new, positions, stream=None):
        _lib.mac_append_kv(self.h, kv, k_new, v_new, positions, stream)

    def decode_step(self, kv, q_pre_rope, out, override_pos=None, stream=None):
        _lib.mac_decode_step(self.h, kv, q_pre_rope, out, override_pos, stream)

    def prefill(self, kv, num_tokens, q_pre, out, override_pos=None, p_out=None, stream=None):
        _lib.mac_prefill(self.h, kv, num_tokens, q_pre, out, override_pos, p_out, stream)

    def prefill_noalloc(self, kv, num_tokens, q_pre, out, override_pos=None, p_out=None,
                        stream=None):
        _lib.mac_prefill_noalloc(self.h, kv, num_tokens, q_pre, out, override_pos, p_out, stream)

    def stats(self):
        return _lib.mac_stats(self.h)

    def debug_last(self):
        return _lib.mac_debug_last(self.h, self.cfg.batch, self.cfg.num_q_heads)
