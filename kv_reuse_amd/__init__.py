"""MAC-Attention decode step for MI355X (gfx950): Python binding of libmac.so.

The compute path is the HIP library built from kv_reuse_amd/csrc (C ABI in
include/mac.h).  This package marshals arguments; see kv_reuse_amd._lib.
"""
from ._lib import (EXPORTS, LIB_PATH, MAC_BF16, MAC_EHIP, MAC_EINVAL, MAC_ENOMEM, MAC_ESTATE,
                   MAC_EUNSUPPORTED, MAC_F_DISABLE_REUSE, MAC_F_FUSED_AMEND, MAC_F_RECORD_DEBUG,
                   MAC_F_RING_BF16, MAC_F_STALE_RING, MAC_F_UNBALANCED_PLAN,
                   MAC_F_SYNC_AMEND,
                   MAC_F_TIMING, MAC_FP32, MAC_KV_CONTIGUOUS, MAC_KV_PAGED, MAC_OK, MacConfig,
                   MacError, MacKvView, MacStats, load, mac_append_kv, mac_aux_bytes,
                   mac_config_validate, mac_debug_last, mac_decode_step, mac_destroy, mac_init,
                   mac_last_error, mac_prefill, mac_prefill_noalloc, mac_reset, mac_stats, mac_status_string, make_config,
                   make_kv_view)
from .layer import MacLayer

__all__ = [n for n in dir() if not n.startswith("_")]
