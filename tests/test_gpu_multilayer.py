"""Several layers, one amend stream: the continuous-generation recipe (AR(1)
queries with topic jumps, K/V appended every step) at a reduced size.

Each layer is its own handle with its own rings; all share one amend stream,
and the layers of a step are issued back to back, so amend(layer l, step t)
runs while later layers of step t are decoded (MAC-Attention, Figure 2 (c),
"async cache update").  Every layer is checked against its own oracle.
"""
import numpy as np
import pytest

from workloads import get_config, scaled

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("fused,shared", [(False, True), (True, True), (False, False)])
def test_layers_share_amend_stream_and_match_oracle(gpu_lib, fused, shared):
    """Default: amend of every layer on one shared stream.  Fused amend: no
    amend stream work at all, the layers' reduce kernels update their rings.
    Not shared: each layer creates its own amend stream, and its thread
    launches each call's amend once the reduce has run while the other
    layers' calls are enqueued."""
    import torch
    import kv_reuse_amd as mac
    from gpu_harness import Lockstep
    w = scaled(get_config("contgen"), B=4, C=1500, steps=40, layers=3, jump_every=16)
    print("case contgen layers", w.layers, "B", w.B, "C", w.C, "fused", fused, "shared", shared,
          flush=True)
    amend = torch.cuda.Stream() if shared else None
    flags = mac.MAC_F_FUSED_AMEND if fused else 0
    runs = [Lockstep(w, layer=layer, amend_stream=amend, flags=flags)
            for layer in range(w.layers)]
    hits = np.zeros(w.layers, int)
    try:
        for t in range(w.steps):
            # every layer of the step is enqueued before anything is awaited
            pending = [ls.launch(t) for ls in runs]
            for layer, (ls, pd) in enumerate(zip(runs, pending)):
                info = ls.finish(pd)
                hits[layer] += info["hits"]
                if t > 0 and t % w.jump_every == 0:
                    assert info["hits"] == 0, "a topic jump misses everywhere"
    finally:
        for ls in runs:
            ls.close()
    print("hits per layer", hits.tolist(), flush=True)
    assert (hits > 0).all()
