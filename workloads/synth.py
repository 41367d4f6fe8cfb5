"""Workload definitions and seeded generators.

Each workload is a stand-in, built from shapes only, for the evaluation the
MAC-Attention pages run (LongBench v2 and RULER at ~120K context, LongGenBench's
16K continuous generation; LLaMA-3.1-8B and Qwen3-30B-A3B head shapes).  No
benchmark item is reproduced: keys, values and queries are random.

Draw recipe (one SeedSequence per workload, spawned into independent streams):
  stream 0  keys and values: N(0,1) fp32 from a torch generator on the target
            device, rounded once to bf16 (round-to-nearest-even) when the
            workload stores bf16.  Keys are taken as already rotated
            (post-RoPE); RoPE is orthogonal, so the distribution is the same.
  stream 1  pre-RoPE queries: per (request, head) an AR(1) walk in fp64,
            q_0 ~ N(0, I), q_t = rho*q_{t-1} + sqrt(1-rho^2)*eps_t, stored fp32.
  stream 2  rho draws (per request, for the mixed workload).
  stream 3  page permutation: one random permutation of all page ids.
  stream 4  topic jumps (continuous generation): fresh eps, rho = 0.
"""
from dataclasses import dataclass, replace
from typing import Optional, Tuple

import numpy as np

PAGE = 16


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    Hq: int
    Hkv: int
    d: int
    C: int            # prefilled context per request
    steps: int        # decode steps
    W: int            # ring length
    r: int            # band width
    tau: float        # relative-L2 threshold
    theta: float      # RoPE base
    kv: str           # "bf16" | "fp32"
    layout: str       # "contiguous" | "paged"
    rho: tuple        # ("const", x) | ("per_request_uniform", lo, hi) | ("per_head_linear", lo, hi)
    layers: int = 1
    jump_every: int = 0   # topic jump (fresh query) every this many steps; 0 = never
    seed: int = 0

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def n_cap(self) -> int:
        """Token capacity per request: prefill + decode steps, rounded up to a page."""
        n = self.C + self.steps
        return (n + PAGE - 1) // PAGE * PAGE

    @property
    def pages_per_req(self) -> int:
        return self.n_cap // PAGE

    @property
    def kv_elem_bytes(self) -> int:
        return 4 if self.kv == "fp32" else 2


CONFIGS = {
    # 1 request, 8q/2kv, fp32 KV, 4096 prefill + 256 steps, rho 0.95, ring 16, r 64
    "cpu4k": Workload("cpu4k", B=1, Hq=8, Hkv=2, d=128, C=4096, steps=256, W=16, r=64,
                      tau=0.3, theta=500000.0, kv="fp32", layout="contiguous",
                      rho=("const", 0.95)),
    # LLaMA-3.1-8B-shaped layer, batch 1, 32K contiguous bf16, 512 steps, rho 0.97
    "llama32k": Workload("llama32k", B=1, Hq=32, Hkv=8, d=128, C=32768, steps=512, W=32,
                         r=256, tau=0.3, theta=500000.0, kv="bf16", layout="contiguous",
                         rho=("const", 0.97)),
    # batch 16 x 128K, paged bf16, per-request rho ~ U[0.8, 0.99]
    "b16_128k": Workload("b16_128k", B=16, Hq=32, Hkv=8, d=128, C=131072, steps=256, W=32,
                         r=256, tau=0.3, theta=500000.0, kv="bf16", layout="paged",
                         rho=("per_request_uniform", 0.8, 0.99)),
    # 32q/4kv MoE-style heads, batch 8 x 122880, per-head rho 0.5 .. 0.99 (r swept 64/256/1024)
    "moe_122k": Workload("moe_122k", B=8, Hq=32, Hkv=4, d=128, C=122880, steps=256, W=32,
                         r=256, tau=0.3, theta=500000.0, kv="bf16", layout="paged",
                         rho=("per_head_linear", 0.5, 0.99)),
    # continuous generation: batch 32, 16K prompt + 16K generated, 32 layers, rho 0.95,
    # topic jump every 2048 steps (ring, band and threshold as the 32q/8kv workloads)
    "contgen": Workload("contgen", B=32, Hq=32, Hkv=8, d=128, C=16384, steps=16384, W=32,
                        r=256, tau=0.3, theta=500000.0, kv="bf16", layout="paged",
                        rho=("const", 0.95), layers=32, jump_every=2048),
}


def get_config(name: str) -> Workload:
    return CONFIGS[name]


def scaled(w: Workload, **kw) -> Workload:
    """A copy of a workload with some fields replaced (smaller test sizes)."""
    return replace(w, **kw)


def _streams(w: Workload):
    return np.random.SeedSequence(w.seed).spawn(5)


def _torch_seed(ss: np.random.SeedSequence, salt: int = 0) -> int:
    return int(ss.generate_state(2, dtype=np.uint64)[salt] & np.uint64(0x7FFFFFFFFFFFFFFF))


def rho_values(w: Workload) -> np.ndarray:
    """AR(1) coefficient per (request, query head), float64 [B, Hq]."""
    kind = w.rho[0]
    if kind == "const":
        return np.full((w.B, w.Hq), float(w.rho[1]))
    if kind == "per_request_uniform":
        g = np.random.Generator(np.random.PCG64(_streams(w)[2]))
        rb = g.uniform(w.rho[1], w.rho[2], size=w.B)
        return np.repeat(rb[:, None], w.Hq, axis=1)
    if kind == "per_head_linear":
        lo, hi = w.rho[1], w.rho[2]
        rh = lo + (hi - lo) * np.arange(w.Hq) / max(w.Hq - 1, 1)
        return np.repeat(rh[None, :], w.B, axis=0)
    raise ValueError(kind)


def queries(w: Workload, steps: Optional[int] = None, layer: int = 0) -> np.ndarray:
    """Pre-RoPE queries, float32 [steps, B, Hq, d] (AR(1) walk in fp64)."""
    steps = w.steps if steps is None else steps
    ss = _streams(w)[1].spawn(w.layers)[layer]
    g = np.random.Generator(np.random.PCG64(ss))
    rho = rho_values(w)[:, :, None]
    c = np.sqrt(1.0 - rho * rho)
    out = np.empty((steps, w.B, w.Hq, w.d), np.float32)
    q = g.standard_normal((w.B, w.Hq, w.d))
    for t in range(steps):
        if t > 0:
            eps = g.standard_normal((w.B, w.Hq, w.d))
            if w.jump_every and t % w.jump_every == 0:
                q = eps
            else:
                q = rho * q + c * eps
        out[t] = q.astype(np.float32)
    return out


def kv_logical(w: Workload, device="cpu", layer: int = 0, n_tokens: Optional[int] = None):
    """Logical keys and values, torch tensors [B, Hkv, n, d] on `device`
    (bf16 or fp32 as the workload stores them); n defaults to the capacity."""
    import torch
    n = w.n_cap if n_tokens is None else n_tokens
    ss = _streams(w)[0].spawn(w.layers)[layer]
    gen = torch.Generator(device=device)
    gen.manual_seed(_torch_seed(ss))
    shape = (w.B, w.Hkv, n, w.d)
    dt = torch.bfloat16 if w.kv == "bf16" else torch.float32
    k = torch.empty(shape, dtype=dt, device=device)
    v = torch.empty(shape, dtype=dt, device=device)
    # fill one (request, head) block at a time: bounded fp32 staging memory
    tmp = torch.empty((n, w.d), dtype=torch.float32, device=device)
    for dst in (k, v):
        for b in range(w.B):
            for g in range(w.Hkv):
                tmp.normal_(generator=gen)
                dst[b, g].copy_(tmp)   # fp32 -> bf16 rounds to nearest even
    return k, v


def page_table(w: Workload) -> np.ndarray:
    """Request b's logical page i lives in physical page perm[b*pages_per_req + i]; int32 [B, P]."""
    g = np.random.Generator(np.random.PCG64(_streams(w)[3]))
    P = w.pages_per_req
    perm = g.permutation(w.B * P).astype(np.int32)
    return perm.reshape(w.B, P)


def to_paged(x, table):
    """Scatter a logical cache [B, Hkv, n, d] into pages [num_pages, Hkv, 16, d]."""
    import torch
    B, Hkv, n, d = x.shape
    P = n // PAGE
    t = torch.as_tensor(np.asarray(table)[:, :P].reshape(-1), dtype=torch.long, device=x.device)
    src = x.reshape(B, Hkv, P, PAGE, d).permute(0, 2, 1, 3, 4).reshape(B * P, Hkv, PAGE, d)
    out = torch.empty((int(np.asarray(table).size), Hkv, PAGE, d), dtype=x.dtype,
                      device=x.device)
    out.index_copy_(0, t, src)
    return out


def bf16_bits(x) -> np.ndarray:
    """Host numpy view of a torch tensor's raw storage: uint16 bf16 bits or float32."""
    import torch
    if x.dtype == torch.bfloat16:
        return x.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    return x.detach().contiguous().cpu().numpy()
