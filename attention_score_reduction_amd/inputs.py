"""Seeded synthetic inputs for reconstruction-attention scoring.

This module is shared by the tests, the benchmark and the oracle's callers.  It
draws random numbers and rounds them to the storage type; it holds none of the
scoring, selection or compaction arithmetic.

Workloads (shapes from the pages: LLaMA3.1-8B, Qwen2.5-14B and Gemma3-12B
contexts up to 170K tokens, 2K-token scoring chunks, a short repeat prompt in
front of each chunk -- KVzip blog post, sections 4.1 and 4.5; paperhub
rebuttal, answers on positional OOD and on computational analysis):

* every tensor entry is N(0, 1) in fp32, then rounded to bf16 with
  round-to-nearest-even (or kept fp32 for the fp32 workload);
* ``key_lognormal_sigma``: one factor exp(sigma * z), z ~ N(0, 1), per
  (layer, head), multiplying that head's context keys and in-chunk keys;
* ``sink``: context key 0 of every head multiplied by 4;
* ``peaked_frac``: that fraction of context positions per head, drawn without
  replacement, with keys multiplied by 3.

Two generators exist.  ``HostGen`` (numpy PCG64 keyed by
``SeedSequence([seed, layer, tensor_id, chunk])``) is exact and reproducible
on any machine and feeds every parity test.  ``device_tensors`` (torch's
device generator) fills a full-size cache directly in device memory for the
throughput benchmark, where 60 GB of host-side sampling would dominate.
"""
from __future__ import annotations

import dataclasses

import numpy as np

BF16 = "bf16"
F32 = "f32"

# tensor ids for the seed sequence
_T_QUERY, _T_KCTX, _T_VCTX, _T_KIN, _T_FACTOR, _T_PEAK, _T_VIN = range(7)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    layers: int
    heads: int          # KV heads per layer
    group: int          # query heads per KV head
    head_dim: int
    n_ctx: int
    chunk: int          # context tokens per reconstruction chunk
    n_prompt: int       # repeat-prompt tokens in front of each chunk
    keep_ratio: float
    dtype: str = BF16
    key_lognormal_sigma: float = 0.0
    sink: bool = False
    peaked_frac: float = 0.0

    @property
    def n_heads(self) -> int:
        return self.layers * self.heads

    @property
    def n_total(self) -> int:
        return self.layers * self.heads * self.n_ctx

    def chunks(self):
        """List of (start, length) of the context chunks, the last one ragged."""
        out = []
        s = 0
        while s < self.n_ctx:
            m = min(self.chunk, self.n_ctx - s)
            out.append((s, m))
            s += m
        return out

    def n_in(self, k: int) -> int:
        return self.n_prompt + self.chunks()[k][1]

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    "tiny_fp32": Workload("tiny_fp32", 0, 1, 1, 2, 64, 512, 128, 8, 0.3, F32,
                          sink=True),
    "llama8b_8k": Workload("llama8b_8k", 1, 32, 8, 4, 128, 8192, 2048, 16, 0.3,
                           key_lognormal_sigma=0.5, sink=True),
    "llama8b_128k": Workload("llama8b_128k", 2, 32, 8, 4, 128, 131072, 2048, 16,
                             0.3, key_lognormal_sigma=0.5, sink=True),
    "qwen14b_120k": Workload("qwen14b_120k", 3, 48, 8, 5, 128, 120000, 2048, 16,
                             0.25, peaked_frac=0.05),
    "gemma12b_170k": Workload("gemma12b_170k", 4, 48, 8, 2, 256, 170000, 1024,
                              16, 0.4, key_lognormal_sigma=1.0),
}


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest, ties to even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounding = ((u >> 16) & 1) + np.uint32(0x7FFF)
    return ((u + rounding) >> 16).astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> fp32 (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


class HostGen:
    """Exact, seeded host-side generator for one workload."""

    def __init__(self, wl: Workload):
        self.wl = wl

    def _rng(self, layer, tensor_id, chunk=0):
        ss = np.random.SeedSequence([self.wl.seed, layer, tensor_id, chunk])
        return np.random.Generator(np.random.PCG64(ss))

    def _store(self, x32):
        return bf16_bits(x32) if self.wl.dtype == BF16 else x32.astype(np.float32)

    def key_factors(self, layer):
        """fp32 factor per KV head of this layer (1.0 when disabled)."""
        wl = self.wl
        if wl.key_lognormal_sigma == 0.0:
            return np.ones(wl.heads, np.float32)
        z = self._rng(layer, _T_FACTOR).standard_normal(wl.heads)
        return np.exp(wl.key_lognormal_sigma * z).astype(np.float32)

    def context(self, layer, heads=None):
        """(K_c, V_c) of one layer: [H][n_c][d] each, storage type.

        ``heads`` restricts the output to a subset of head indices (the draws
        stay those of the full layer, so a subset equals the slice).
        """
        wl = self.wl
        hs = list(range(wl.heads)) if heads is None else list(heads)
        f = self.key_factors(layer)
        rk = self._rng(layer, _T_KCTX)
        rv = self._rng(layer, _T_VCTX)
        kout, vout = [], []
        for h in range(wl.heads):
            # draw every head in order so that subsets reproduce the full layer
            k = rk.standard_normal((wl.n_ctx, wl.head_dim), dtype=np.float32)
            v = rv.standard_normal((wl.n_ctx, wl.head_dim), dtype=np.float32)
            if h not in hs:
                continue
            k *= f[h]
            if wl.sink:
                k[0] *= 4.0
            if wl.peaked_frac > 0.0:
                cnt = int(round(wl.peaked_frac * wl.n_ctx))
                pos = self._rng(layer, _T_PEAK, h).choice(wl.n_ctx, cnt, replace=False)
                k[pos] *= 3.0
            kout.append(self._store(k))
            vout.append(self._store(v))
        return np.stack(kout), np.stack(vout)

    def chunk_inputs(self, layer, k, heads=None):
        """(Q [H][G][n_in][d], K_in [H][n_in][d]) of chunk k of one layer."""
        wl = self.wl
        hs = list(range(wl.heads)) if heads is None else list(heads)
        n_in = wl.n_in(k)
        f = self.key_factors(layer)
        rq = self._rng(layer, _T_QUERY, k)
        rk = self._rng(layer, _T_KIN, k)
        q = rq.standard_normal((wl.heads, wl.group, n_in, wl.head_dim), dtype=np.float32)
        kin = rk.standard_normal((wl.heads, n_in, wl.head_dim), dtype=np.float32)
        kin *= f[:, None, None]
        return self._store(q[hs]), self._store(kin[hs])

    def chunk_values(self, layer, k, heads=None):
        """V_in [H][n_in][d] of chunk k of one layer (the values of the
        repeat-prompt and copied-context tokens), N(0, 1) like V_c."""
        wl = self.wl
        hs = list(range(wl.heads)) if heads is None else list(heads)
        rv = self._rng(layer, _T_VIN, k)
        vin = rv.standard_normal((wl.heads, wl.n_in(k), wl.head_dim), dtype=np.float32)
        return self._store(vin[hs])


def device_tensors(wl: Workload, device="cuda", layers=None):
    """Full-size synthetic inputs generated in device memory (torch generator).

    Returns a dict with
      kc, vc : [L][H][n_c][d]
      q      : list over layers of list over chunks of [H][G][n_in][d]
      kin    : list over layers of list over chunks of [H][n_in][d]
    Chunks of equal length share one allocation per layer ([n_chunks][...]),
    so the list entries are views.
    """
    import torch

    dt = torch.bfloat16 if wl.dtype == BF16 else torch.float32
    L = wl.layers if layers is None else layers
    g = torch.Generator(device=device)
    g.manual_seed(wl.seed)
    H, G, D, n_c = wl.heads, wl.group, wl.head_dim, wl.n_ctx

    def randn(*shape):
        return torch.randn(*shape, generator=g, device=device, dtype=torch.float32)

    fac = torch.exp(wl.key_lognormal_sigma * randn(L, H))
    kc = torch.empty(L, H, n_c, D, device=device, dtype=dt)
    vc = torch.empty(L, H, n_c, D, device=device, dtype=dt)
    for l in range(L):
        k = randn(H, n_c, D) * fac[l][:, None, None]
        if wl.sink:
            k[:, 0] *= 4.0
        if wl.peaked_frac > 0.0:
            cnt = int(round(wl.peaked_frac * n_c))
            for h in range(H):
                pos = torch.randperm(n_c, generator=g, device=device)[:cnt]
                k[h, pos] *= 3.0
        kc[l] = k.to(dt)
        vc[l] = randn(H, n_c, D).to(dt)
        del k
    chunks = wl.chunks()
    full = [c for c in chunks if c[1] == wl.chunk]
    tail = [c for c in chunks if c[1] != wl.chunk]
    q, kin = [], []
    for l in range(L):
        ql, kl = [], []
        if full:
            n_in = wl.n_prompt + wl.chunk
            qa = randn(len(full), H, G, n_in, D).to(dt)
            ka = (randn(len(full), H, n_in, D) * fac[l][None, :, None, None]).to(dt)
            ql += [qa[i] for i in range(len(full))]
            kl += [ka[i] for i in range(len(full))]
        for (_, m) in tail:
            n_in = wl.n_prompt + m
            ql.append(randn(H, G, n_in, D).to(dt))
            kl.append((randn(H, n_in, D) * fac[l][:, None, None]).to(dt))
        q.append(ql)
        kin.append(kl)
    return {"kc": kc, "vc": vc, "q": q, "kin": kin}

