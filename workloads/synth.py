"""Seeded synthetic inputs for the DFlash draft step.

Shared by the oracle-side tests and by the GPU-side tests and benchmark, so
that both see identical bytes.  Only random draws and test-data
construction live here; none of the method's arithmetic does.

Every tensor is drawn from its own stream: seed = config_seed * 1_000_003 +
crc32(name), split into fixed chunks of 2**22 elements that each get a derived
seed, so any tensor (or any chunk) can be regenerated alone and the draw is
independent of thread count.  Distributions follow the workload descriptions:
weights N(0, 0.02), RMSNorm gains 1 + N(0, 0.02), target features N(0, 1),
token ids uniform over the vocabulary.  The second parameter of N(., .) is a
standard deviation.
"""
from __future__ import annotations

import zlib
from concurrent.futures import ThreadPoolExecutor
from typing import Dict, Tuple

import numpy as np
import torch

from .configs import DrafterConfig, Workload

_CHUNK = 1 << 22
_POOL = None


def _pool() -> ThreadPoolExecutor:
    global _POOL
    if _POOL is None:
        import os
        _POOL = ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 1))
    return _POOL


def torch_dtype(dtype: str) -> torch.dtype:
    return {"f32": torch.float32, "bf16": torch.bfloat16}[dtype]


def stream_seed(seed: int, name: str) -> int:
    return (seed * 1_000_003 + zlib.crc32(name.encode())) % (1 << 62)


def normal(name: str, shape, std: float = 1.0, mean: float = 0.0, dtype: str = "f32",
           seed: int = 0) -> torch.Tensor:
    """N(mean, std) tensor rounded to `dtype`, drawn chunk by chunk in parallel."""
    shape = tuple(int(s) for s in shape)
    n = int(np.prod(shape)) if shape else 1
    out = torch.empty(n, dtype=torch_dtype(dtype))
    base = stream_seed(seed, name)

    def fill(ci: int) -> None:
        lo = ci * _CHUNK
        hi = min(n, lo + _CHUNK)
        g = torch.Generator().manual_seed((base * 7919 + ci * 104729 + 1) % (1 << 62))
        v = torch.randn(hi - lo, generator=g, dtype=torch.float32)
        if std != 1.0:
            v.mul_(std)
        if mean != 0.0:
            v.add_(mean)
        out[lo:hi] = v.to(out.dtype)

    nchunks = (n + _CHUNK - 1) // _CHUNK
    if nchunks <= 1:
        fill(0)
    else:
        list(_pool().map(fill, range(nchunks)))
    return out.view(shape)


def uniform_ints(name: str, shape, lo: int, hi: int, seed: int = 0) -> np.ndarray:
    """Integers uniform over [lo, hi] inclusive, int32."""
    rng = np.random.Generator(np.random.PCG64(stream_seed(seed, name)))
    return rng.integers(lo, hi + 1, size=shape, dtype=np.int64).astype(np.int32)


def uniforms(name: str, shape, seed: int = 0) -> np.ndarray:
    """float32 uniforms in [0, 1), clamped strictly below 1."""
    rng = np.random.Generator(np.random.PCG64(stream_seed(seed, name)))
    u = rng.random(size=shape, dtype=np.float64).astype(np.float32)
    return np.minimum(u, np.float32(1.0 - 2.0 ** -24))


# ----------------------------------------------------------------------------------------
# Model weights
# ----------------------------------------------------------------------------------------

def drafter_weights(cfg: DrafterConfig, seed: int = 0, std: float = 0.02,
                    gain_std: float = 0.02) -> Dict[str, torch.Tensor]:
    """Random-init drafter in logical nn.Linear layout ([out, in], row-major), on the host."""
    w = {}
    for name, shp in cfg.weight_shapes().items():
        key = f"{cfg.name}/{name}"
        if "norm" in name:
            w[name] = normal(key, shp, std=gain_std, mean=1.0, dtype=cfg.dtype, seed=seed)
        else:
            w[name] = normal(key, shp, std=std, dtype=cfg.dtype, seed=seed)
    return w


def target_features(cfg: DrafterConfig, n_tok: int, tag: str, seed: int = 0) -> torch.Tensor:
    """Concatenated multi-layer target hidden states [n_tok, n_feat_layers * target_hidden].

    Layer-major concatenation, ascending layer: row t = [h^(1)_t | h^(2)_t | ...]."""
    return normal(f"{cfg.name}/features/{tag}", (n_tok, cfg.feat_dim), std=1.0,
                  dtype=cfg.dtype, seed=seed)


def anchor_ids(cfg: DrafterConfig, batch: int, seed: int = 0, tag: str = "anchor") -> np.ndarray:
    return uniform_ints(f"{cfg.name}/{tag}", (batch,), 0, cfg.vocab - 1, seed)


# ----------------------------------------------------------------------------------------
# Context lengths and the paged KV cache geometry
# ----------------------------------------------------------------------------------------

def context_lengths(wl: Workload) -> np.ndarray:
    lo, hi = wl.ctx
    if lo == hi:
        return np.full((wl.batch,), lo, dtype=np.int32)
    return uniform_ints(f"{wl.name}/ctx_lens", (wl.batch,), lo, hi, wl.seed)


def page_table(name: str, ctx_caps: np.ndarray, page: int, seed: int = 0,
               spare_pages: int = 0) -> Tuple[np.ndarray, int]:
    """Block table [B, max_pages] over a randomly permuted physical page pool.

    ctx_caps[b] is the number of token slots request b must be able to hold.
    Unused table entries are -1.  Returns (table, num_pages)."""
    caps = np.asarray(ctx_caps, dtype=np.int64)
    need = (caps + page - 1) // page
    total = int(need.sum()) + spare_pages
    max_pages = max(1, int(need.max()) if len(need) else 1)
    rng = np.random.Generator(np.random.PCG64(stream_seed(seed, name + "/pages")))
    perm = rng.permutation(total).astype(np.int32)
    table = np.full((len(caps), max_pages), -1, dtype=np.int32)
    off = 0
    for b, nb in enumerate(need):
        table[b, :nb] = perm[off:off + nb]
        off += nb
    return table, total


# ----------------------------------------------------------------------------------------
# Verify inputs
# ----------------------------------------------------------------------------------------

def plant_draws(name: str, batch: int, vocab: int, seed: int = 0, k: np.ndarray = None,
                n_drafts: int = 15):
    """Seeded draws of the planting rule that do not depend on the drafts: k [B] ~
    U{0..n_drafts} matching drafts (unless given), the free target ids fill [B, n_drafts+1]
    ~ U{0..V-1} and the mismatch offsets r [B] ~ U{0..V-2}."""
    rng = np.random.Generator(np.random.PCG64(stream_seed(seed, name + "/plant")))
    if k is None:
        k = rng.integers(0, n_drafts + 1, size=batch)
    fill = rng.integers(0, vocab, size=(batch, n_drafts + 1))
    r = rng.integers(0, vocab - 1, size=batch)
    return np.asarray(k, dtype=np.int64), fill, r


def plant(draft_ids: np.ndarray, k, fill, r, vocab: int) -> np.ndarray:
    """Target ids [B, 16] from drafts [B, 15]: t[i-1] = d[i] for i <= k; if k < 15, slot k
    is d[k+1] shifted by 1 + r (mod V), so it differs; the rest are `fill`.  This pins the
    greedy accept length to k + 1."""
    d = np.asarray(draft_ids, dtype=np.int64)
    B, nd = d.shape
    t = np.array(fill, dtype=np.int64, copy=True)
    for b in range(B):
        t[b, :k[b]] = d[b, :k[b]]
        if k[b] < nd:
            t[b, k[b]] = (d[b, k[b]] + 1 + r[b]) % vocab
    return t.astype(np.int32)


def plant_device(draft_ids, k, fill, r, vocab: int):
    """`plant` on device tensors (drafts [B, 15] int32; k [B], fill [B, 16], r [B] int64), so
    a captured decoding loop can build its synthetic target ids without the host."""
    B, nd = draft_ids.shape
    dev = draft_ids.device
    j = torch.arange(nd + 1, device=dev)[None, :]
    dpad = torch.cat([draft_ids.long(), torch.zeros((B, 1), dtype=torch.long, device=dev)], 1)
    kk = k.long()[:, None]
    t = torch.where(j < kk, dpad, fill.long())
    miss = (torch.gather(dpad, 1, kk.clamp(max=nd - 1)) + 1 + r.long()[:, None]) % vocab
    t = torch.where((j == kk) & (kk < nd), miss, t)
    return t.to(torch.int32)


def planted_targets(draft_ids: np.ndarray, vocab: int, name: str, seed: int = 0,
                    k: np.ndarray = None) -> Tuple[np.ndarray, np.ndarray]:
    """Target ids [B, 16] with a planted matching prefix against `draft_ids` [B, 15]
    (k[b] ~ U{0..15} unless given; see `plant`).  Returns (target_ids, k)."""
    d = np.asarray(draft_ids, dtype=np.int64)
    k, fill, r = plant_draws(name, d.shape[0], vocab, seed, k, d.shape[1])
    return plant(d, k, fill, r, vocab), k.astype(np.int32)


def sampled_verify_inputs(wl: Workload, batch: int = None, vocab: int = None):
    """Draft logits [B,15,V], target logits [B,16,V] (fp32, N(0, logit_std)) and the
    three uniform streams of the speculative accept/reject rule."""
    B = wl.batch if batch is None else batch
    V = wl.cfg.vocab if vocab is None else vocab
    nd = wl.cfg.block_size - 1
    tag = f"{wl.name}/B{B}/V{V}"
    dl = normal(tag + "/draft_logits", (B, nd, V), std=wl.logit_std, dtype="f32", seed=wl.seed)
    tl = normal(tag + "/target_logits", (B, nd + 1, V), std=wl.logit_std, dtype="f32",
                seed=wl.seed)
    u_draft = uniforms(tag + "/u_draft", (B, nd), wl.seed)
    u_accept = uniforms(tag + "/u_accept", (B, nd), wl.seed)
    u_resample = uniforms(tag + "/u_resample", (B,), wl.seed)
    return dl, tl, u_draft, u_accept, u_resample
