"""Shared set-up for the GPU parity tests: seeded inputs on both sides, the drafter on the
device through the C ABI, and the oracle's view of the same request."""
from dataclasses import dataclass
from typing import List

import numpy as np
import torch

import oracle.dflash_oracle as ref
from block_diffusion_drafter_hidden_amd import Drafter
from workloads import synth


def gpu_available() -> bool:
    return torch.cuda.is_available()


@dataclass
class Setup:
    cfg: object
    w: dict                   # host weights (oracle side)
    wd: dict                  # device weights
    dr: Drafter
    cache: object
    ctx_lens: np.ndarray
    table: np.ndarray
    feats: List[torch.Tensor]  # per-request context features (host)


def build(cfg, ctx_lens, tag="t", seed=0, extra=16, weight_std=0.02, gain_std=0.02,
          inject=True, max_batch=None) -> Setup:
    ctx_lens = np.asarray(ctx_lens, dtype=np.int32)
    B = len(ctx_lens)
    w = synth.drafter_weights(cfg, seed=seed, std=weight_std, gain_std=gain_std)
    wd = {k: v.to("cuda") for k, v in w.items()}
    table, num_pages = synth.page_table(f"{cfg.name}/{tag}", ctx_lens + extra, cfg.page_size,
                                        seed, spare_pages=3)
    dr = Drafter(cfg, wd, max_batch=max_batch or B, max_ctx=table.shape[1] * cfg.page_size,
                 max_inject_rows=256)
    cache = dr.new_cache(table, ctx_lens, num_pages)
    feats = [synth.target_features(cfg, int(T), f"{tag}/ctx/b{b}", seed=seed)
             for b, T in enumerate(ctx_lens)]
    s = Setup(cfg, w, wd, dr, cache, ctx_lens, table, feats)
    if inject and ctx_lens.sum() > 0:
        inject_rows(s, feats, [np.arange(T) for T in ctx_lens])
    return s


def inject_rows(s: Setup, feats_per_req, pos_per_req) -> None:
    rows = [f for f in feats_per_req if f.shape[0] > 0]
    if not rows:
        return
    X = torch.cat(rows).to("cuda")
    seq = np.concatenate([np.full(len(p), b, dtype=np.int32) for b, p in enumerate(pos_per_req)])
    pos = np.concatenate([np.asarray(p, dtype=np.int32) for p in pos_per_req])
    s.dr.inject(s.cache, X, torch.from_numpy(seq).to("cuda"), torch.from_numpy(pos).to("cuda"))


def gather_pool(s: Setup, b: int, T: int, which: str = "k") -> np.ndarray:
    """Cached K or V of request b, positions 0..T-1, as [L, T, n_kv, d] float64 (host)."""
    t = np.arange(T)
    pages = s.table[b, t // s.cfg.page_size]
    if which == "k":   # [L, pages, n_kv, 16, d]
        pool = s.cache.k_pool.float().cpu().numpy()
        g = pool[:, pages, :, t % s.cfg.page_size, :]
    else:              # [L, pages, n_kv, d, 16]
        pool = s.cache.v_pool.float().cpu().numpy()
        g = pool[:, pages, :, :, t % s.cfg.page_size]
    return g.transpose(1, 0, 2, 3).astype(np.float64)


def oracle_context(s: Setup, b: int):
    return ref.prefill_context(s.cfg, s.w, s.feats[b]) if s.ctx_lens[b] > 0 else ([], [])


def run_draft(s: Setup, anchors, want_logits=False):
    B = len(anchors)
    a = torch.as_tensor(np.asarray(anchors, dtype=np.int32)).to("cuda")
    ids = torch.full((B, 15), -7, dtype=torch.int32, device="cuda")
    logits = torch.empty((B, 15, s.cfg.vocab), dtype=torch.float32, device="cuda") \
        if want_logits else None
    s.dr.draft(s.cache, a, ids, logits)
    torch.cuda.synchronize()
    return ids.cpu().numpy(), (logits.cpu().numpy() if want_logits else None)


def cache_matches(gpu, exact, dtype, rel=2e-5, max_flip_frac=0.01):
    """GPU cache values against the exact (float64) injected values.

    fp32 cache: within 1e-5 of RMS.  bf16 cache: every value must be the bf16 rounding of
    some number within delta = rel * (|exact| + RMS) of the exact value -- fp32 accumulation
    of the projection lands that close, and rounding is monotone, so the value must lie in
    [round(exact - delta), round(exact + delta)] -- and at most `max_flip_frac` of the values
    may differ from round(exact) at all."""
    exact = np.asarray(exact, dtype=np.float64)
    rms = np.sqrt(np.mean(exact * exact))
    if dtype == "f32":
        err = np.abs(gpu - exact).max() / rms
        return bool(err <= 1e-5), {"rel_err": float(err)}
    delta = rel * (np.abs(exact) + rms)
    lo, hi = ref.round_bf16(exact - delta), ref.round_bf16(exact + delta)
    inside = (gpu >= lo) & (gpu <= hi)
    frac = float((gpu != ref.round_bf16(exact)).mean())
    ok = bool(inside.all() and frac < max_flip_frac)
    return ok, {"outside": int((~inside).sum()), "flip_frac": frac}


def compare_ids(gpu_ids, orc, dtype):
    """Bit-exact ids except at the oracle's near-ties.  Returns (mismatches, excused)."""
    tie = ref.near_tie(orc["gap"], orc["top1"], orc["top2"], dtype)
    bad = (gpu_ids != orc["ids"]) & ~tie
    return int(bad.sum()), int(tie.sum())
