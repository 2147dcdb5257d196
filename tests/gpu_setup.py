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
          inject=True, max_batch=None, max_inject_rows=256) -> Setup:
    ctx_lens = np.asarray(ctx_lens, dtype=np.int32)
    B = len(ctx_lens)
    w = synth.drafter_weights(cfg, seed=seed, std=weight_std, gain_std=gain_std)
    wd = {k: v.to("cuda") for k, v in w.items()}
    table, num_pages = synth.page_table(f"{cfg.name}/{tag}", ctx_lens + extra, cfg.page_size,
                                        seed, spare_pages=3)
    dr = Drafter(cfg, wd, max_batch=max_batch or B, max_ctx=table.shape[1] * cfg.page_size,
                 max_inject_rows=max_inject_rows)
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


def run_draft(s: Setup, anchors, want_logits=False, want_gap=False):
    """Draft ids [B, nb - 1] and, when asked, logits [B, nb - 1, V] and the reported top-2
    gaps (nb = the config's block size)."""
    B = len(anchors)
    nd = s.cfg.block_size - 1
    a = torch.as_tensor(np.asarray(anchors, dtype=np.int32)).to("cuda")
    ids = torch.full((B, nd), -7, dtype=torch.int32, device="cuda")
    logits = torch.empty((B, nd, s.cfg.vocab), dtype=torch.float32, device="cuda") \
        if want_logits else None
    gap = torch.full((B, nd), -1.0, dtype=torch.float32, device="cuda") if want_gap else None
    s.dr.draft(s.cache, a, ids, logits, top2_gap=gap)
    torch.cuda.synchronize()
    out = (ids.cpu().numpy(), (logits.cpu().numpy() if want_logits else None))
    return out + ((gap.cpu().numpy(),) if want_gap else ())


def cache_matches(gpu, exact, dtype, rel=2e-5, max_flip_frac=0.01, f32_rel=1e-5):
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
        return bool(err <= f32_rel), {"rel_err": float(err)}
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


# Logit bounds of a bf16 model (bf16 weights and cache, fp32 activations and accumulation).
# When both sides draft from the same seeded cache contents, the largest error must stay
# well within half the 2e-2 near-tie band, so a drafted id can only differ from the
# oracle's where the oracle's own gap is inside the band.  When the cache holds an injection, each
# side rounds its own projection to bf16 (the GPU its fp32 result, the oracle the exact
# value), and values near a rounding midpoint land one bf16 step apart (checked by
# cache_matches); this random-weight drafter amplifies those steps through attention and
# its five layers (measured: 4e-4 on a shared cache, up to ~3e-2 after the two
# injections), so there the bound is 5e-2 while the top-1/top-2 gap must still agree
# within the band.  (Shared cache, measured at the 8B shapes: max 2.3e-4 .. 3.4e-4, mean
# under 4.2e-5; the bounds below keep a margin of about 6x.)
# Temperature-1 verify: a decision is excused when the oracle's margin (distance of u * total
# to the nearest cumulative boundary, relative to the mass; or |u q - p| relative) is at most
# this.  Both sides evaluate the weights exp(x - max) and their sums in fp64 (the GPU's exp
# to below 4e-10 relative), so only margins below ~4e-10 can decide differently.
SAMPLED_MARGIN = 1e-9
LOGIT_MAX = 2e-3
LOGIT_MEAN = 2.5e-4
INJECTED_LOGIT_MAX = 5e-2
INJECTED_LOGIT_MEAN = 3e-3
GAP_TOL = 2e-2


def pool_context(cache, table, b, T):
    """Request b's cached K and V as the oracle takes them: per layer [T, n_kv, d] float64,
    read back from the device pages (bf16 or fp32 values widened exactly)."""
    if T == 0:
        return [], []
    pages = torch.from_numpy(np.ascontiguousarray(table[b, :(T + 15) // 16])).long().cuda()
    k = cache.k_pool[:, pages].permute(0, 1, 3, 2, 4)       # [L, np, 16, n_kv, d]
    v = cache.v_pool[:, pages].permute(0, 1, 4, 2, 3)       # [L, np, 16, n_kv, d]
    L, npg, P, nkv, d = k.shape
    k = k.reshape(L, npg * P, nkv, d)[:, :T].double().cpu().numpy()
    v = v.reshape(L, npg * P, nkv, d)[:, :T].double().cpu().numpy()
    return list(k), list(v)


def check_request(tag, b, got_ids, got_logits, got_gap, orc, dtype, logit_max=LOGIT_MAX,
                  logit_mean=LOGIT_MEAN):
    """ids bit-exact except at the oracle's near-ties; the logit error within `logit_max`;
    the GPU's top-1/top-2 gap (from its logits at the oracle's top two ids, and as the
    library reports it) within the band of the oracle's gap."""
    err = np.abs(got_logits - orc["logits"])
    bad, excused = compare_ids(got_ids, orc, dtype)
    two = np.argsort(-orc["logits"], axis=1, kind="stable")[:, :2]
    rows = np.arange(got_logits.shape[0])
    gpu_gap_at = got_logits[rows, two[:, 0]] - got_logits[rows, two[:, 1]]
    gap_err = np.abs(gpu_gap_at - orc["gap"])
    same = got_ids == orc["ids"]
    lib_gap_err = np.abs(got_gap - orc["gap"])[same]
    print(f"[{tag}] request {b}: mismatches {bad}, near-ties {excused}, logit error max "
          f"{err.max():.3e} mean {err.mean():.3e}, gap error {gap_err.max():.3e}, reported "
          f"gap error {lib_gap_err.max() if len(lib_gap_err) else 0:.3e}", flush=True)
    assert bad == 0
    assert err.max() <= logit_max and err.mean() <= logit_mean
    assert gap_err.max() < GAP_TOL
    assert (lib_gap_err < GAP_TOL).all() and (got_gap >= 0).all()




def check_injected_request(tag, s_cfg, w, b, anchor, got_ids, got_logits, got_gap, own_ctx):
    """A request whose context the library injected, against the oracle's own injection of
    the same features: ids, gaps, and logits within INJECTED_LOGIT_MAX."""
    orc = ref.draft_block(s_cfg, w, *own_ctx, anchor, want_logits=True)
    check_request(tag, b, got_ids, got_logits, got_gap, orc, s_cfg.dtype,
                  logit_max=INJECTED_LOGIT_MAX, logit_mean=INJECTED_LOGIT_MEAN)
    return orc


def fill_cache(cache, seed: int, tag: str, std: float = 3.0) -> None:
    """Seeded synthetic K/V in every page (device RNG; the scale of injected K/V at the
    8B shapes).  The oracle reads these inputs back with pool_context."""
    gen = torch.Generator(device="cuda").manual_seed(synth.stream_seed(seed, tag + "/fill"))
    for pool in (cache.k_pool, cache.v_pool):
        pool.normal_(0.0, std, generator=gen)
