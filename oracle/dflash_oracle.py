"""CPU oracle for one DFlash draft step with KV injection, then verification.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this module.  The GPU library never calls it, and
it shares no code with the GPU path: inputs come from the seeded generators in
`workloads/`, outputs are compared by the tests.

Everything is plain float64 numpy (inputs, which may be bf16, are widened
exactly), written as the definition of each step with no blocking, fusion or
reordering beyond what the definition states; a matrix product is used as a
library primitive.  Sources, by page and section:

  [wiki]  "DFlash" wiki page (aisparkup.com): "Parallel drafting with block
          diffusion" (one forward pass drafts a whole block); "Conditioning on
          target-model features" items 1-3 (fuse features of several target
          layers with a light projection, inject the result into the KV cache
          of every draft layer, draft the next block in parallel) and its last
          paragraph (embedding and LM head are shared with the target);
          "Performance comparison" (greedy decoding, temperature 0; sampling at
          temperature 1).
  [faq]   z-lab/dflash overview page, FAQ on KV injection versus input fusion
          (the context goes straight into K/V without full token processing).
  [blog]  NVIDIA technical blog "Boost inference performance up to 15x on
          NVIDIA Blackwell using DFlash speculative decoding", section "How does
          DFlash speculative decoding work?" (verify accepts the longest valid
          prefix; the drafter predicts a block of masked future tokens in one
          forward pass; context features are injected into the key-value
          projections of the draft layers; the target's output distribution is
          preserved).

Readings where the pages are silent:
  R1 block = [anchor (last accepted token), mask x 15]; 15 drafted tokens.
  R3 context occupies positions 0..T-1, the block T..T+15, one RoPE frame.
  R4 the fusion is one linear map without bias or norm.
  R5 the context K/V use each draft layer's own W_k, W_v; no norm on the
     fused feature.
  R6 block K/V are transient, never appended to the cache.
  R7 attention is fully bidirectional over context + block (no mask).
  R8 pre-norm Llama-style layers: RMSNorm, GQA attention with rotate-half
     RoPE, SwiGLU MLP; final RMSNorm before the shared LM head.
  R12 argmax ties go to the lowest index.
  R13 no logits for slot 0 (15 LM-head rows per request).
  R18 draft i (slot i, i = 1..15) is compared with the target's prediction
      after slot i-1; the bonus is the target's prediction at the first
      mismatch (or after slot 15).
  R19 precision of a bf16 drafter: its weights, the target features it reads
      and its KV cache are bf16; every activation (fused feature, residual
      stream, norms, q/k/v, attention, SwiGLU, logits) is carried at full
      precision.  The cache is the one value the model itself writes in bf16,
      so `precision="bf16"` rounds (to nearest, ties to even, 8 significant
      bits) exactly the injected K and V; "exact" rounds nowhere.  f32 models
      use "exact".
  R20 the closed loop: after a verify with accept length a, the anchor and the
      a - 1 accepted drafts join the context -- the target's hidden features of
      block slots 0..a-1 are injected at positions T..T+a-1 -- and the bonus
      token is the next anchor.
  R21 the input-fusion variant [faq]: the fused feature is the drafter's input hidden
      state at each context position (in place of a token embedding), and the context
      rows run through the draft layers causally (row t attends to positions 0..t) before
      the block is drafted; each layer caches the K/V of the context rows, as stored
      values (bf16 for a bf16 drafter), and context rows attend to those stored values.
  R22 block sizes other than 16 (8 and 32): the block is [anchor, mask x (B - 1)] at
      positions T..T+B-1 and yields B - 1 drafts; everything else is unchanged.
"""
from __future__ import annotations

import math
from typing import Dict, List, Sequence

import numpy as np

try:  # torch tensors are accepted as inputs (the seeded generators produce bf16 tensors)
    import torch
except Exception:  # pragma: no cover
    torch = None

DRAFTS_PER_BLOCK = 15


def f64(x) -> np.ndarray:
    """Widen an input (numpy array or torch tensor, possibly bf16) to float64 exactly."""
    if torch is not None and isinstance(x, torch.Tensor):
        return x.detach().to(torch.float64).cpu().numpy()
    return np.asarray(x, dtype=np.float64)


# ------------------------------------------------------------------------------------------
# Building blocks
# ------------------------------------------------------------------------------------------

def round_bf16(x) -> np.ndarray:
    """Round to the nearest bfloat16 value (8 significant bits, ties to even), from the
    definition of the format: x = m * 2^e with m in [0.5, 1); keep round(m * 2^8) / 2^8.
    Valid for normal values below the bf16 maximum (no subnormal or overflow handling; the
    drafter's tensors stay many binades away from both limits)."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)
    return np.ldexp(np.round(np.ldexp(m, 8)), e - 8)


def store(x, precision: str) -> np.ndarray:
    """A value written to the KV cache (reading R19)."""
    return round_bf16(x) if precision == "bf16" else np.asarray(x, dtype=np.float64)


def precision_of(cfg, precision=None) -> str:
    if precision is not None:
        return precision
    return "bf16" if cfg.dtype == "bf16" else "exact"


def fuse_features(feats, w_fuse) -> np.ndarray:
    """Feature fusion [wiki, Conditioning item 1]: c[t] = W_fuse . X[t].

    feats [n, F] are the concatenated hidden states of several target layers;
    w_fuse [H, F].  A single linear map (reading R4)."""
    return f64(feats) @ f64(w_fuse).T


def rope(z: np.ndarray, pos, theta: float) -> np.ndarray:
    """Rotary position embedding, rotate-half pairing (reading R8).

    z [n, heads, d], pos [n].  For i < d/2 with angle a = pos * theta^(-2i/d):
      z'[i]       = z[i] cos a - z[i+d/2] sin a
      z'[i+d/2]   = z[i+d/2] cos a + z[i] sin a
    """
    z = np.asarray(z, dtype=np.float64)
    d = z.shape[-1]
    half = d // 2
    inv_freq = theta ** (-2.0 * np.arange(half, dtype=np.float64) / d)
    ang = np.asarray(pos, dtype=np.float64)[:, None, None] * inv_freq[None, None, :]
    c, s = np.cos(ang), np.sin(ang)
    lo, hi = z[..., :half], z[..., half:]
    return np.concatenate([lo * c - hi * s, hi * c + lo * s], axis=-1)


def inject_kv(c, pos, wk, wv, n_kv: int, head_dim: int, theta: float):
    """KV injection for one draft layer [wiki, Conditioning item 2; blog, How it works].

    The fused context feature c[t] goes through the layer's own K and V projections;
    K is rotated at the context position t (readings R3, R5).  Returns K, V [n, n_kv, d]."""
    c = np.asarray(c, dtype=np.float64)
    k = (c @ f64(wk).T).reshape(len(c), n_kv, head_dim)
    v = (c @ f64(wv).T).reshape(len(c), n_kv, head_dim)
    return rope(k, pos, theta), v


def rms_norm(z: np.ndarray, gamma, eps: float) -> np.ndarray:
    """RMSNorm(z; g) = z / sqrt(mean(z^2) + eps) * g over the last axis."""
    z = np.asarray(z, dtype=np.float64)
    return z / np.sqrt(np.mean(z * z, axis=-1, keepdims=True) + eps) * f64(gamma)


def attention(q: np.ndarray, keys: np.ndarray, vals: np.ndarray) -> np.ndarray:
    """Non-causal grouped-query attention, written as the explicit softmax (reading R7).

    q [R, n_q, d]; keys, vals [N, n_kv, d].  Query head h reads kv head
    h // (n_q / n_kv).  s_n = q . key_n / sqrt(d) over all N keys, no mask;
    p = exp(s - max s) / sum exp(s - max s); o = sum_n p_n val_n."""
    R, n_q, d = q.shape
    n_kv = keys.shape[1]
    group = n_q // n_kv
    out = np.empty((R, n_q, d), dtype=np.float64)
    for h in range(n_q):
        g = h // group
        s = q[:, h, :] @ keys[:, g, :].T / math.sqrt(d)      # [R, N]
        s = s - s.max(axis=1, keepdims=True)
        p = np.exp(s)
        p = p / p.sum(axis=1, keepdims=True)
        out[:, h, :] = p @ vals[:, g, :]
    return out


def causal_attention(q: np.ndarray, keys: np.ndarray, vals: np.ndarray) -> np.ndarray:
    """Causal grouped-query attention over one sequence (reading R21): q, keys, vals hold
    the same positions in order, [N, heads, d], and row t sees keys 0..t only.  Written as
    the explicit softmax over the allowed keys; disallowed keys get no weight."""
    N, n_q, d = q.shape
    group = n_q // keys.shape[1]
    allowed = np.tril(np.ones((N, N), dtype=bool))            # allowed[t, n] = n <= t
    out = np.empty((N, n_q, d), dtype=np.float64)
    for h in range(n_q):
        g = h // group
        s = q[:, h, :] @ keys[:, g, :].T / math.sqrt(d)        # [N, N]
        s = np.where(allowed, s, -np.inf)
        s = s - s.max(axis=1, keepdims=True)
        p = np.where(allowed, np.exp(s), 0.0)
        p = p / p.sum(axis=1, keepdims=True)
        out[:, h, :] = p @ vals[:, g, :]
    return out


def embed_rows(table, ids) -> np.ndarray:
    """Rows `ids` of the embedding table, widened to float64."""
    if torch is not None and isinstance(table, torch.Tensor):
        return f64(table[torch.as_tensor(np.asarray(ids), dtype=torch.long)])
    return f64(table)[np.asarray(ids)]


def silu(z: np.ndarray) -> np.ndarray:
    return z / (1.0 + np.exp(-z))


def top2(logits: np.ndarray):
    """Per row: (top-1 index, top-1 value, top-2 value); exact ties -> lowest index (R12)."""
    idx = np.argmax(logits, axis=-1)                  # numpy returns the first maximum
    v1 = np.take_along_axis(logits, idx[..., None], axis=-1)[..., 0]
    rest = logits.copy()
    np.put_along_axis(rest, idx[..., None], -np.inf, axis=-1)
    v2 = rest.max(axis=-1)
    return idx, v1, v2


# ------------------------------------------------------------------------------------------
# The draft step
# ------------------------------------------------------------------------------------------

def prefill_context(cfg, weights: Dict, feats, positions=None, precision=None):
    """Inject a whole context: fuse every position, then K/V for every layer.

    Returns per-layer lists K[l], V[l] of shape [T, n_kv, d] (contiguous per request;
    paging is a storage detail of the GPU cache)."""
    p = precision_of(cfg, precision)
    T = feats.shape[0]
    pos = np.arange(T) if positions is None else np.asarray(positions)
    c = fuse_features(feats, weights["w_fuse"])
    ks, vs = [], []
    for l in range(cfg.n_layers):
        k, v = inject_kv(c, pos, weights[f"wk.{l}"], weights[f"wv.{l}"], cfg.n_kv_heads,
                         cfg.head_dim, cfg.rope_theta)
        ks.append(store(k, p))
        vs.append(store(v, p))
    return ks, vs


def prefill_input_fusion(cfg, weights: Dict, feats, precision=None, want_unrounded=False):
    """The input-fusion variant's context prefill [faq: KV injection versus input fusion],
    for a fresh context at positions 0..T-1 (reading R21).

    The fused feature c[t] = W_fuse . X[t] is the drafter's input hidden state at context
    position t.  Every layer l takes the context rows as the block's rows are taken in
    draft_block -- RMSNorm, Q/K/V with RoPE at position t, attention, output projection,
    SwiGLU MLP, both residual adds -- except that attention is causal: row t attends to
    the layer's cached K/V of positions 0..t, i.e. the stored (bf16 for a bf16 drafter)
    values, its own included.  The result is each layer's cached K, V [T, n_kv, d]; the
    last layer's attention and MLP feed nothing the draft step reads and are not run.
    The draft step over this cache is draft_block, unchanged.  With want_unrounded, also
    returns each layer's K, V before they are stored (the values the cache rounds)."""
    p = precision_of(cfg, precision)
    H, d, nq, nkv = cfg.hidden, cfg.head_dim, cfg.n_q_heads, cfg.n_kv_heads
    T = feats.shape[0]
    pos = np.arange(T)
    x = fuse_features(feats, weights["w_fuse"])                    # [T, H] input rows
    ks, vs, ku, vu = [], [], [], []
    for l in range(cfg.n_layers):
        u = rms_norm(x, weights[f"attn_norm.{l}"], cfg.rms_eps)
        k_raw = rope((u @ f64(weights[f"wk.{l}"]).T).reshape(T, nkv, d), pos, cfg.rope_theta)
        v_raw = (u @ f64(weights[f"wv.{l}"]).T).reshape(T, nkv, d)
        k, v = store(k_raw, p), store(v_raw, p)
        ks.append(k)
        vs.append(v)
        ku.append(k_raw)
        vu.append(v_raw)
        if l + 1 == cfg.n_layers:
            break
        q = rope((u @ f64(weights[f"wq.{l}"]).T).reshape(T, nq, d), pos, cfg.rope_theta)
        o = causal_attention(q, k, v).reshape(T, nq * d)
        x = x + o @ f64(weights[f"wo.{l}"]).T
        u = rms_norm(x, weights[f"mlp_norm.{l}"], cfg.rms_eps)
        g = u @ f64(weights[f"w_gate.{l}"]).T
        up = u @ f64(weights[f"w_up.{l}"]).T
        x = x + (silu(g) * up) @ f64(weights[f"w_down.{l}"]).T
    return (ks, vs, ku, vu) if want_unrounded else (ks, vs)


def draft_block(cfg, weights: Dict, k_ctx: Sequence[np.ndarray], v_ctx: Sequence[np.ndarray],
                anchor: int, want_logits: bool = False, want_hidden: bool = False,
                precision=None) -> Dict:
    """One block-diffusion forward pass over [anchor, mask x 15] [wiki, Parallel drafting;
    blog, How it works], attending to the injected context K/V of every layer.

    k_ctx[l], v_ctx[l]: [T, n_kv, d] context entries of layer l (T may be 0).
    Returns draft ids [15] (argmax of the shared LM head over slots 1..15), the top-1 and
    top-2 logit values and their gap, and optionally the logits [15, V] and per-layer
    residual streams."""
    p = precision_of(cfg, precision)
    H, d, nq, nkv = cfg.hidden, cfg.head_dim, cfg.n_q_heads, cfg.n_kv_heads
    nb = cfg.block_size
    T = 0 if len(k_ctx) == 0 else k_ctx[0].shape[0]
    ids = np.array([anchor] + [cfg.mask_id] * (nb - 1))
    x = embed_rows(weights["embed"], ids)                          # shared embedding [wiki]
    pos = T + np.arange(nb)
    hidden = [x.copy()]
    for l in range(cfg.n_layers):
        u = rms_norm(x, weights[f"attn_norm.{l}"], cfg.rms_eps)
        q = rope((u @ f64(weights[f"wq.{l}"]).T).reshape(nb, nq, d), pos, cfg.rope_theta)
        k = rope((u @ f64(weights[f"wk.{l}"]).T).reshape(nb, nkv, d), pos, cfg.rope_theta)
        v = (u @ f64(weights[f"wv.{l}"]).T).reshape(nb, nkv, d)
        if T > 0:
            keys = np.concatenate([np.asarray(k_ctx[l], dtype=np.float64), k], axis=0)
            vals = np.concatenate([np.asarray(v_ctx[l], dtype=np.float64), v], axis=0)
        else:
            keys, vals = k, v
        o = attention(q, keys, vals).reshape(nb, nq * d)
        x = x + o @ f64(weights[f"wo.{l}"]).T
        u = rms_norm(x, weights[f"mlp_norm.{l}"], cfg.rms_eps)
        g = u @ f64(weights[f"w_gate.{l}"]).T
        up = u @ f64(weights[f"w_up.{l}"]).T
        x = x + (silu(g) * up) @ f64(weights[f"w_down.{l}"]).T
        hidden.append(x.copy())
    y = rms_norm(x[1:], weights["final_norm"], cfg.rms_eps)          # slots 1..15 (R13)
    logits = y @ f64(weights["lm_head"]).T                             # [15, V]
    idx, v1, v2 = top2(logits)
    out = {"ids": idx.astype(np.int32), "top1": v1, "top2": v2, "gap": v1 - v2}
    if want_logits:
        out["logits"] = logits
    if want_hidden:
        out["hidden"] = hidden
    return out


def near_tie(gap: np.ndarray, top1: np.ndarray, top2: np.ndarray, dtype: str) -> np.ndarray:
    """Positions whose top-1/top-2 gap is inside the parity tolerance: 1e-4 relative
    for fp32 storage, 2e-2 absolute for bf16 storage with fp32 accumulation."""
    if dtype == "f32":
        return gap < 1e-4 * np.maximum(np.abs(top1), np.abs(top2))
    return gap < 2e-2


# ------------------------------------------------------------------------------------------
# Verification
# ------------------------------------------------------------------------------------------

def verify_greedy(draft_ids, target_ids):
    """Greedy verification [blog, How it works: accept the longest valid prefix;
    wiki, Performance comparison: temperature 0].

    draft_ids [15]: d_1..d_15.  target_ids [16]: t_0..t_15, the target's argmax after
    consuming block slot j.  m = number of leading i with d_i == t_{i-1};
    accept_len = m + 1; the bonus token is t_m; emitted = d_1..d_m, t_m (R18)."""
    d = [int(x) for x in draft_ids]
    t = [int(x) for x in target_ids]
    m = 0
    while m < len(d) and d[m] == t[m]:
        m += 1
    emitted = d[:m] + [t[m]]
    return m + 1, t[m], emitted


def softmax(z) -> np.ndarray:
    z = np.asarray(z, dtype=np.float64)
    e = np.exp(z - z.max())
    return e / e.sum()


def inv_cdf(w: np.ndarray, u: float):
    """Smallest j with sum_{v<=j} w_v > u * sum_v w_v; if rounding leaves none, the last j
    with w_j > 0.  Also returns the distance from u*sum(w) to the nearest cumulative
    boundary, relative to sum(w) (used to excuse boundary near-ties)."""
    c = np.cumsum(w)
    total = c[-1]
    thr = u * total
    hits = np.nonzero(c > thr)[0]
    if len(hits):
        j = int(hits[0])
    else:
        j = int(np.nonzero(w > 0)[0][-1])
    lo = c[j - 1] if j > 0 else 0.0
    margin = min(abs(thr - lo), abs(c[j] - thr)) / total if total > 0 else 0.0
    return j, margin


def verify_sampled(draft_logits, target_logits, u_draft, u_accept, u_resample: float):
    """Temperature-1 speculative verification that preserves the target distribution
    [blog, How it works; wiki, Performance comparison (sampling at temperature 1)].

    The rule is the standard speculative accept/reject with residual resampling (the
    pages name the property, not the rule):
      q_i = softmax(draft_logits[i-1]), p_i = softmax(target_logits[i-1]), i = 1..15;
      d_i = InvCDF(q_i, u_draft[i-1]);
      for i = 1..15: accept d_i iff u_accept[i-1] * q_i(d_i) < p_i(d_i); at the first
      rejection emit InvCDF(max(0, p_i - q_i), u_resample) (p_i if that mass is 0) and
      stop with accept_len = i; if all 15 are accepted emit InvCDF(p_16, u_resample),
      accept_len = 16.
    Returns draft ids [15], accept_len, emitted tokens and the decision margins."""
    dl = f64(draft_logits)
    tl = f64(target_logits)
    nd = dl.shape[0]
    q = [softmax(dl[i]) for i in range(nd)]
    p = [softmax(tl[i]) for i in range(nd + 1)]
    drafts, margins = [], []
    for i in range(nd):
        j, mg = inv_cdf(q[i], float(u_draft[i]))
        drafts.append(j)
        margins.append(("draft", i, mg))
    emitted = []
    for i in range(nd):
        di = drafts[i]
        lhs = float(u_accept[i]) * q[i][di]
        rhs = p[i][di]
        margins.append(("accept", i, abs(lhs - rhs) / max(lhs, rhs, 1e-300)))
        if lhs < rhs:
            emitted.append(di)
            continue
        r = np.maximum(p[i] - q[i], 0.0)
        if not r.sum() > 0:
            r = p[i]
        x, mg = inv_cdf(r, float(u_resample))
        margins.append(("resample", i, mg))
        emitted.append(x)
        return {"draft_ids": np.array(drafts, dtype=np.int32), "accept_len": i + 1,
                "emitted": emitted, "margins": margins}
    x, mg = inv_cdf(p[nd], float(u_resample))
    margins.append(("bonus", nd, mg))
    emitted.append(x)
    return {"draft_ids": np.array(drafts, dtype=np.int32), "accept_len": nd + 1,
            "emitted": emitted, "margins": margins}


# ------------------------------------------------------------------------------------------
# One whole step (inject the newly accepted positions, draft, verify)
# ------------------------------------------------------------------------------------------

def draft_step(cfg, weights: Dict, k_ctx: List[np.ndarray], v_ctx: List[np.ndarray],
               new_feats, anchor: int, target_ids, precision=None) -> Dict:
    """Inject `new_feats` [n_new, F] at the positions after the current context, draft a
    block from the grown context, then greedily verify against `target_ids` [16]."""
    p = precision_of(cfg, precision)
    T0 = 0 if len(k_ctx) == 0 else k_ctx[0].shape[0]
    n_new = new_feats.shape[0]
    pos = T0 + np.arange(n_new)
    c = fuse_features(new_feats, weights["w_fuse"])
    ks, vs = [], []
    for l in range(cfg.n_layers):
        k, v = inject_kv(c, pos, weights[f"wk.{l}"], weights[f"wv.{l}"], cfg.n_kv_heads,
                         cfg.head_dim, cfg.rope_theta)
        k, v = store(k, p), store(v, p)
        if T0:
            k = np.concatenate([k_ctx[l], k], axis=0)
            v = np.concatenate([v_ctx[l], v], axis=0)
        ks.append(k)
        vs.append(v)
    dr = draft_block(cfg, weights, ks, vs, anchor, precision=p)
    acc, bonus, emitted = verify_greedy(dr["ids"], target_ids)
    dr.update({"accept_len": acc, "bonus": bonus, "emitted": emitted})
    return dr


# ------------------------------------------------------------------------------------------
# The closed speculative loop (several iterations)
# ------------------------------------------------------------------------------------------

def decode_loop(cfg, weights: Dict, k_ctx: List[np.ndarray], v_ctx: List[np.ndarray],
                anchor: int, block_feats: Sequence, target_ids_for, precision=None) -> Dict:
    """Drafting and verification alternating [blog, How it works: the drafter proposes a
    block, the target accepts the longest valid prefix, so one verification pass yields
    several tokens; wiki, Background].  Iteration i, with T the context length:
      1. draft a block from [anchor, mask x 15] at positions T..T+15;
      2. the target's ids for that block, target_ids_for(i, draft_ids) [16], verified
         greedily: accept_len a, bonus token;
      3. the anchor and the a - 1 accepted drafts join the context: the target's hidden
         features of block slots 0..a-1, block_feats[i][:a] ([16, F] per iteration), are
         fused and injected at positions T..T+a-1 (R20);
      4. T += a; the bonus token is the next anchor.
    Returns per-iteration records and the final context K/V."""
    p = precision_of(cfg, precision)
    ks = [np.asarray(k, dtype=np.float64) for k in k_ctx]
    vs = [np.asarray(v, dtype=np.float64) for v in v_ctx]
    T = 0 if len(ks) == 0 else ks[0].shape[0]
    records = []
    for i, feats in enumerate(block_feats):
        dr = draft_block(cfg, weights, ks, vs, anchor, precision=p)
        t = np.asarray(target_ids_for(i, dr["ids"]))
        acc, bonus, emitted = verify_greedy(dr["ids"], t)
        nk, nv = prefill_context(cfg, weights, feats[:acc], positions=T + np.arange(acc),
                                 precision=p)
        if T == 0 and len(ks) == 0:
            ks, vs = nk, nv
        else:
            ks = [np.concatenate([a, b], axis=0) for a, b in zip(ks, nk)]
            vs = [np.concatenate([a, b], axis=0) for a, b in zip(vs, nv)]
        records.append({"ids": dr["ids"], "gap": dr["gap"], "top1": dr["top1"],
                        "top2": dr["top2"], "target_ids": t, "accept_len": acc,
                        "bonus": bonus, "emitted": emitted, "ctx_len": T, "anchor": anchor})
        T += acc
        anchor = bonus
    return {"iterations": records, "k_ctx": ks, "v_ctx": vs, "ctx_len": T, "anchor": anchor}

