"""An independent float64 PyTorch-CPU transformer used only to pin the oracle.

It is written differently from the oracle on purpose: library layers
(F.linear, F.rms_norm, F.scaled_dot_product_attention, F.silu) and RoPE as a
complex rotation (z_lo + i z_hi) * exp(i pos w), so a slip in the oracle's
explicit formulas (a dropped gain, a swapped sign, a transposed operand, a
wrong head grouping) shows up as a mismatch.
"""
import numpy as np
import torch
import torch.nn.functional as F


def _t(x):
    if isinstance(x, torch.Tensor):
        return x.detach().to(torch.float64)
    return torch.as_tensor(np.asarray(x), dtype=torch.float64)


def rope_complex(z: torch.Tensor, pos: torch.Tensor, theta: float) -> torch.Tensor:
    """z [n, heads, d]; rotate (z[:d/2] + i z[d/2:]) by pos * theta^(-2i/d)."""
    d = z.shape[-1]
    half = d // 2
    w = theta ** (-torch.arange(0, half, dtype=torch.float64) * 2.0 / d)
    rot = torch.polar(torch.ones(len(pos), 1, half, dtype=torch.float64),
                      pos.to(torch.float64)[:, None, None] * w[None, None, :])
    zc = torch.complex(z[..., :half], z[..., half:]) * rot
    return torch.cat([zc.real, zc.imag], dim=-1)


def _bf(x: torch.Tensor, on: bool) -> torch.Tensor:
    return x.float().to(torch.bfloat16).to(torch.float64) if on else x


def context_kv(cfg, weights, feats, bf16: bool = False):
    """Injected K/V of every layer for context features [T, F] (positions 0..T-1); with
    `bf16`, the cached values are cast to bf16 as a bf16 drafter's cache holds them."""
    T = feats.shape[0]
    c = F.linear(_t(feats), _t(weights["w_fuse"]))
    pos = torch.arange(T)
    ks, vs = [], []
    for l in range(cfg.n_layers):
        k = F.linear(c, _t(weights[f"wk.{l}"])).view(T, cfg.n_kv_heads, cfg.head_dim)
        v = F.linear(c, _t(weights[f"wv.{l}"])).view(T, cfg.n_kv_heads, cfg.head_dim)
        ks.append(_bf(rope_complex(k, pos, cfg.rope_theta), bf16))
        vs.append(_bf(v, bf16))
    return ks, vs


def draft_logits(cfg, weights, k_ctx, v_ctx, anchor: int) -> torch.Tensor:
    """Logits [15, V] of the block-diffusion pass, float64."""
    nb, d = cfg.block_size, cfg.head_dim
    nq, nkv = cfg.n_q_heads, cfg.n_kv_heads
    T = 0 if len(k_ctx) == 0 else int(np.asarray(k_ctx[0]).shape[0])
    ids = torch.tensor([anchor] + [cfg.mask_id] * (nb - 1))
    x = F.embedding(ids, _t(weights["embed"]))
    pos = torch.arange(T, T + nb)
    for l in range(cfg.n_layers):
        u = F.rms_norm(x, (cfg.hidden,), _t(weights[f"attn_norm.{l}"]), eps=cfg.rms_eps)
        q = rope_complex(F.linear(u, _t(weights[f"wq.{l}"])).view(nb, nq, d), pos, cfg.rope_theta)
        k = rope_complex(F.linear(u, _t(weights[f"wk.{l}"])).view(nb, nkv, d), pos, cfg.rope_theta)
        v = F.linear(u, _t(weights[f"wv.{l}"])).view(nb, nkv, d)
        if T:
            k = torch.cat([_t(k_ctx[l]), k], 0)
            v = torch.cat([_t(v_ctx[l]), v], 0)
        kk = k.repeat_interleave(nq // nkv, dim=1).transpose(0, 1).contiguous()
        vv = v.repeat_interleave(nq // nkv, dim=1).transpose(0, 1).contiguous()
        o = F.scaled_dot_product_attention(q.transpose(0, 1).contiguous(), kk, vv)
        x = x + F.linear(o.transpose(0, 1).reshape(nb, nq * d), _t(weights[f"wo.{l}"]))
        u = F.rms_norm(x, (cfg.hidden,), _t(weights[f"mlp_norm.{l}"]), eps=cfg.rms_eps)
        h = F.silu(F.linear(u, _t(weights[f"w_gate.{l}"]))) * F.linear(u, _t(weights[f"w_up.{l}"]))
        x = x + F.linear(h, _t(weights[f"w_down.{l}"]))
    y = F.rms_norm(x[1:], (cfg.hidden,), _t(weights["final_norm"]), eps=cfg.rms_eps)
    return F.linear(y, _t(weights["lm_head"]))


def input_fusion_kv(cfg, weights, feats, bf16: bool = False):
    """Cached K/V of every layer when the fused features are the drafter's input rows and
    the context runs causally through the layers (positions 0..T-1).  With `bf16` the
    cached values are cast to bf16 and the context rows attend to the cast values."""
    T, d = feats.shape[0], cfg.head_dim
    nq, nkv = cfg.n_q_heads, cfg.n_kv_heads
    x = F.linear(_t(feats), _t(weights["w_fuse"]))
    pos = torch.arange(T)
    ks, vs = [], []
    for l in range(cfg.n_layers):
        u = F.rms_norm(x, (cfg.hidden,), _t(weights[f"attn_norm.{l}"]), eps=cfg.rms_eps)
        k = _bf(rope_complex(F.linear(u, _t(weights[f"wk.{l}"])).view(T, nkv, d), pos,
                             cfg.rope_theta), bf16)
        v = _bf(F.linear(u, _t(weights[f"wv.{l}"])).view(T, nkv, d), bf16)
        ks.append(k)
        vs.append(v)
        q = rope_complex(F.linear(u, _t(weights[f"wq.{l}"])).view(T, nq, d), pos, cfg.rope_theta)
        kk = k.repeat_interleave(nq // nkv, dim=1).transpose(0, 1).contiguous()
        vv = v.repeat_interleave(nq // nkv, dim=1).transpose(0, 1).contiguous()
        o = F.scaled_dot_product_attention(q.transpose(0, 1).contiguous(), kk, vv, is_causal=True)
        x = x + F.linear(o.transpose(0, 1).reshape(T, nq * d), _t(weights[f"wo.{l}"]))
        u = F.rms_norm(x, (cfg.hidden,), _t(weights[f"mlp_norm.{l}"]), eps=cfg.rms_eps)
        h = F.silu(F.linear(u, _t(weights[f"w_gate.{l}"]))) * F.linear(u, _t(weights[f"w_up.{l}"]))
        x = x + F.linear(h, _t(weights[f"w_down.{l}"]))
    return ks, vs
