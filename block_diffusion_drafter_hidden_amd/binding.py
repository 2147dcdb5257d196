"""ctypes binding of libdflash.so (argument marshalling only).

Every computation of the draft step runs in the HIP kernels of libdflash.so; this module
only turns torch device tensors into pointers, fills the C structs and checks status
codes.  Importing it fails loudly if the library has not been built.
"""
from __future__ import annotations

import ctypes as C
import os
from dataclasses import dataclass
from typing import Dict, Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdflash.so")

DFLASH_F32, DFLASH_BF16 = 0, 1
STATUS = {0: "ok", -1: "invalid argument", -2: "unsupported shape or dtype",
          -3: "workspace or packed buffer too small", -4: "HIP launch error"}

# Symbols declared in include/dflash.h.
EXPORTS = (
    "dflash_packed_weights_size", "dflash_pack_weights", "dflash_workspace_size",
    "dflash_workspace_init", "dflash_fuse_inject_kv", "dflash_draft_block",
    "dflash_lm_head_argmax",
    "dflash_verify_accept", "dflash_advance", "dflash_verify_sampled_workspace_size",
    "dflash_verify_accept_sampled", "dflash_error_string", "dflash_noalloc_scratch_bytes",
    "dflash_draft_block_noalloc", "dflash_prefill_workspace_size", "dflash_prefill_input_fusion",
)


class DflashError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {STATUS.get(status, status)} ({status})")
        self.status = status


class Config(C.Structure):
    _fields_ = [("n_layers", C.c_int32), ("hidden", C.c_int32), ("n_q_heads", C.c_int32),
                ("n_kv_heads", C.c_int32), ("head_dim", C.c_int32),
                ("intermediate", C.c_int32), ("vocab", C.c_int32), ("feat_dim", C.c_int32),
                ("block_size", C.c_int32), ("page_size", C.c_int32),
                ("mask_token_id", C.c_int32), ("rope_theta", C.c_float),
                ("rms_eps", C.c_float), ("dtype", C.c_int32)]


class Weights(C.Structure):
    _fields_ = [("w_fuse", C.c_void_p), ("lm_head", C.c_void_p), ("final_norm", C.c_void_p),
                ("attn_norm", C.POINTER(C.c_void_p)), ("wq", C.POINTER(C.c_void_p)),
                ("wk", C.POINTER(C.c_void_p)), ("wv", C.POINTER(C.c_void_p)),
                ("wo", C.POINTER(C.c_void_p)), ("mlp_norm", C.POINTER(C.c_void_p)),
                ("w_gate", C.POINTER(C.c_void_p)), ("w_up", C.POINTER(C.c_void_p)),
                ("w_down", C.POINTER(C.c_void_p))]


class KVCache(C.Structure):
    _fields_ = [("k_pool", C.c_void_p), ("v_pool", C.c_void_p), ("block_table", C.c_void_p),
                ("ctx_lens", C.c_void_p), ("num_pages", C.c_int32),
                ("max_pages_per_seq", C.c_int32)]


_lib = None


def load_library(path: str = LIB_PATH) -> C.CDLL:
    """Load libdflash.so; raises if it is missing (no fallback path exists)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built; run `python -m block_diffusion_drafter_hidden_amd.build`")
    lib = C.CDLL(path)
    P, S, I32, SZ = C.c_void_p, C.c_int, C.c_int32, C.c_size_t
    sig = {
        "dflash_packed_weights_size": (SZ, [P]),
        "dflash_pack_weights": (S, [P, P, P, SZ, P]),
        "dflash_workspace_size": (SZ, [P, I32, I32, I32]),
        "dflash_workspace_init": (S, [P, SZ, P]),
        "dflash_fuse_inject_kv": (S, [P, P, P, P, P, P, I32, P, SZ, P]),
        "dflash_draft_block": (S, [P, P, P, P, P, I32, P, P, P, P, SZ, P]),
        "dflash_lm_head_argmax": (S, [P, P, P, I32, P, P, P, SZ, P]),
        "dflash_verify_accept": (S, [P, P, I32, I32, P, P, P, P]),
        "dflash_advance": (S, [P, P, I32, I32, I32, P, P, P, P, P]),
        "dflash_verify_sampled_workspace_size": (SZ, [I32, I32]),
        "dflash_verify_accept_sampled": (S, [P, P, P, P, P, I32, I32, P, P, P, P, SZ, P]),
        "dflash_error_string": (C.c_char_p, [S]),
        "dflash_noalloc_scratch_bytes": (SZ, []),
        "dflash_draft_block_noalloc": (S, [P, P, P, P, P, I32, P, P, P, P]),
        "dflash_prefill_workspace_size": (SZ, [P, I32, I32]),
        "dflash_prefill_input_fusion": (S, [P, P, P, P, I32, I32, P, SZ, P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    return C.c_void_p(t.data_ptr())


def _model_dtype(ccfg: "Config"):
    return torch.bfloat16 if ccfg.dtype == DFLASH_BF16 else torch.float32


def _arg(t, name: str, dtype, shape=None, device=None, optional: bool = False):
    """Check one tensor argument before its pointer crosses the ABI: a contiguous tensor
    on a GPU (on `device` when given) with the dtype and shape the library reads.  Raises
    ValueError; the library is not called."""
    if t is None:
        if optional:
            return None
        raise ValueError(f"{name}: required")
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name}: expected a torch tensor, got {type(t).__name__}")
    if not t.is_cuda:
        raise ValueError(f"{name}: must be a GPU tensor (got {t.device})")
    if device is not None and t.device != device:
        raise ValueError(f"{name}: on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if shape is not None:
        want = tuple(shape)
        if t.dim() != len(want) or any(w is not None and int(a) != w
                                       for a, w in zip(t.shape, want)):
            raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {want}")
    return t


def _nbytes(t: torch.Tensor) -> int:
    return t.numel() * t.element_size()


def _stream(stream=None):
    if stream is None:
        stream = torch.cuda.current_stream()
    return C.c_void_p(stream.cuda_stream)


def _check(status: int, what: str) -> None:
    if status != 0:
        raise DflashError(status, what)


def make_config(cfg) -> Config:
    """C config from a workloads.DrafterConfig (or any object with the same fields)."""
    return Config(cfg.n_layers, cfg.hidden, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim,
                  cfg.intermediate, cfg.vocab, cfg.feat_dim, cfg.block_size, cfg.page_size,
                  cfg.mask_id, float(cfg.rope_theta), float(cfg.rms_eps),
                  DFLASH_BF16 if cfg.dtype == "bf16" else DFLASH_F32)


# ---------------------------------------------------------------------------------------
# Thin wrappers with the ABI's names
# ---------------------------------------------------------------------------------------

def packed_weights_size(ccfg: Config) -> int:
    return int(load_library().dflash_packed_weights_size(C.byref(ccfg)))


def pack_weights(ccfg: Config, w: Dict[str, torch.Tensor], n_layers: int,
                 packed: torch.Tensor, stream=None) -> None:
    arr = lambda key: (C.c_void_p * n_layers)(*[w[f"{key}.{l}"].data_ptr() for l in range(n_layers)])
    keep = {k: arr(k) for k in ("attn_norm", "wq", "wk", "wv", "wo", "mlp_norm", "w_gate",
                                "w_up", "w_down")}
    cw = Weights(w["w_fuse"].data_ptr(), w["lm_head"].data_ptr(), w["final_norm"].data_ptr(),
                 *[C.cast(keep[k], C.POINTER(C.c_void_p)) for k in
                   ("attn_norm", "wq", "wk", "wv", "wo", "mlp_norm", "w_gate", "w_up", "w_down")])
    _check(load_library().dflash_pack_weights(C.byref(ccfg), C.byref(cw), _ptr(packed),
                                              packed.numel() * packed.element_size(),
                                              _stream(stream)), "dflash_pack_weights")


def workspace_size(ccfg: Config, max_batch: int, max_inject_rows: int, max_ctx: int) -> int:
    return int(load_library().dflash_workspace_size(C.byref(ccfg), max_batch, max_inject_rows,
                                                    max_ctx))


def workspace_init(ws: torch.Tensor, stream=None) -> None:
    _check(load_library().dflash_workspace_init(_ptr(ws), ws.numel() * ws.element_size(),
                                                _stream(stream)), "dflash_workspace_init")


def make_cache(k_pool, v_pool, block_table, ctx_lens, num_pages, max_pages) -> KVCache:
    dev = _arg(k_pool, "k_pool", None).device
    _arg(v_pool, "v_pool", k_pool.dtype, tuple(k_pool.shape[:2]) + (None,) * (k_pool.dim() - 2), dev)
    if k_pool.dim() != 5 or k_pool.shape[1] != num_pages or k_pool.shape[3] != 16:
        raise ValueError(f"k_pool: shape {tuple(k_pool.shape)}, expected [L, {num_pages}, n_kv, 16, d]")
    _arg(block_table, "block_table", torch.int32, (None, max_pages), dev)
    _arg(ctx_lens, "ctx_lens", torch.int32, (block_table.shape[0],), dev)
    return KVCache(k_pool.data_ptr(), v_pool.data_ptr(), block_table.data_ptr(),
                   ctx_lens.data_ptr(), num_pages, max_pages)


def fuse_inject_kv(ccfg: Config, packed, cache: KVCache, feats, seq_idx, pos, ws,
                   stream=None) -> None:
    dev = _arg(ws, "ws", torch.uint8, (None,)).device
    _arg(packed, "packed", torch.uint8, (None,), dev)
    n_tok = int(_arg(feats, "feats", _model_dtype(ccfg), (None, ccfg.feat_dim), dev).shape[0])
    _arg(seq_idx, "seq_idx", torch.int32, (n_tok,), dev)
    _arg(pos, "pos", torch.int32, (n_tok,), dev)
    _check(load_library().dflash_fuse_inject_kv(
        C.byref(ccfg), _ptr(packed), C.byref(cache), _ptr(feats), _ptr(seq_idx), _ptr(pos),
        n_tok, _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)),
        "dflash_fuse_inject_kv")


def draft_block(ccfg: Config, packed, embed, cache: KVCache, anchor_ids, draft_ids, ws,
                logits_out=None, stream=None, top2_gap=None) -> None:
    dev = _arg(ws, "ws", torch.uint8, (None,)).device
    _arg(packed, "packed", torch.uint8, (None,), dev)
    _arg(embed, "embed", _model_dtype(ccfg), (ccfg.vocab, ccfg.hidden), dev)
    batch = int(_arg(anchor_ids, "anchor_ids", torch.int32, (None,), dev).shape[0])
    nd = ccfg.block_size - 1
    _arg(draft_ids, "draft_ids", torch.int32, (batch, nd), dev)
    _arg(logits_out, "logits_out", torch.float32, (batch, nd, ccfg.vocab), dev, optional=True)
    _arg(top2_gap, "top2_gap", torch.float32, (batch, nd), dev, optional=True)
    _check(load_library().dflash_draft_block(
        C.byref(ccfg), _ptr(packed), _ptr(embed), C.byref(cache), _ptr(anchor_ids), batch,
        _ptr(draft_ids), _ptr(top2_gap), _ptr(logits_out), _ptr(ws), _nbytes(ws),
        _stream(stream)), "dflash_draft_block")


def noalloc_scratch_bytes() -> int:
    return int(load_library().dflash_noalloc_scratch_bytes())


def draft_block_noalloc(ccfg: Config, packed, embed, cache: KVCache, anchor_ids, draft_ids,
                        logits_out=None, stream=None, top2_gap=None) -> None:
    """dflash_draft_block_noalloc: the draft step on the library's own scratch array."""
    dev = _arg(packed, "packed", torch.uint8, (None,)).device
    _arg(embed, "embed", _model_dtype(ccfg), (ccfg.vocab, ccfg.hidden), dev)
    batch = int(_arg(anchor_ids, "anchor_ids", torch.int32, (None,), dev).shape[0])
    nd = ccfg.block_size - 1
    _arg(draft_ids, "draft_ids", torch.int32, (batch, nd), dev)
    _arg(logits_out, "logits_out", torch.float32, (batch, nd, ccfg.vocab), dev, optional=True)
    _arg(top2_gap, "top2_gap", torch.float32, (batch, nd), dev, optional=True)
    _check(load_library().dflash_draft_block_noalloc(
        C.byref(ccfg), _ptr(packed), _ptr(embed), C.byref(cache), _ptr(anchor_ids), batch,
        _ptr(draft_ids), _ptr(top2_gap), _ptr(logits_out), _stream(stream)),
        "dflash_draft_block_noalloc")


def lm_head_argmax(ccfg: Config, packed, y, ids_out, ws, logits_out=None, stream=None) -> None:
    dev = _arg(ws, "ws", torch.uint8, (None,)).device
    _arg(packed, "packed", torch.uint8, (None,), dev)
    rows = int(_arg(y, "y", torch.float32, (None, ccfg.hidden), dev).shape[0])
    _arg(ids_out, "ids_out", torch.int32, (rows,), dev)
    _arg(logits_out, "logits_out", torch.float32, (rows, ccfg.vocab), dev, optional=True)
    _check(load_library().dflash_lm_head_argmax(
        C.byref(ccfg), _ptr(packed), _ptr(y), rows, _ptr(ids_out), _ptr(logits_out), _ptr(ws),
        ws.numel() * ws.element_size(), _stream(stream)), "dflash_lm_head_argmax")


def verify_accept(draft_ids, target_ids, accept_len, bonus, emitted=None, stream=None) -> None:
    """Greedy verify; the block size B is taken from target_ids [batch, B]."""
    batch, nb = _arg(target_ids, "target_ids", torch.int32, (None, None)).shape
    dev = target_ids.device
    _arg(draft_ids, "draft_ids", torch.int32, (batch, nb - 1), dev)
    _arg(accept_len, "accept_len", torch.int32, (batch,), dev)
    _arg(bonus, "bonus", torch.int32, (batch,), dev)
    _arg(emitted, "emitted", torch.int32, (batch, nb), dev, optional=True)
    _check(load_library().dflash_verify_accept(
        _ptr(draft_ids), _ptr(target_ids), int(batch), int(nb), _ptr(accept_len), _ptr(bonus),
        _ptr(emitted), _stream(stream)), "dflash_verify_accept")


def advance(accept_len, bonus, max_ctx: int, ctx_lens, anchor_ids, inject_seq, inject_pos,
            stream=None, block_size: int = 16) -> None:
    batch = int(_arg(accept_len, "accept_len", torch.int32, (None,)).shape[0])
    dev = accept_len.device
    for name, t, shp in (("bonus", bonus, (batch,)), ("ctx_lens", ctx_lens, (batch,)),
                         ("anchor_ids", anchor_ids, (batch,)),
                         ("inject_seq", inject_seq, (batch * block_size,)),
                         ("inject_pos", inject_pos, (batch * block_size,))):
        _arg(t, name, torch.int32, shp, dev)
    _check(load_library().dflash_advance(
        _ptr(accept_len), _ptr(bonus), batch, int(block_size), int(max_ctx), _ptr(ctx_lens),
        _ptr(anchor_ids), _ptr(inject_seq), _ptr(inject_pos), _stream(stream)),
        "dflash_advance")


def prefill_workspace_size(ccfg: Config, max_tok: int, max_ctx: int) -> int:
    return int(load_library().dflash_prefill_workspace_size(C.byref(ccfg), max_tok, max_ctx))


def prefill_input_fusion(ccfg: Config, packed, cache: KVCache, feats, seq: int, ws,
                         stream=None) -> None:
    """dflash_prefill_input_fusion: request `seq`'s next feats.shape[0] context rows."""
    dev = _arg(ws, "ws", torch.uint8, (None,)).device
    _arg(packed, "packed", torch.uint8, (None,), dev)
    n_tok = int(_arg(feats, "feats", _model_dtype(ccfg), (None, ccfg.feat_dim), dev).shape[0])
    _check(load_library().dflash_prefill_input_fusion(
        C.byref(ccfg), _ptr(packed), C.byref(cache), _ptr(feats), int(seq), n_tok, _ptr(ws),
        _nbytes(ws), _stream(stream)), "dflash_prefill_input_fusion")


def verify_sampled_workspace_size(batch: int, vocab: int) -> int:
    return int(load_library().dflash_verify_sampled_workspace_size(batch, vocab))


def verify_accept_sampled(draft_logits, target_logits, u_draft, u_accept, u_resample,
                          draft_ids, accept_len, emitted, ws, stream=None) -> None:
    batch, _, vocab = _arg(draft_logits, "draft_logits", torch.float32, (None, 15, None)).shape
    dev = draft_logits.device
    _arg(target_logits, "target_logits", torch.float32, (batch, 16, vocab), dev)
    _arg(u_draft, "u_draft", torch.float32, (batch, 15), dev)
    _arg(u_accept, "u_accept", torch.float32, (batch, 15), dev)
    _arg(u_resample, "u_resample", torch.float32, (batch,), dev)
    _arg(draft_ids, "draft_ids", torch.int32, (batch, 15), dev)
    _arg(accept_len, "accept_len", torch.int32, (batch,), dev)
    _arg(emitted, "emitted", torch.int32, (batch, 16), dev)
    _arg(ws, "ws", torch.uint8, (None,), dev)
    _check(load_library().dflash_verify_accept_sampled(
        _ptr(draft_logits), _ptr(target_logits), _ptr(u_draft), _ptr(u_accept),
        _ptr(u_resample), int(batch), int(vocab), _ptr(draft_ids), _ptr(accept_len),
        _ptr(emitted), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)),
        "dflash_verify_accept_sampled")


def error_string(status: int) -> str:
    return load_library().dflash_error_string(status).decode()


# ---------------------------------------------------------------------------------------
# Device-memory holder for one drafter (torch owns the memory; the library fills it)
# ---------------------------------------------------------------------------------------

@dataclass
class PagedCache:
    k_pool: torch.Tensor          # [L, num_pages, n_kv, 16, d]
    v_pool: torch.Tensor          # [L, num_pages, n_kv, d, 16] (pages transposed)
    block_table: torch.Tensor     # [B, max_pages] int32
    ctx_lens: torch.Tensor        # [B] int32
    num_pages: int
    max_pages: int

    def c(self) -> KVCache:
        return make_cache(self.k_pool, self.v_pool, self.block_table, self.ctx_lens,
                          self.num_pages, self.max_pages)


class Drafter:
    """Packed weights + workspace of one drafter on one device."""

    def __init__(self, cfg, weights_dev: Dict[str, torch.Tensor], max_batch: int,
                 max_ctx: int, max_inject_rows: int = 256, device="cuda"):
        self.cfg = cfg
        self.ccfg = make_config(cfg)
        self.device = torch.device(device)
        n = packed_weights_size(self.ccfg)
        if n == 0:
            raise DflashError(-2, "dflash_packed_weights_size")
        self.packed = torch.empty(n, dtype=torch.uint8, device=self.device)
        pack_weights(self.ccfg, weights_dev, cfg.n_layers, self.packed)
        self.embed = weights_dev["embed"]
        self.ws_bytes = workspace_size(self.ccfg, max_batch, max_inject_rows, max_ctx)
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device=self.device)
        workspace_init(self.ws)

    def sibling(self, max_batch: int, max_ctx: int, max_inject_rows: int = 256,
                block_size: Optional[int] = None) -> "Drafter":
        """Another drafter over the same packed weights with its own workspace (for a
        different batch or context bound, or another block size: the packed weights do not
        depend on it)."""
        d = object.__new__(Drafter)
        d.cfg, d.ccfg, d.device, d.packed, d.embed = (self.cfg, self.ccfg, self.device,
                                                       self.packed, self.embed)
        if block_size is not None and block_size != self.cfg.block_size:
            from dataclasses import replace
            d.cfg = replace(self.cfg, block_size=block_size)
            d.ccfg = make_config(d.cfg)
        d.ws_bytes = workspace_size(d.ccfg, max_batch, max_inject_rows, max_ctx)
        d.ws = torch.empty(d.ws_bytes, dtype=torch.uint8, device=self.device)
        workspace_init(d.ws)
        return d

    def new_cache(self, block_table, ctx_lens, num_pages: int) -> PagedCache:
        cfg = self.cfg
        dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
        k_shape = (cfg.n_layers, num_pages, cfg.n_kv_heads, cfg.page_size, cfg.head_dim)
        v_shape = (cfg.n_layers, num_pages, cfg.n_kv_heads, cfg.head_dim, cfg.page_size)
        bt = torch.as_tensor(block_table, dtype=torch.int32).to(self.device).contiguous()
        cl = torch.as_tensor(ctx_lens, dtype=torch.int32).to(self.device).contiguous()
        return PagedCache(torch.zeros(k_shape, dtype=dt, device=self.device),
                          torch.zeros(v_shape, dtype=dt, device=self.device), bt, cl,
                          num_pages, int(bt.shape[1]))

    def inject(self, cache: PagedCache, feats, seq_idx, pos, stream=None) -> None:
        fuse_inject_kv(self.ccfg, self.packed, cache.c(), feats, seq_idx, pos, self.ws, stream)

    def draft(self, cache: PagedCache, anchor_ids, draft_ids, logits_out=None,
              stream=None, top2_gap=None) -> None:
        draft_block(self.ccfg, self.packed, self.embed, cache.c(), anchor_ids, draft_ids,
                    self.ws, logits_out, stream, top2_gap)

    def advance(self, cache: PagedCache, accept_len, bonus, anchor_ids, inject_seq,
                inject_pos, stream=None) -> None:
        advance(accept_len, bonus, cache.max_pages * self.cfg.page_size, cache.ctx_lens,
                anchor_ids, inject_seq, inject_pos, stream, block_size=self.cfg.block_size)

    def prefill_input_fusion(self, cache: PagedCache, feats, seq: int, ws=None,
                             stream=None) -> None:
        """Input-fusion context prefill of request `seq` (see dflash_prefill_input_fusion);
        `ws` defaults to a workspace sized for feats on first use."""
        if ws is None:
            need = prefill_workspace_size(self.ccfg, int(feats.shape[0]),
                                          cache.max_pages * self.cfg.page_size)
            if getattr(self, "_pf_ws", None) is None or self._pf_ws.numel() < need:
                self._pf_ws = torch.empty(need, dtype=torch.uint8, device=self.device)
                workspace_init(self._pf_ws)
            ws = self._pf_ws
        prefill_input_fusion(self.ccfg, self.packed, cache.c(), feats, seq, ws, stream)
