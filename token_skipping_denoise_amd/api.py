"""Thin torch-facing binding of libdllm (argument marshalling only).

Every step of the denoising path runs in the HIP kernels behind the C ABI;
this module only allocates device memory with torch, passes raw pointers and
the current HIP stream, and checks the returned status.
"""
from __future__ import annotations

import ctypes

import torch

from . import _ffi
from ._ffi import (DLLM_BF16, DLLM_F32, FORCE_EXCLUDED, FORCE_NONE, FORCE_ON, SEL_THRESH_CAP, SEL_TOPK,  # noqa: F401
                   SEL_UNLOCKED, UNMASK_CONF, UNMASK_FORCED, VAR_COS, VAR_KL, VAR_L1N, VAR_L2REL, VAR_NONE)


class DllmError(RuntimeError):
    pass


def _lib():
    return _ffi.load()


def _check(status: int, what: str):
    if status != 0:
        msg = _lib().dllm_status_string(status).decode()
        raise DllmError(f"{what}: {msg} (status {status})")


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return DLLM_F32
    if t.dtype == torch.bfloat16:
        return DLLM_BF16
    raise DllmError(f"unsupported dtype {t.dtype}")


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise DllmError("tensor must be on the GPU")
    if not t.is_contiguous():
        raise DllmError("tensor must be contiguous")
    return t.data_ptr()


def _stream(device=None) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def version() -> int:
    return _lib().dllm_version()


def score_cfg(alpha=0.5, conf_inverted=False, var=VAR_L1N, sel=SEL_TOPK, k=1, tau=0.0) -> _ffi.ScoreCfg:
    return _ffi.ScoreCfg(float(alpha), int(bool(conf_inverted)), int(var), int(sel), int(k), float(tau))


def score_select(h_cur, h_prev, conf_prev, cfg: _ffi.ScoreCfg, *, kl_prev=None, force=None, k_max=None,
                 h_next=None):
    """Scores [B,S] fp32, idx [B,k_max] int32, n_active [B] int32 from h_cur/h_prev [B,S,w]."""
    B, S, w = h_cur.shape
    k_max = int(k_max if k_max is not None else (S if cfg.sel == SEL_UNLOCKED else max(cfg.k, 1)))
    dev = h_cur.device
    score = torch.empty((B, S), dtype=torch.float32, device=dev)
    idx = torch.empty((B, k_max), dtype=torch.int32, device=dev)
    n_act = torch.empty((B,), dtype=torch.int32, device=dev)
    st = _lib().dllm_score_select(_ptr(h_cur), _ptr(h_prev), _ptr(h_next), _dtype_code(h_cur), _ptr(conf_prev),
                                  _ptr(kl_prev), _ptr(force), B, S, w, ctypes.byref(cfg), _ptr(score), _ptr(idx),
                                  _ptr(n_act), k_max, _stream(dev))
    _check(st, "dllm_score_select")
    return score, idx, n_act


def gather_rows(src, idx, n_active):
    """src [B,S,w] -> [B*k_max, w] (rows of dead slots unspecified)."""
    B, S, w = src.shape
    k_max = idx.shape[1]
    dst = torch.empty((B * k_max, w), dtype=src.dtype, device=src.device)
    st = _lib().dllm_gather_rows(_ptr(src), _ptr(idx), _ptr(n_active), B, S, k_max, w, _dtype_code(src), _ptr(dst),
                                 _stream(src.device))
    _check(st, "dllm_gather_rows")
    return dst


def scatter_rows(src, idx, n_active, dst):
    """src [B*k_max, w] -> dst [B,S,w] at the active positions (in place)."""
    B, S, w = dst.shape
    k_max = idx.shape[1]
    st = _lib().dllm_scatter_rows(_ptr(src), _ptr(idx), _ptr(n_active), B, S, k_max, w, _dtype_code(dst), _ptr(dst),
                                  _stream(dst.device))
    _check(st, "dllm_scatter_rows")
    return dst


def confidence_kl(logits, row_pos, conf, argmax, *, kl=None, logits_prev=None, exclude_id=-1, have_prev=False):
    """logits_prev: fp32 or bf16 [B*S, V] state (its dtype selects the state precision), or None."""
    R, V = logits.shape
    prev_dtype = DLLM_F32
    if logits_prev is not None:
        if logits_prev.dtype not in (torch.float32, torch.bfloat16):
            raise DllmError("logits_prev must be float32 or bfloat16")
        prev_dtype = _dtype_code(logits_prev)
    st = _lib().dllm_confidence_kl(_ptr(logits), _ptr(logits_prev), prev_dtype, _ptr(row_pos), R, V, int(exclude_id),
                                   int(bool(have_prev)), _ptr(conf), _ptr(argmax), _ptr(kl), _stream(logits.device))
    _check(st, "dllm_confidence_kl")


def dus_mark(force, lo: int, block: int, round: int, *, a: int = 2, rounds: int = 0, mark: int = FORCE_ON):
    """Marks the positions of one dilated unmasking round in force [B, S] u8 (device, in place)."""
    if force.dtype != torch.uint8 or force.dim() != 2:
        raise DllmError("force must be a [B, S] uint8 tensor")
    B, S = force.shape
    st = _lib().dllm_dus_mark(_ptr(force), B, S, int(lo), int(block), int(a), int(rounds), int(round), int(mark),
                              _stream(force.device))
    _check(st, "dllm_dus_mark")


def packed_plan(M: int, N: int, K: int, swiglu: bool = False):
    """(waves per workgroup, K splits) of the packed-weight product over M rows, or None when the
    packed path does not take that shape (host-side query)."""
    nw, sp = ctypes.c_int32(), ctypes.c_int32()
    ok = _lib().dllm_packed_plan(int(M), int(N), int(K), int(bool(swiglu)), ctypes.byref(nw), ctypes.byref(sp))
    return (nw.value, sp.value) if ok else None


def pack_weight(w, interleave_f: int = 0):
    """A [N, K] bf16 weight repacked into MFMA fragment order (new tensor, same device)."""
    if w.dtype != torch.bfloat16 or w.dim() != 2:
        raise DllmError("pack_weight takes a [N, K] bfloat16 tensor")
    N, K = w.shape
    out = torch.empty_like(w)
    st = _lib().dllm_pack_weight(_ptr(w), _ptr(out), N, K, int(interleave_f), _stream(w.device))
    _check(st, "dllm_pack_weight")
    return out


class Model:
    """Device weights in the C ABI layout plus the dllm_model struct.

    ``weights`` holds per-layer tensors wq/wk/wv/wo/wg/wu/wd and norms (as
    produced by synth.workloads); Q/K/V and gate/up are concatenated once
    here into the fused row layout the library expects.  With ``pack`` (bf16
    only) the QKV, gate/up and down weights are also stored in MFMA fragment
    order (dllm_pack_weight), which the library streams for the active-row
    products (at most 128 rows) those copies fit; so is the LM head when the
    vocabulary is a multiple of 64.
    """

    def __init__(self, weights: dict, n_heads: int, n_kv_heads: int, mask_id: int, rope_base=1e4, rms_eps=1e-5,
                 pack: bool = True):
        emb = weights["embed"]
        self.dtype = emb.dtype
        self.device = emb.device
        V, d = emb.shape
        lw0 = weights["layers"][0]
        D = lw0["wq"].shape[0] // n_heads
        F = lw0["wg"].shape[0]
        L = len(weights["layers"])
        self.embed = emb.contiguous()
        self.final_norm = weights["final_norm"].contiguous()
        self.lm_head = weights["lm_head"].contiguous()
        self.layers = []
        for lw in weights["layers"]:
            self.layers.append({
                "attn_norm": lw["attn_norm"].contiguous(),
                "w_qkv": torch.cat([lw["wq"], lw["wk"], lw["wv"]], 0).contiguous(),
                "w_o": lw["wo"].contiguous(),
                "ffn_norm": lw["ffn_norm"].contiguous(),
                "w_gate_up": torch.cat([lw["wg"], lw["wu"]], 0).contiguous(),
                "w_down": lw["wd"].contiguous(),
            })
        if pack and emb.dtype == torch.bfloat16 and F % 16 == 0 and d % 64 == 0 and F % 64 == 0:
            for t in self.layers:
                t["w_gate_up_packed"] = pack_weight(t["w_gate_up"], interleave_f=F)
                t["w_down_packed"] = pack_weight(t["w_down"])
                t["w_qkv_packed"] = pack_weight(t["w_qkv"])
        self.lm_head_packed = None
        if pack and emb.dtype == torch.bfloat16 and V % 64 == 0 and d % 64 == 0:
            self.lm_head_packed = pack_weight(self.lm_head)
        self._lw = (_ffi.LayerW * L)()
        names = ("attn_norm", "w_qkv", "w_o", "ffn_norm", "w_gate_up", "w_down", "w_gate_up_packed", "w_down_packed",
                 "w_qkv_packed")
        for i, t in enumerate(self.layers):
            self._lw[i] = _ffi.LayerW(*[_ptr(t.get(k)) for k in names])
        self.dims_tuple = (V, d, n_heads, n_kv_heads, D, F, L)
        self.mask_id = mask_id
        self.c = _ffi.ModelC()
        self.c.dtype = _dtype_code(emb)
        self.c.rope_base = float(rope_base)
        self.c.rms_eps = float(rms_eps)
        self.c.mask_id = int(mask_id)
        self.c.embed = _ptr(self.embed)
        self.c.layers = ctypes.cast(self._lw, ctypes.POINTER(_ffi.LayerW))
        self.c.final_norm = _ptr(self.final_norm)
        self.c.lm_head = _ptr(self.lm_head)
        self.c.lm_head_packed = _ptr(self.lm_head_packed)

    def dims(self, B: int, S: int) -> _ffi.Dims:
        V, d, Hq, Hkv, D, F, L = self.dims_tuple
        return _ffi.Dims(B, S, d, Hq, Hkv, D, F, V, L)

    def bind(self, B: int, S: int):
        self.c.dims = self.dims(B, S)
        return self.c


def workspace_size(dims: _ffi.Dims, dtype_code: int, k_max: int) -> int:
    n = _lib().dllm_workspace_size(ctypes.byref(dims), dtype_code, k_max)
    if n == 0:
        raise DllmError("invalid dims for workspace")
    return n


def layer_sparse(model: Model, layer: int, x_act, idx, n_active, k_cache, v_cache, ws):
    B, S = k_cache.shape[0], k_cache.shape[1]
    k_max = idx.shape[1]
    mc = model.bind(B, S)
    st = _lib().dllm_layer_sparse(ctypes.byref(mc), layer, _ptr(x_act), _ptr(idx), _ptr(n_active), k_max,
                                  _ptr(k_cache), _ptr(v_cache), _ptr(ws), ws.numel() * ws.element_size(),
                                  _stream(x_act.device))
    _check(st, "dllm_layer_sparse")


def layer_sparse_noalloc(model: Model, layer: int, x_act, idx, n_active, k_cache, v_cache):
    """dllm_layer_sparse without a workspace: the library's per-GPU scratch array instead (calls that
    overlap on one GPU race on it)."""
    B, S = k_cache.shape[0], k_cache.shape[1]
    k_max = idx.shape[1]
    mc = model.bind(B, S)
    st = _lib().dllm_layer_sparse_noalloc(ctypes.byref(mc), layer, _ptr(x_act), _ptr(idx), _ptr(n_active), k_max,
                                          _ptr(k_cache), _ptr(v_cache), _stream(x_act.device))
    _check(st, "dllm_layer_sparse_noalloc")


class State:
    """Persistent device state of one generation run (tensors + dllm_state struct)."""

    def __init__(self, model: Model, tokens: torch.Tensor, k_max: int, track_kl: bool = False, with_force: bool = True,
                 kl_state: str = "f32", n_nested: int = 0, layer_cache: bool = False):
        """kl_state: "f32" or "bf16", the precision the previous logits are kept in (with track_kl).
        n_nested: hidden-state caches for that many nested boundaries.
        layer_cache: per-layer input/output hidden-state caches for the per-layer cache steps."""
        if kl_state not in ("f32", "bf16"):
            raise DllmError("kl_state must be 'f32' or 'bf16'")
        if not 0 <= n_nested <= _ffi.MAX_NESTED:
            raise DllmError(f"n_nested must be 0..{_ffi.MAX_NESTED}")
        B, S = tokens.shape
        V, d, Hq, Hkv, D, F, L = model.dims_tuple
        dev, dt = model.device, model.dtype
        self.B, self.S, self.k_max = B, S, k_max
        self.tokens = tokens.to(dev, torch.int32).contiguous()
        self.k_cache = [torch.zeros((B, S, Hkv, D), dtype=dt, device=dev) for _ in range(L)]
        self.v_cache = [torch.zeros((B, S, Hkv, D), dtype=dt, device=dev) for _ in range(L)]
        self.h_bnd = [torch.zeros((B, S, d), dtype=dt, device=dev) for _ in range(2)]
        self.h_fin = torch.zeros((B, S, d), dtype=dt, device=dev)
        self.h_nested = [torch.zeros((B, S, d), dtype=dt, device=dev) for _ in range(n_nested)]
        self.x_in = [torch.zeros((B, S, d), dtype=dt, device=dev) for _ in range(L)] if layer_cache else []
        self.x_out = [torch.zeros((B, S, d), dtype=dt, device=dev) for _ in range(L)] if layer_cache else []
        self.conf = torch.zeros((B, S), dtype=torch.float32, device=dev)
        self.kl = torch.full((B, S), float("inf"), dtype=torch.float32, device=dev)
        self.argmax = torch.zeros((B, S), dtype=torch.int32, device=dev)
        prev_dt = torch.bfloat16 if kl_state == "bf16" else torch.float32
        self.logits_prev = torch.zeros((B * S, V), dtype=prev_dt, device=dev) if track_kl else None
        self.force = torch.zeros((B, S), dtype=torch.uint8, device=dev) if with_force else None
        self.idx = torch.full((B, k_max), -1, dtype=torch.int32, device=dev)
        self.n_active = torch.zeros((B,), dtype=torch.int32, device=dev)
        self._kp = (ctypes.c_void_p * L)(*[_ptr(t) for t in self.k_cache])
        self._vp = (ctypes.c_void_p * L)(*[_ptr(t) for t in self.v_cache])
        self.c = _ffi.StateC()
        self.c.tokens = _ptr(self.tokens)
        self.c.k_cache = ctypes.cast(self._kp, ctypes.POINTER(ctypes.c_void_p))
        self.c.v_cache = ctypes.cast(self._vp, ctypes.POINTER(ctypes.c_void_p))
        self.c.h_bnd[0] = _ptr(self.h_bnd[0])
        self.c.h_bnd[1] = _ptr(self.h_bnd[1])
        self.c.bnd_cur = 0
        self.c.h_fin = _ptr(self.h_fin)
        self.c.conf = _ptr(self.conf)
        self.c.kl = _ptr(self.kl)
        self.c.argmax = _ptr(self.argmax)
        self.c.logits_prev = _ptr(self.logits_prev)
        self.c.force = _ptr(self.force)
        self.c.idx = _ptr(self.idx)
        self.c.n_active = _ptr(self.n_active)
        self.c.k_max = int(k_max)
        self.c.have_prev = 0
        self.c.logits_prev_dtype = DLLM_BF16 if kl_state == "bf16" else DLLM_F32
        for j, t in enumerate(self.h_nested):
            self.c.h_nested[j] = _ptr(t)
        if layer_cache:
            self._xi = (ctypes.c_void_p * L)(*[_ptr(t) for t in self.x_in])
            self._xo = (ctypes.c_void_p * L)(*[_ptr(t) for t in self.x_out])
            self.c.x_in_cache = ctypes.cast(self._xi, ctypes.POINTER(ctypes.c_void_p))
            self.c.x_out_cache = ctypes.cast(self._xo, ctypes.POINTER(ctypes.c_void_p))

    @property
    def h_bnd_prev(self) -> torch.Tensor:
        """Hidden state entering the boundary layer, as stored by the last step."""
        return self.h_bnd[self.c.bnd_cur]


def step_cfg(boundary_layer: int, full_step: bool, score: _ffi.ScoreCfg | None = None, *, lock_kl_eps=-1.0,
             lock_conf_min=0.9, unmask_n=0, block_lo=0, block_hi=0, unmask_mode=UNMASK_CONF,
             ws=None, nested=(), layer_cache=False, timing=None) -> _ffi.StepCfg:
    """nested: ((layer, k), ...) later layers that narrow the active set (at most MAX_NESTED).
    layer_cache: per-layer partial update from the boundary layer on (needs State(layer_cache=True)),
    comparing the hidden state entering each layer (True or "hidden") or the layer's V projection of
    it against the cached V ("value").
    timing: an _ffi.Timing measurement hook for this call (kept alive by the caller), or None."""
    if len(nested) > _ffi.MAX_NESTED:
        raise DllmError(f"at most {_ffi.MAX_NESTED} nested boundaries")
    c = _ffi.StepCfg()
    c.boundary_layer = int(boundary_layer)
    c.full_step = int(bool(full_step))
    c.score = score if score is not None else score_cfg()
    c.lock_kl_eps = float(lock_kl_eps)
    c.lock_conf_min = float(lock_conf_min)
    c.unmask_n = int(unmask_n)
    c.block_lo = int(block_lo)
    c.block_hi = int(block_hi)
    c.unmask_mode = int(unmask_mode)
    if ws is not None:
        c.ws = _ptr(ws)
        c.ws_bytes = ws.numel() * ws.element_size()
    c.n_nested = len(nested)
    for j, (nl, nk) in enumerate(nested):
        c.nested_layer[j] = int(nl)
        c.nested_k[j] = int(nk)
    modes = {False: 0, True: 1, "hidden": 1, "value": 2}
    if layer_cache not in modes:
        raise DllmError("layer_cache must be False, True / 'hidden' or 'value'")
    c.layer_cache = modes[layer_cache]
    if timing is not None:
        c.timing = ctypes.pointer(timing)
    return c


def alloc_workspace(model: Model, B: int, S: int, k_max: int) -> torch.Tensor:
    n = workspace_size(model.dims(B, S), _dtype_code(model.embed), k_max)
    return torch.empty(n, dtype=torch.uint8, device=model.device)


def skip_step(model: Model, state: State, cfg: _ffi.StepCfg):
    mc = model.bind(state.B, state.S)
    st = _lib().dllm_skip_step(ctypes.byref(mc), ctypes.byref(state.c), ctypes.byref(cfg), _stream(model.device))
    _check(st, "dllm_skip_step")
