"""Python binding of libmuse_attn.so: the Muse Glimmer / Muse Spark Open
attention layer on MI355X (gfx950).

Argument marshalling only: every step of the layer runs in the library's HIP
kernels.  PyTorch supplies device memory and the current stream.  There is no
fallback: without the built library every call raises.

Entry points (same names as the C ABI in include/muse_attn.h):
    rope_qknorm(layer, q, k, positions=None, out_dtype=torch.bfloat16)
    prefill(layer, q, k, v, gate, positions=None, out=None, workspace=None)
    decode(layer, q_new, k_new, v_new, gate, kv_len, max_kv_len, cache, out=None, workspace=None)
    layer_is_global(i, n_layers)
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass
from typing import Optional

from . import _capi
from ._capi import MuseError, MUSE_KV_PAGED, MUSE_KV_RING  # noqa: F401

__all__ = ["LayerParams", "KvCache", "rope_qknorm", "prefill", "decode", "layer_is_global",
           "prefill_workspace_size", "decode_workspace_size", "version", "MuseError"]


@dataclass(frozen=True)
class LayerParams:
    """One layer's settings; field meanings as muse_attn_params."""
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    sliding_window: int = 0        # 0 = global layer
    rope_theta: float = 0.0        # 0 = NoPE
    qk_scale: float = 1.0
    qk_norm_eps: float = 1e-5
    out_norm: bool = False
    out_norm_eps: float = 1e-6

    @classmethod
    def from_layer(cls, layer) -> "LayerParams":
        """From an object with hq/hkv/d/window/theta/scale/qk_eps/out_norm/out_eps."""
        return cls(layer.hq, layer.hkv, layer.d, layer.window, layer.theta, layer.scale,
                   layer.qk_eps, bool(layer.out_norm), layer.out_eps)

    def c(self) -> _capi.MuseAttnParams:
        return _capi.MuseAttnParams(self.num_q_heads, self.num_kv_heads, self.head_dim,
                                    self.sliding_window, self.rope_theta, self.qk_scale,
                                    self.qk_norm_eps, 1 if self.out_norm else 0, self.out_norm_eps)


@dataclass
class KvCache:
    """A caller-owned KV cache (see muse_kv_cache).

    ring:  k [B, Hkv, W, D], v [B, Hkv, D, W]
    paged: k [num_pages, Hkv, page_tokens, D], v [num_pages, Hkv, D, page_tokens],
           block_table int32 [B, max_pages_per_seq]
    Entries are bf16, or E4M3 codes (uint8 or float8_e4m3fn tensors) with
    fp32 scales k_scale, v_scale: [num_pages, Hkv] (paged) or [B, Hkv] (ring).
    """
    kind: int
    k: "object"
    v: "object"
    block_table: Optional["object"] = None
    page_tokens: int = 0
    k_scale: Optional["object"] = None
    v_scale: Optional["object"] = None

    @classmethod
    def ring(cls, k, v, k_scale=None, v_scale=None):
        return cls(MUSE_KV_RING, k, v, None, 0, k_scale, v_scale)

    @classmethod
    def paged(cls, k, v, block_table, page_tokens, k_scale=None, v_scale=None):
        return cls(MUSE_KV_PAGED, k, v, block_table, page_tokens, k_scale, v_scale)

    @property
    def dtype(self) -> int:
        torch = _torch()
        if self.k.dtype == torch.bfloat16:
            return _capi.MUSE_DTYPE_BF16
        if self.k.dtype in (torch.uint8, getattr(torch, "float8_e4m3fn", None)):
            return _capi.MUSE_DTYPE_FP8_E4M3
        raise TypeError(f"cache entries must be bfloat16 or E4M3 codes, got {self.k.dtype}")

    def c(self) -> _capi.MuseKvCache:
        fp8 = self.dtype == _capi.MUSE_DTYPE_FP8_E4M3
        if fp8 and (self.k_scale is None or self.v_scale is None):
            raise ValueError("an E4M3 cache needs k_scale and v_scale")
        ks = self.k_scale.data_ptr() if fp8 else None
        vs = self.v_scale.data_ptr() if fp8 else None
        if self.kind == MUSE_KV_RING:
            return _capi.MuseKvCache(MUSE_KV_RING, int(self.k.shape[2]), self.k.data_ptr(), self.v.data_ptr(),
                                     None, 0, 0, 0, self.dtype, ks, vs)
        return _capi.MuseKvCache(MUSE_KV_PAGED, 0, self.k.data_ptr(), self.v.data_ptr(),
                                 self.block_table.data_ptr(), int(self.block_table.shape[1]),
                                 int(self.page_tokens), int(self.k.shape[0]), self.dtype, ks, vs)


def _torch():
    import torch
    return torch


def _stream():
    return ctypes.c_void_p(_torch().cuda.current_stream().cuda_stream)


def _check_bf16(name, t, heads, d):
    torch = _torch()
    if t.dtype != torch.bfloat16:
        raise TypeError(f"{name} must be bfloat16, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.shape[-1] != d or t.shape[-2] != heads:
        raise ValueError(f"{name} must end in [{heads}, {d}], got {tuple(t.shape)}")
    if t.stride(-1) != 1 or t.stride(-2) != d:
        raise ValueError(f"{name}: heads and dims must be contiguous")


def _check_aux(name, t, dtype, numel, device):
    """An auxiliary tensor (positions, lengths, starts, block table, scales,
    workspace): its element type, its element count (None: any) and its
    device are checked before anything reaches the library, which takes a
    device pointer for it and reads exactly that many entries."""
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} must hold {numel} entries, got {t.numel()}")
    if not t.is_cuda or t.device != device:
        raise ValueError(f"{name} must be a device tensor on {device}, got {t.device}")


def _check_workspace(workspace, need, device):
    torch = _torch()
    _check_aux("workspace", workspace, torch.uint8, None, device)
    if not workspace.is_contiguous():
        raise ValueError("workspace must be contiguous")
    if workspace.numel() < need:
        raise ValueError(f"workspace holds {workspace.numel()} bytes, the call needs {need}")


def _check_cache(cache, device):
    torch = _torch()
    for name, t in (("cache.k", cache.k), ("cache.v", cache.v)):
        if not t.is_cuda or t.device != device:
            raise ValueError(f"{name} must be a device tensor on {device}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if cache.kind == MUSE_KV_PAGED:
        bt = cache.block_table
        if bt is None or bt.dim() != 2 or not bt.is_contiguous():
            raise ValueError("a paged cache needs a contiguous [B, max_pages] block_table")
        _check_aux("cache.block_table", bt, torch.int32, None, device)
    if cache.dtype == _capi.MUSE_DTYPE_FP8_E4M3:
        n = int(cache.k.shape[0]) * int(cache.k.shape[1])   # [num_pages or B] x Hkv
        for name, t in (("cache.k_scale", cache.k_scale), ("cache.v_scale", cache.v_scale)):
            if t is None:
                raise ValueError("an E4M3 cache needs k_scale and v_scale")
            _check_aux(name, t, torch.float32, n, device)
            if not t.is_contiguous():
                raise ValueError(f"{name} must be contiguous")


def version() -> int:
    return _capi.load().muse_version()


def layer_is_global(i: int, n_layers: int) -> bool:
    r = _capi.load().muse_layer_is_global(i, n_layers)
    if r < 0:
        raise ValueError("layer index out of range")
    return bool(r)


def rope_qknorm(layer: LayerParams, q=None, k=None, positions=None, out_dtype=None):
    """Weightless QK-norm, query multiplier and (if rope_theta) RoPE.
    q [T, Hq, D], k [T, Hkv, D] bf16 (token stride free).  Returns (q_hat, k_hat)."""
    torch = _torch()
    lib = _capi.load()
    out_dtype = out_dtype or torch.bfloat16
    code = {torch.bfloat16: _capi.MUSE_DTYPE_BF16, torch.float16: _capi.MUSE_DTYPE_F16,
            torch.float32: _capi.MUSE_DTYPE_F32}[out_dtype]
    ref = q if q is not None else k
    n = int(ref.shape[0])
    qo = ko = None
    if q is not None:
        _check_bf16("q", q, layer.num_q_heads, layer.head_dim)
        qo = torch.empty((n, layer.num_q_heads, layer.head_dim), dtype=out_dtype, device=q.device)
    if k is not None:
        _check_bf16("k", k, layer.num_kv_heads, layer.head_dim)
        ko = torch.empty((n, layer.num_kv_heads, layer.head_dim), dtype=out_dtype, device=k.device)
    if positions is not None:
        _check_aux("positions", positions, torch.int32, n, ref.device)
        positions = positions.contiguous()
    if q is not None and k is not None and q.device != k.device:
        raise ValueError("q and k must be on one device")
    p = layer.c()
    _capi.check(lib.muse_rope_qknorm(
        ctypes.byref(p), n,
        q.data_ptr() if q is not None else None, q.stride(0) if q is not None else 0,
        k.data_ptr() if k is not None else None, k.stride(0) if k is not None else 0,
        positions.data_ptr() if positions is not None else None,
        qo.data_ptr() if qo is not None else None, ko.data_ptr() if ko is not None else None,
        code, _stream()))
    return qo, ko


def prefill_workspace_size(layer: LayerParams, batch: int, seq: int) -> int:
    p = layer.c()
    return int(_capi.load().muse_attn_prefill_workspace_size(ctypes.byref(p), batch, seq))


def prefill(layer: LayerParams, q, k, v, gate, positions=None, out=None, workspace=None):
    """The layer over [B, T] tokens: q, gate [B, T, Hq, D]; k, v [B, T, Hkv, D] (bf16).
    Returns out [B, T, Hq, D] bf16."""
    torch = _torch()
    lib = _capi.load()
    B, T = int(q.shape[0]), int(q.shape[1])
    _check_bf16("q", q, layer.num_q_heads, layer.head_dim)
    _check_bf16("k", k, layer.num_kv_heads, layer.head_dim)
    _check_bf16("v", v, layer.num_kv_heads, layer.head_dim)
    _check_bf16("gate", gate, layer.num_q_heads, layer.head_dim)
    for name, t in (("k", k), ("v", v), ("gate", gate)):
        if int(t.shape[0]) != B or int(t.shape[1]) != T:
            raise ValueError(f"{name} batch/sequence shape mismatch")
    if out is None:
        out = torch.empty((B, T, layer.num_q_heads, layer.head_dim), dtype=torch.bfloat16, device=q.device)
    _check_bf16("out", out, layer.num_q_heads, layer.head_dim)
    for name, t in (("k", k), ("v", v), ("gate", gate), ("out", out)):
        if t.device != q.device:
            raise ValueError(f"{name} must be on the device of q ({q.device})")
    need = prefill_workspace_size(layer, B, T)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _check_workspace(workspace, need, q.device)
    strides = (ctypes.c_int64 * 10)(*[int(s) for t in (q, k, v, gate, out) for s in (t.stride(0), t.stride(1))])
    if positions is not None:
        _check_aux("positions", positions, torch.int32, B * T, q.device)
        positions = positions.contiguous()
    p = layer.c()
    _capi.check(lib.muse_attn_prefill(
        ctypes.byref(p), B, T, q.data_ptr(), k.data_ptr(), v.data_ptr(), gate.data_ptr(), strides,
        positions.data_ptr() if positions is not None else None, out.data_ptr(),
        workspace.data_ptr(), workspace.numel() * workspace.element_size(), _stream()))
    return out


def prefill_chunk_workspace_size(layer: LayerParams, batch: int, seq: int, max_start: int) -> int:
    p = layer.c()
    return int(_capi.load().muse_attn_prefill_chunk_workspace_size(ctypes.byref(p), batch, seq, max_start))


def prefill_chunk(layer: LayerParams, q, k, v, gate, start, max_start: int, cache: KvCache, out=None,
                  workspace=None):
    """Chunked prefill: q, gate [B, T, Hq, D]; k, v [B, T, Hkv, D] (bf16) are the chunk's
    projections at positions start[b] .. start[b] + T - 1 (start: device int32 [B], each
    <= max_start).  Attends over the cached history and the chunk, writes the chunk's
    keys and values into the cache, and returns out [B, T, Hq, D] bf16."""
    return _chunk_like("muse_attn_prefill_chunk", layer, q, k, v, gate, start, max_start, cache, out, workspace)


def draft_block_workspace_size(layer: LayerParams, batch: int, seq: int, max_start: int) -> int:
    p = layer.c()
    return int(_capi.load().muse_attn_draft_block_workspace_size(ctypes.byref(p), batch, seq, max_start))


def draft_block(layer: LayerParams, q, k, v, gate, start, max_start: int, cache: KvCache, out=None,
                workspace=None):
    """A block-diffusion drafter's block: the T block tokens at positions start[b] ..
    start[b] + T - 1 attend to the cached context and to every block key within the
    window in both directions (no causal mask).  The cache is read only.  Shapes as for
    prefill_chunk; returns out [B, T, Hq, D] bf16."""
    return _chunk_like("muse_attn_draft_block", layer, q, k, v, gate, start, max_start, cache, out, workspace)


def _chunk_like(entry, layer, q, k, v, gate, start, max_start, cache, out, workspace):
    torch = _torch()
    lib = _capi.load()
    B, T = int(q.shape[0]), int(q.shape[1])
    _check_bf16("q", q, layer.num_q_heads, layer.head_dim)
    _check_bf16("k", k, layer.num_kv_heads, layer.head_dim)
    _check_bf16("v", v, layer.num_kv_heads, layer.head_dim)
    _check_bf16("gate", gate, layer.num_q_heads, layer.head_dim)
    for name, t in (("k", k), ("v", v), ("gate", gate)):
        if int(t.shape[0]) != B or int(t.shape[1]) != T:
            raise ValueError(f"{name} batch/sequence shape mismatch")
    _check_aux("start", start, torch.int32, B, q.device)
    if out is None:
        out = torch.empty((B, T, layer.num_q_heads, layer.head_dim), dtype=torch.bfloat16, device=q.device)
    _check_bf16("out", out, layer.num_q_heads, layer.head_dim)
    for name, t in (("k", k), ("v", v), ("gate", gate), ("out", out)):
        if t.device != q.device:
            raise ValueError(f"{name} must be on the device of q ({q.device})")
    _check_cache(cache, q.device)
    size_fn = draft_block_workspace_size if entry == "muse_attn_draft_block" else prefill_chunk_workspace_size
    need = size_fn(layer, B, T, max_start)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _check_workspace(workspace, need, q.device)
    strides = (ctypes.c_int64 * 10)(*[int(s) for t in (q, k, v, gate, out) for s in (t.stride(0), t.stride(1))])
    p = layer.c()
    c = cache.c()
    _capi.check(getattr(lib, entry)(
        ctypes.byref(p), B, T, q.data_ptr(), k.data_ptr(), v.data_ptr(), gate.data_ptr(), strides,
        start.contiguous().data_ptr(), int(max_start), ctypes.byref(c), out.data_ptr(),
        workspace.data_ptr(), workspace.numel() * workspace.element_size(), _stream()))
    return out


def decode_workspace_size(layer: LayerParams, batch: int, max_kv_len: int, cache: KvCache) -> int:
    p = layer.c()
    c = cache.c()
    return int(_capi.load().muse_attn_decode_workspace_size(ctypes.byref(p), batch, max_kv_len, ctypes.byref(c)))


def decode(layer: LayerParams, q_new, k_new, v_new, gate, kv_len, max_kv_len: int, cache: KvCache,
           out=None, workspace=None):
    """One decode step: q_new, gate [B, Hq, D]; k_new, v_new [B, Hkv, D] (bf16, contiguous);
    kv_len int32 device [B] including the new token.  Writes the new entry into the cache
    and returns out [B, Hq, D] bf16."""
    torch = _torch()
    lib = _capi.load()
    B = int(q_new.shape[0])
    for name, t, h in (("q_new", q_new, layer.num_q_heads), ("k_new", k_new, layer.num_kv_heads),
                       ("v_new", v_new, layer.num_kv_heads), ("gate", gate, layer.num_q_heads)):
        _check_bf16(name, t, h, layer.head_dim)
        if not t.is_contiguous() or int(t.shape[0]) != B:
            raise ValueError(f"{name} must be contiguous [B, H, D]")
        if t.device != q_new.device:
            raise ValueError(f"{name} must be on the device of q_new ({q_new.device})")
    _check_aux("kv_len", kv_len, torch.int32, B, q_new.device)
    if out is None:
        out = torch.empty((B, layer.num_q_heads, layer.head_dim), dtype=torch.bfloat16, device=q_new.device)
    _check_bf16("out", out, layer.num_q_heads, layer.head_dim)
    if not out.is_contiguous() or int(out.shape[0]) != B or out.device != q_new.device:
        raise ValueError("out must be a contiguous [B, Hq, D] tensor on the device of q_new")
    _check_cache(cache, q_new.device)
    need = decode_workspace_size(layer, B, max_kv_len, cache)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q_new.device)
    _check_workspace(workspace, need, q_new.device)
    p = layer.c()
    c = cache.c()
    _capi.check(lib.muse_attn_decode(
        ctypes.byref(p), B, q_new.data_ptr(), k_new.data_ptr(), v_new.data_ptr(), gate.data_ptr(),
        kv_len.data_ptr(), int(max_kv_len), ctypes.byref(c), out.data_ptr(),
        workspace.data_ptr(), workspace.numel() * workspace.element_size(), _stream()))
    return out


def decode_noalloc(layer: LayerParams, q_new, k_new, v_new, gate, kv_len, max_kv_len: int, cache: KvCache,
                   out=None):
    """decode() through muse_attn_decode_noalloc: the library's fixed per-device
    scratch replaces the workspace, so the call itself allocates nothing (pass
    `out` to allocate nothing on the Python side either).  Calls that overlap on
    one device race on that scratch."""
    torch = _torch()
    lib = _capi.load()
    B = int(q_new.shape[0])
    for name, t, h in (("q_new", q_new, layer.num_q_heads), ("k_new", k_new, layer.num_kv_heads),
                       ("v_new", v_new, layer.num_kv_heads), ("gate", gate, layer.num_q_heads)):
        _check_bf16(name, t, h, layer.head_dim)
        if not t.is_contiguous() or int(t.shape[0]) != B:
            raise ValueError(f"{name} must be contiguous [B, H, D]")
        if t.device != q_new.device:
            raise ValueError(f"{name} must be on the device of q_new ({q_new.device})")
    _check_aux("kv_len", kv_len, torch.int32, B, q_new.device)
    if out is None:
        out = torch.empty((B, layer.num_q_heads, layer.head_dim), dtype=torch.bfloat16, device=q_new.device)
    _check_bf16("out", out, layer.num_q_heads, layer.head_dim)
    if not out.is_contiguous() or int(out.shape[0]) != B or out.device != q_new.device:
        raise ValueError("out must be a contiguous [B, Hq, D] tensor on the device of q_new")
    _check_cache(cache, q_new.device)
    p = layer.c()
    c = cache.c()
    _capi.check(lib.muse_attn_decode_noalloc(
        ctypes.byref(p), B, q_new.data_ptr(), k_new.data_ptr(), v_new.data_ptr(), gate.data_ptr(),
        kv_len.data_ptr(), int(max_kv_len), ctypes.byref(c), out.data_ptr(), _stream()))
    return out


@dataclass
class BlockWeights:
    """Weights of a decoder block's attention half (see muse_block_weights):
    in_norm [hidden] bf16; w_qkvg [(2 Hq + 2 Hkv) D, hidden] bf16; w_o [hidden, Hq D]
    bf16; post_norm [hidden] bf16 (plain residual add) or residual_gate [hidden] fp32."""
    in_norm: object
    w_qkvg: object
    w_o: object
    post_norm: object = None
    residual_gate: object = None
    temperature: float = 0.3

    @property
    def hidden(self) -> int:
        return int(self.in_norm.shape[0])

    def c(self):
        def ptr(t):
            return t.data_ptr() if t is not None else None
        return _capi.MuseBlockWeights(self.hidden, ptr(self.in_norm), ptr(self.w_qkvg), ptr(self.w_o),
                                      ptr(self.post_norm), ptr(self.residual_gate), float(self.temperature))


def block_prefill_workspace_size(layer: LayerParams, weights: BlockWeights, batch: int, seq: int) -> int:
    p = layer.c()
    w = weights.c()
    return int(_capi.load().muse_attn_block_prefill_workspace_size(ctypes.byref(p), ctypes.byref(w), batch, seq))


def _check_block_out(out, x):
    """out of a block call: a contiguous bf16 tensor of x's shape on x's device."""
    torch = _torch()
    if out.dtype != torch.bfloat16 or out.device != x.device or not out.is_contiguous() or out.shape != x.shape:
        raise ValueError(f"out must be a contiguous bf16 tensor of shape {tuple(x.shape)} on {x.device}")


def _check_block_weights(layer, w, device):
    """The block's weights: bf16 in_norm [hidden], w_qkvg [(2 Hq + 2 Hkv) D, hidden],
    w_o [hidden, Hq D] and post_norm [hidden], fp32 residual_gate [hidden], all
    contiguous on the call's device."""
    torch = _torch()
    h, hq, hkv, d = w.hidden, layer.num_q_heads, layer.num_kv_heads, layer.head_dim
    numel = {"in_norm": h, "w_qkvg": (2 * hq + 2 * hkv) * d * h, "w_o": h * hq * d, "post_norm": h,
             "residual_gate": h}
    for name, n in numel.items():
        t = getattr(w, name)
        if t is None:
            continue
        want = torch.float32 if name == "residual_gate" else torch.bfloat16
        if t.dtype != want or t.device != device or not t.is_contiguous() or t.numel() != n:
            raise ValueError(f"weights.{name} must be a contiguous {want} tensor of {n} elements on {device}")


def attention_block_prefill(layer: LayerParams, weights: BlockWeights, x, out=None, workspace=None):
    """The attention half of a decoder block on x [B, T, hidden] (bf16, contiguous):
    input norm, projections, the layer, o_proj, post-norm and residual.  Returns
    out [B, T, hidden] bf16."""
    torch = _torch()
    lib = _capi.load()
    if x.dtype != torch.bfloat16 or not x.is_cuda or not x.is_contiguous() or x.dim() != 3:
        raise ValueError("x must be a contiguous device bf16 tensor [B, T, hidden]")
    B, T, H = (int(s) for s in x.shape)
    if H != weights.hidden:
        raise ValueError("x width does not match the weights")
    if out is None:
        out = torch.empty_like(x)
    _check_block_out(out, x)
    _check_block_weights(layer, weights, x.device)
    need = block_prefill_workspace_size(layer, weights, B, T)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    _check_workspace(workspace, need, x.device)
    p = layer.c()
    w = weights.c()
    _capi.check(lib.muse_attn_block_prefill(ctypes.byref(p), ctypes.byref(w), B, T, x.data_ptr(), out.data_ptr(),
                                            workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                                            _stream()))
    return out


def attention_block_tune(layer: LayerParams, weights: BlockWeights, rows: int, workspace=None):
    """Time hipBLASLt's candidate algorithms for the block's two projection GEMMs
    at `rows` token rows and record the fastest for later block calls on this
    device.  Waits for the stream: call it outside timed or captured regions."""
    torch = _torch()
    lib = _capi.load()
    _check_block_weights(layer, weights, weights.w_qkvg.device)
    need = block_prefill_workspace_size(layer, weights, 1, rows)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=weights.w_qkvg.device)
    _check_workspace(workspace, need, weights.w_qkvg.device)
    p = layer.c()
    w = weights.c()
    _capi.check(lib.muse_attn_block_tune(ctypes.byref(p), ctypes.byref(w), int(rows), workspace.data_ptr(),
                                         workspace.numel(), _stream()))


def block_decode_workspace_size(layer: LayerParams, weights: BlockWeights, batch: int, max_kv_len: int,
                                cache: KvCache) -> int:
    p = layer.c()
    w = weights.c()
    c = cache.c()
    return int(_capi.load().muse_attn_block_decode_workspace_size(ctypes.byref(p), ctypes.byref(w), batch,
                                                                   max_kv_len, ctypes.byref(c)))


def attention_block_decode(layer: LayerParams, weights: BlockWeights, x, kv_len, max_kv_len: int, cache: KvCache,
                           out=None, workspace=None):
    """One new token per sequence through a decoder block's attention half: x [B, hidden]
    (bf16, contiguous), kv_len int32 device [B] including the new token.  Appends the new
    key and value to the cache and returns out [B, hidden] bf16."""
    torch = _torch()
    lib = _capi.load()
    if x.dtype != torch.bfloat16 or not x.is_cuda or not x.is_contiguous() or x.dim() != 2:
        raise ValueError("x must be a contiguous device bf16 tensor [B, hidden]")
    B, H = (int(s) for s in x.shape)
    if H != weights.hidden:
        raise ValueError("x width does not match the weights")
    if kv_len.dtype != torch.int32 or not kv_len.is_cuda or kv_len.numel() != B:
        raise ValueError("kv_len must be a device int32 tensor of B entries")
    if kv_len.device != x.device:
        raise ValueError(f"kv_len must be on the device of x ({x.device})")
    if out is None:
        out = torch.empty_like(x)
    _check_block_out(out, x)
    _check_block_weights(layer, weights, x.device)
    _check_cache(cache, x.device)
    need = block_decode_workspace_size(layer, weights, B, max_kv_len, cache)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    _check_workspace(workspace, need, x.device)
    p = layer.c()
    w = weights.c()
    c = cache.c()
    _capi.check(lib.muse_attn_block_decode(ctypes.byref(p), ctypes.byref(w), B, x.data_ptr(), kv_len.data_ptr(),
                                           int(max_kv_len), ctypes.byref(c), out.data_ptr(), workspace.data_ptr(),
                                           workspace.numel() * workspace.element_size(), _stream()))
    return out

