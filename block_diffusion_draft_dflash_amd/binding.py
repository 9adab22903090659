"""Thin ctypes binding of libdflash (include/dflash.h).

Functions carry the C names and only marshal arguments: torch tensors become
device pointers and sizes, the stream is torch's current HIP stream. Every
step runs in the library's HIP kernels; there is no fallback. If the library
is missing, ``load()`` raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdflash.so")

DFLASH_OK = 0
DFLASH_ERR_INVALID_ARG = -1
DFLASH_ERR_UNSUPPORTED = -2
DFLASH_ERR_WORKSPACE = -3
DFLASH_ERR_HIP = -4
DFLASH_F32 = 0
DFLASH_BF16 = 1

# Every symbol include/dflash.h declares.
EXPORTED = (
    "dflash_last_error",
    "dflash_abi_version",
    "dflash_rope_table",
    "dflash_qk_norm_rope",
    "dflash_block_attention_workspace_size",
    "dflash_block_attention_check",
    "dflash_block_attention",
    "dflash_block_attention_noalloc",
    "dflash_context_kv_workspace_size",
    "dflash_context_kv",
    "dflash_block_attention_paged",
    "dflash_block_attention_paged_workspace_size",
    "dflash_kv_scatter",
    "dflash_block_qkv_workspace_size",
    "dflash_block_qkv",
    "dflash_o_proj_workspace_size",
    "dflash_o_proj",
    "dflash_prepare_inputs",
    "dflash_fc_combine_workspace_size",
    "dflash_fc_combine",
)


class DflashError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"dflash status {status}: {msg}")
        self.status = status


class BlockAttnParams(ctypes.Structure):
    """Mirror of ``dflash_block_attn_params``."""

    _fields_ = [
        ("num_reqs", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("dtype", ctypes.c_int),
        ("total_ctx", ctypes.c_int64),
        ("total_blk", ctypes.c_int64),
        ("max_blk_len", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("causal", ctypes.c_int32),
        ("window", ctypes.c_int32),
        ("split_keys", ctypes.c_int32),
        ("host_cu_ctx_lens", ctypes.c_void_p),
        ("host_cu_blk_lens", ctypes.c_void_p),
    ]


class QkPrologue(ctypes.Structure):
    """Mirror of ``dflash_qk_prologue`` (fused q/k norm + RoPE of the attention)."""

    _fields_ = [
        ("q_norm_w", ctypes.c_void_p),
        ("k_norm_w", ctypes.c_void_p),
        ("positions", ctypes.c_void_p),
        ("rope_table", ctypes.c_void_p),
        ("max_pos", ctypes.c_int32),
        ("eps", ctypes.c_float),
    ]


class PagedCtx(ctypes.Structure):
    """Mirror of ``dflash_paged_ctx``."""

    _fields_ = [
        ("block_table", ctypes.c_void_p),
        ("max_pages_per_req", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("num_pages", ctypes.c_int64),
    ]


class PrepareParams(ctypes.Structure):
    """Mirror of ``dflash_prepare_params``."""

    _fields_ = [
        ("num_reqs", ctypes.c_int32), ("max_num_reqs", ctypes.c_int32),
        ("max_num_tokens", ctypes.c_int32), ("num_query_per_req", ctypes.c_int32),
        ("num_speculative_steps", ctypes.c_int32), ("block_size", ctypes.c_int32),
        ("block_table_stride", ctypes.c_int32), ("max_model_len", ctypes.c_int32),
        ("mask_token_id", ctypes.c_int32), ("sample_from_anchor", ctypes.c_int32),
        ("num_states", ctypes.c_int32), ("num_target_tokens", ctypes.c_int64),
    ]


PREP_IN = ("idx_mapping", "target_query_start_loc", "target_positions", "num_rejected",
           "num_sampled", "last_sampled", "next_prefill_tokens", "block_table")
PREP_OUT = ("input_ids", "query_positions", "query_start_loc", "seq_lens", "query_slot_mapping",
            "context_positions", "context_slot_mapping", "sample_indices", "sample_pos",
            "sample_idx_mapping", "ctx_cu")


class PrepareIn(ctypes.Structure):
    """Mirror of ``dflash_prepare_inputs_in`` (device pointers)."""

    _fields_ = [(n, ctypes.c_void_p) for n in PREP_IN]


class PrepareOut(ctypes.Structure):
    """Mirror of ``dflash_prepare_inputs_out`` (device pointers)."""

    _fields_ = [(n, ctypes.c_void_p) for n in PREP_OUT]


_lib: Optional[ctypes.CDLL] = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libdflash and declare its signatures (idempotent)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with `python -m block_diffusion_draft_dflash_amd.build`")
    lib = ctypes.CDLL(path)
    P, I32, I64, F, D, SZ = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float,
                             ctypes.c_double, ctypes.c_size_t)
    lib.dflash_last_error.restype = ctypes.c_char_p
    lib.dflash_last_error.argtypes = []
    lib.dflash_abi_version.restype = ctypes.c_int
    lib.dflash_abi_version.argtypes = []
    lib.dflash_rope_table.restype = ctypes.c_int
    lib.dflash_rope_table.argtypes = [P, I32, I32, D, P]
    lib.dflash_qk_norm_rope.restype = ctypes.c_int
    lib.dflash_qk_norm_rope.argtypes = [ctypes.c_int, P, P, P, P, P, I64, I32, I32, I32, F, P, I32, P]
    lib.dflash_block_attention_workspace_size.restype = SZ
    lib.dflash_block_attention_workspace_size.argtypes = [ctypes.POINTER(BlockAttnParams)]
    lib.dflash_block_attention_check.restype = ctypes.c_int
    lib.dflash_block_attention_check.argtypes = [ctypes.POINTER(BlockAttnParams)]
    lib.dflash_block_attention.restype = ctypes.c_int
    lib.dflash_block_attention.argtypes = [ctypes.POINTER(BlockAttnParams),
                                           ctypes.POINTER(QkPrologue), P, P, P, P, P, P, P, P,
                                           P, SZ, P]
    lib.dflash_block_attention_noalloc.restype = ctypes.c_int
    lib.dflash_block_attention_noalloc.argtypes = [ctypes.POINTER(BlockAttnParams),
                                                   ctypes.POINTER(QkPrologue), P, P, P, P, P, P,
                                                   P, P, P]
    lib.dflash_context_kv_workspace_size.restype = SZ
    lib.dflash_context_kv_workspace_size.argtypes = [I64, I32, I32, I32]
    lib.dflash_context_kv.restype = ctypes.c_int
    lib.dflash_context_kv.argtypes = [P, P, P, P, P, P, I64, I32, I32, I32, F, P, I32, P, P, P, SZ, P]
    lib.dflash_block_attention_paged.restype = ctypes.c_int
    lib.dflash_block_attention_paged.argtypes = [ctypes.POINTER(BlockAttnParams),
                                                 ctypes.POINTER(PagedCtx),
                                                 ctypes.POINTER(QkPrologue), P, P, P, P, P, P, P,
                                                 P, P, SZ, P]
    lib.dflash_block_attention_paged_workspace_size.restype = SZ
    lib.dflash_block_attention_paged_workspace_size.argtypes = [ctypes.POINTER(BlockAttnParams)]
    lib.dflash_kv_scatter.restype = ctypes.c_int
    lib.dflash_kv_scatter.argtypes = [ctypes.c_int, P, P, P, I64, I32, I32, P, P, I64, P]
    lib.dflash_block_qkv_workspace_size.restype = SZ
    lib.dflash_block_qkv_workspace_size.argtypes = [I64, I32, I32, I32, I32]
    lib.dflash_block_qkv.restype = ctypes.c_int
    lib.dflash_block_qkv.argtypes = [P, P, P, P, I64, I32, I32, I32, I32, F, P, P, P, P, SZ, P]
    lib.dflash_o_proj_workspace_size.restype = SZ
    lib.dflash_o_proj_workspace_size.argtypes = [I64, I32, I32]
    lib.dflash_o_proj.restype = ctypes.c_int
    lib.dflash_o_proj.argtypes = [P, P, I64, I32, I32, P, P, SZ, P]
    lib.dflash_prepare_inputs.restype = ctypes.c_int
    lib.dflash_prepare_inputs.argtypes = [ctypes.POINTER(PrepareParams), ctypes.POINTER(PrepareIn),
                                          ctypes.POINTER(PrepareOut), P]
    lib.dflash_fc_combine_workspace_size.restype = SZ
    lib.dflash_fc_combine_workspace_size.argtypes = [I64, I32, I32]
    lib.dflash_fc_combine.restype = ctypes.c_int
    lib.dflash_fc_combine.argtypes = [P, P, I64, I32, I32, P, P, SZ, P]
    _lib = lib
    return lib


def _check(status: int) -> None:
    if status != DFLASH_OK:
        raise DflashError(status, _lib.dflash_last_error().decode())


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if t.device.type != "cuda":
        raise ValueError("libdflash takes device tensors")
    if not t.is_contiguous():
        raise ValueError("libdflash takes contiguous tensors")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return DFLASH_BF16
    if t.dtype == torch.float32:
        return DFLASH_F32
    raise ValueError(f"unsupported dtype {t.dtype}")


def dflash_last_error() -> str:
    return load().dflash_last_error().decode()


def dflash_abi_version() -> int:
    return load().dflash_abi_version()


def dflash_rope_table(table: torch.Tensor, max_pos: int, head_dim: int, theta: float,
                      stream=None) -> None:
    """Fill ``table`` (f32, [max_pos, head_dim/2, 2]) with the RoPE cos/sin cache."""
    lib = load()
    _check(lib.dflash_rope_table(_ptr(table), max_pos, head_dim, float(theta), _stream(stream)))


def dflash_qk_norm_rope(q: Optional[torch.Tensor], k: torch.Tensor,
                        q_norm_w: Optional[torch.Tensor], k_norm_w: torch.Tensor,
                        positions: torch.Tensor, eps: float, rope_table: torch.Tensor,
                        stream=None) -> None:
    """In-place q/k RMSNorm + NeoX RoPE. q ``[T, Hq, Dh]`` (or None), k ``[T, Hkv, Dh]``."""
    lib = load()
    t, hkv, dh = k.shape
    hq = q.shape[1] if q is not None else 0
    max_pos = rope_table.shape[0]
    _check(lib.dflash_qk_norm_rope(_dtype_code(k), _ptr(q), _ptr(k), _ptr(q_norm_w),
                                   _ptr(k_norm_w), _ptr(positions), t, hq, hkv, dh, float(eps),
                                   _ptr(rope_table), max_pos, _stream(stream)))


def make_block_attn_params(num_reqs: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                           dtype: int, total_ctx: int, total_blk: int, max_blk_len: int,
                           scale: float, causal: bool = False, window: int = 0,
                           split_keys: int = 0, host_cu_ctx_lens=None,
                           host_cu_blk_lens=None) -> BlockAttnParams:
    """``host_cu_*``: optional host copies of the cumulative lengths (array-likes
    of R+1 ints); the returned struct keeps int32 copies of them alive."""
    p = BlockAttnParams(num_reqs, num_q_heads, num_kv_heads, head_dim, dtype, total_ctx,
                        total_blk, max_blk_len, scale, int(bool(causal)), window, split_keys,
                        None, None)
    if host_cu_ctx_lens is not None or host_cu_blk_lens is not None:
        if host_cu_ctx_lens is None or host_cu_blk_lens is None:
            raise ValueError("give both host_cu_ctx_lens and host_cu_blk_lens, or neither")
        keep = tuple((ctypes.c_int32 * len(a))(*[int(x) for x in a])
                     for a in (host_cu_ctx_lens, host_cu_blk_lens))
        p._host_lens = keep
        p.host_cu_ctx_lens = ctypes.cast(keep[0], ctypes.c_void_p)
        p.host_cu_blk_lens = ctypes.cast(keep[1], ctypes.c_void_p)
    return p


def dflash_block_attention_check(p: BlockAttnParams) -> int:
    return load().dflash_block_attention_check(ctypes.byref(p))


def dflash_block_attention_workspace_size(p: BlockAttnParams) -> int:
    return load().dflash_block_attention_workspace_size(ctypes.byref(p))


def make_qk_prologue(q_norm_w: torch.Tensor, k_norm_w: torch.Tensor, positions: torch.Tensor,
                     rope_table: torch.Tensor, eps: float) -> QkPrologue:
    rec = QkPrologue(_ptr(q_norm_w), _ptr(k_norm_w), _ptr(positions), _ptr(rope_table),
                     rope_table.shape[0], float(eps))
    rec._keep = (q_norm_w, k_norm_w, positions, rope_table)  # the record holds their pointers
    return rec


def dflash_block_attention(p: BlockAttnParams, cu_ctx_lens: torch.Tensor,
                           cu_blk_lens: torch.Tensor, q: torch.Tensor, k_blk: torch.Tensor,
                           v_blk: torch.Tensor, k_ctx: Optional[torch.Tensor],
                           v_ctx: Optional[torch.Tensor], out: torch.Tensor,
                           workspace: Optional[torch.Tensor], stream=None,
                           prologue: Optional[QkPrologue] = None) -> None:
    """Block attention; with ``prologue`` q and k_blk are raw and get q/k norm +
    RoPE inside the kernel (they are not modified)."""
    lib = load()
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.dflash_block_attention(ctypes.byref(p),
                                      ctypes.byref(prologue) if prologue is not None else None,
                                      _ptr(cu_ctx_lens), _ptr(cu_blk_lens),
                                      _ptr(q), _ptr(k_blk), _ptr(v_blk), _ptr(k_ctx), _ptr(v_ctx),
                                      _ptr(out), _ptr(workspace), ws_bytes, _stream(stream)))


NOALLOC_SCRATCH_BYTES = 32 << 20  # DFLASH_NOALLOC_SCRATCH_BYTES


def dflash_block_attention_noalloc(p: BlockAttnParams, cu_ctx_lens: torch.Tensor,
                                   cu_blk_lens: torch.Tensor, q: torch.Tensor, k_blk: torch.Tensor,
                                   v_blk: torch.Tensor, k_ctx: Optional[torch.Tensor],
                                   v_ctx: Optional[torch.Tensor], out: torch.Tensor, stream=None,
                                   prologue: Optional[QkPrologue] = None) -> None:
    """``dflash_block_attention`` with the library's own per-GPU scratch in
    place of a caller workspace (for callers that cannot allocate)."""
    lib = load()
    _check(lib.dflash_block_attention_noalloc(ctypes.byref(p),
                                              ctypes.byref(prologue) if prologue is not None else None,
                                              _ptr(cu_ctx_lens), _ptr(cu_blk_lens), _ptr(q),
                                              _ptr(k_blk), _ptr(v_blk), _ptr(k_ctx), _ptr(v_ctx),
                                              _ptr(out), _stream(stream)))


def dflash_context_kv_workspace_size(T: int, hidden_size: int, num_kv_heads: int,
                                     head_dim: int) -> int:
    return load().dflash_context_kv_workspace_size(T, hidden_size, num_kv_heads, head_dim)


def dflash_context_kv(hidden: torch.Tensor, hidden_norm_w: torch.Tensor, w_k: torch.Tensor,
                      w_v: torch.Tensor, k_norm_w: torch.Tensor, positions: torch.Tensor,
                      num_kv_heads: int, head_dim: int, eps: float, rope_table: torch.Tensor,
                      k_out: torch.Tensor, v_out: torch.Tensor, workspace: torch.Tensor,
                      stream=None) -> None:
    lib = load()
    t, h = hidden.shape
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib.dflash_context_kv(_ptr(hidden), _ptr(hidden_norm_w), _ptr(w_k), _ptr(w_v),
                                 _ptr(k_norm_w), _ptr(positions), t, h, num_kv_heads, head_dim,
                                 float(eps), _ptr(rope_table), rope_table.shape[0], _ptr(k_out),
                                 _ptr(v_out), _ptr(workspace), ws_bytes, _stream(stream)))


def alloc_workspace(nbytes: int, device="cuda") -> Optional[torch.Tensor]:
    """A zero-filled, 256-byte aligned workspace of at least ``nbytes`` bytes."""
    if nbytes == 0:
        return None
    return torch.zeros((nbytes + 255) // 256 * 256, dtype=torch.uint8, device=device)


def make_paged_ctx(block_table: torch.Tensor, num_pages: int, page_size: int = 16) -> PagedCtx:
    """``block_table``: device int32 [num_reqs, max_pages_per_req]."""
    if block_table.dtype != torch.int32 or block_table.dim() != 2:
        raise ValueError("block_table must be a 2-D int32 tensor")
    rec = PagedCtx(_ptr(block_table), block_table.shape[1], page_size, num_pages)
    rec._keep = block_table  # the record holds its pointer
    return rec


def dflash_block_attention_paged_workspace_size(p: BlockAttnParams) -> int:
    return load().dflash_block_attention_paged_workspace_size(ctypes.byref(p))


def dflash_block_attention_paged(p: BlockAttnParams, pg: PagedCtx, cu_ctx_lens: torch.Tensor,
                                 cu_blk_lens: torch.Tensor, q: torch.Tensor, k_blk: torch.Tensor,
                                 v_blk: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor,
                                 out: torch.Tensor, workspace: Optional[torch.Tensor], stream=None,
                                 prologue: Optional[QkPrologue] = None) -> None:
    """Block attention over a paged context store (pools ``[pages, 16, Hkv, Dh]``)."""
    lib = load()
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.dflash_block_attention_paged(ctypes.byref(p), ctypes.byref(pg),
                                            ctypes.byref(prologue) if prologue is not None else None,
                                            _ptr(cu_ctx_lens), _ptr(cu_blk_lens), _ptr(q),
                                            _ptr(k_blk), _ptr(v_blk), _ptr(k_pool), _ptr(v_pool),
                                            _ptr(out), _ptr(workspace), ws_bytes, _stream(stream)))


def dflash_kv_scatter(k_src: torch.Tensor, v_src: torch.Tensor, slot_mapping: torch.Tensor,
                      k_pool: torch.Tensor, v_pool: torch.Tensor, stream=None) -> None:
    """Rows of ``k_src``/``v_src`` ``[T, Hkv, Dh]`` to pool slots (pools viewed as
    ``[slots, Hkv, Dh]``); slots outside the pool (e.g. -1) are skipped."""
    lib = load()
    t, hkv, dh = k_src.shape
    num_slots = k_pool.numel() // (hkv * dh)
    _check(lib.dflash_kv_scatter(_dtype_code(k_src), _ptr(k_src), _ptr(v_src), _ptr(slot_mapping),
                                 t, hkv, dh, _ptr(k_pool), _ptr(v_pool), num_slots,
                                 _stream(stream)))


def dflash_block_qkv_workspace_size(T: int, hidden_size: int, num_q_heads: int,
                                    num_kv_heads: int, head_dim: int) -> int:
    return load().dflash_block_qkv_workspace_size(T, hidden_size, num_q_heads, num_kv_heads,
                                                  head_dim)


def dflash_block_qkv(hidden: torch.Tensor, residual: Optional[torch.Tensor], norm_w: torch.Tensor,
                     w_qkv: torch.Tensor, num_q_heads: int, num_kv_heads: int, head_dim: int,
                     eps: float, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                     workspace: Optional[torch.Tensor], stream=None) -> None:
    """Input norm (residual add + RMSNorm) and the merged q/k/v projection of
    ``hidden [T, H]``; q, k, v are written raw."""
    lib = load()
    t, h = hidden.shape
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.dflash_block_qkv(_ptr(hidden), _ptr(residual), _ptr(norm_w), _ptr(w_qkv), t, h,
                                num_q_heads, num_kv_heads, head_dim, float(eps), _ptr(q), _ptr(k),
                                _ptr(v), _ptr(workspace), ws_bytes, _stream(stream)))


def dflash_o_proj_workspace_size(T: int, hidden_size: int, in_dim: int) -> int:
    return load().dflash_o_proj_workspace_size(T, hidden_size, in_dim)


def dflash_o_proj(attn: torch.Tensor, w_o: torch.Tensor, out: torch.Tensor,
                  workspace: Optional[torch.Tensor], stream=None) -> None:
    """``out [T, H] = attn [T, in_dim] @ w_o [H, in_dim]^T`` (attn may be [T, Hq, Dh])."""
    lib = load()
    t = attn.shape[0]
    in_dim = attn.numel() // max(t, 1) if t > 0 else w_o.shape[1]
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.dflash_o_proj(_ptr(attn), _ptr(w_o), t, w_o.shape[0], in_dim, _ptr(out),
                             _ptr(workspace), ws_bytes, _stream(stream)))


def dflash_prepare_inputs(params: PrepareParams, inputs: dict, outputs: dict, stream=None) -> None:
    """``inputs`` / ``outputs``: device int32 tensors keyed by the field names
    of ``dflash_prepare_inputs_in`` / ``_out``."""
    lib = load()
    pin = PrepareIn(*[_ptr(inputs[n]) for n in PREP_IN])
    pout = PrepareOut(*[_ptr(outputs[n]) for n in PREP_OUT])
    _check(lib.dflash_prepare_inputs(ctypes.byref(params), ctypes.byref(pin), ctypes.byref(pout),
                                     _stream(stream)))


def dflash_fc_combine_workspace_size(T: int, hidden_size: int, num_taps: int) -> int:
    return load().dflash_fc_combine_workspace_size(T, hidden_size, num_taps)


def dflash_fc_combine(aux: torch.Tensor, w_fc: torch.Tensor, out: torch.Tensor,
                      workspace: Optional[torch.Tensor], stream=None) -> None:
    """``out [T, H] = bf16(aux [T, H * taps]) @ w_fc [H, H * taps]^T``."""
    lib = load()
    t = aux.shape[0]
    h = w_fc.shape[0]
    taps = w_fc.shape[1] // h
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.dflash_fc_combine(_ptr(aux), _ptr(w_fc), t, h, taps, _ptr(out), _ptr(workspace),
                                 ws_bytes, _stream(stream)))
