"""MI355X (gfx950) 64-token block-sparse attention, VSA style: forward, backward, k2q inversion.

A thin ctypes binding over ``libvsa.so`` (the C ABI in ``include/vsa.h``). This layer only checks
tensor metadata (device, dtype, shape, contiguity -- never tensor contents), allocates outputs and
workspaces with PyTorch, and passes raw device pointers plus the current HIP stream. Every step of
the computation runs in the library's HIP kernels; there is no CPU path. If the library is not
built, every entry point raises.

Semantics follow the FastVideo pages (sm_100a backward commit message; the backward Python
module: ``is_supported``, ``block_sparse_attn_backward_sm100a_from_k2q`` and the q2k entry that
inverts first; the forward module docstring for the lse "M form"):
  * activations are bf16 ``[B, H, S, 128]`` contiguous (BHSD), ``S = 64 * num_kv_blocks``;
  * ``lse = max(q k^T * sm_scale * log2 e) + log2(l)``, fp32 ``[B, H, S]``;
  * ``sm_scale = 1 / sqrt(head_dim)``; dq and dk carry it, dv does not;
  * kv blocks no q block selects get exact-zero dk/dv rows, as do kv rows at or past vbs;
  * the gradient with respect to lse is not supported (the pages' backward ignores it).
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Tuple

import torch

__all__ = [
    "BLOCK", "HEAD_DIM", "ORDER_MIN_KV_BLOCKS", "ORDER_BIN_WIDTH", "CHUNK_MIN_KV_BLOCKS",
    "CHUNK_BLOCKS", "SPILL_CHUNK_BLOCKS", "FWD_CHUNK_KV_BLOCKS", "FWD_CHUNK_MIN_KV_BLOCKS",
    "fwd_workspace_bytes", "library_path", "is_built", "is_supported",
    "invert_indices", "forward", "backward_from_k2q", "backward", "bwd_order",
    "bwd_workspace_bytes", "bwd_workspace_offset", "invert_workspace_bytes", "BwdPlan",
    "DQ_RECOMPUTE", "DQ_SPILL", "default_dq_mode", "backward_noalloc", "NOALLOC_SCRATCH_BYTES",
]

BLOCK = 64
HEAD_DIM = 128
ORDER_MIN_KV_BLOCKS = 64   # VSA_ORDER_MIN_KV_BLOCKS
ORDER_BIN_WIDTH = 4        # VSA_ORDER_BIN_WIDTH
CHUNK_MIN_KV_BLOCKS = 4096  # VSA_CHUNK_MIN_KV_BLOCKS
CHUNK_BLOCKS = 1024       # VSA_CHUNK_BLOCKS
SPILL_CHUNK_BLOCKS = 512  # VSA_SPILL_CHUNK_BLOCKS
FWD_CHUNK_KV_BLOCKS = 512   # VSA_FWD_CHUNK_KV_BLOCKS
FWD_CHUNK_MIN_KV_BLOCKS = 1024  # VSA_FWD_CHUNK_MIN_KV_BLOCKS
ORDER_MAX_KV_BLOCKS = 16384
_LOG2E = 1.4426950408889634

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libvsa.so")
_lib = None

_p = ctypes.c_void_p


class _FwdArgs(ctypes.Structure):
    _fields_ = [("q", _p), ("k", _p), ("v", _p), ("q2k_idx", _p), ("q2k_num", _p), ("vbs", _p),
                ("o", _p), ("lse", _p), ("batch", ctypes.c_int), ("heads", ctypes.c_int),
                ("seqlen", ctypes.c_int), ("head_dim", ctypes.c_int),
                ("num_kv_blocks", ctypes.c_int), ("q2k_stride", ctypes.c_int),
                ("sm_scale", ctypes.c_float), ("workspace", _p),
                ("workspace_bytes", ctypes.c_size_t), ("kv_chunk_blocks", ctypes.c_int)]


class _BwdArgs(ctypes.Structure):
    _fields_ = [("q", _p), ("k", _p), ("v", _p), ("o", _p), ("dout", _p), ("lse", _p),
                ("k2q_idx", _p), ("k2q_num", _p), ("q2k_idx", _p), ("q2k_num", _p), ("vbs", _p),
                ("order", _p), ("dq", _p), ("dk", _p), ("dv", _p), ("workspace", _p),
                ("workspace_bytes", ctypes.c_size_t), ("batch", ctypes.c_int),
                ("heads", ctypes.c_int), ("seqlen", ctypes.c_int), ("head_dim", ctypes.c_int),
                ("num_kv_blocks", ctypes.c_int), ("max_q_blocks", ctypes.c_int),
                ("q2k_stride", ctypes.c_int), ("sm_scale", ctypes.c_float),
                ("dq_mode", ctypes.c_int), ("chunk_blocks", ctypes.c_int)]


# workspace regions of the backward (vsa_bwd_ws_region)
(WS_LSE_DELTA, WS_KV_ORDER, WS_Q_ORDER, WS_Q2K_NUM, WS_Q2K_IDX, WS_BITMAP, WS_KBASE, WS_QENT,
 WS_DS, WS_CHUNK_BOUNDS, WS_DKV_PART, WS_DQ_BOUNDS, WS_DQ_PART, WS_STATS, WS_SCALES, WS_Q16,
 WS_K16, WS_DO16, WS_V16, WS_END) = range(20)
# words of a head's entry in WS_SCALES (vsa.h): the fp16 operands are q 2^-eq, k 2^-ek, v 2^-ev,
# dO 2^-eo, P 2^pp and dS 2^es; c = fp32(sm_scale log2 e) 2^(eq + ek), stored as fp32 bits
SC_EQ, SC_EK, SC_EV, SC_EO, SC_PP, SC_ES, SC_C = range(7)
# how the q-major kernel gets dS (vsa_dq_mode): recomputed from Q, K, V, dO, or spilled by the
# kv-major kernel into the workspace (8 KiB per possible pair)
DQ_RECOMPUTE, DQ_SPILL = 0, 1


# name -> (restype, argtypes); exactly the symbols include/vsa.h declares
_SIGNATURES = {
    "vsa_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "vsa_last_error": (ctypes.c_char_p, []),
    "vsa_invert_workspace_bytes": (ctypes.c_size_t, [ctypes.c_int] * 4),
    "vsa_invert_indices": (ctypes.c_int, [_p, _p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                          ctypes.c_int, ctypes.c_int, _p, _p, _p,
                                          ctypes.c_size_t, _p]),
    "vsa_fwd_workspace_bytes": (ctypes.c_size_t, [ctypes.c_int] * 4),
    "vsa_fwd_check": (ctypes.c_int, [ctypes.POINTER(_FwdArgs)]),
    "vsa_fwd": (ctypes.c_int, [ctypes.POINTER(_FwdArgs), _p]),
    "vsa_bwd_workspace_bytes": (ctypes.c_size_t, [ctypes.c_int] * 6),
    "vsa_bwd_workspace_offset": (ctypes.c_size_t, [ctypes.c_int] * 7),
    "vsa_bwd_check": (ctypes.c_int, [ctypes.POINTER(_BwdArgs)]),
    "vsa_bwd": (ctypes.c_int, [ctypes.POINTER(_BwdArgs), _p]),
    "vsa_bwd_stage": (ctypes.c_int, [ctypes.POINTER(_BwdArgs), ctypes.c_int, _p]),
    "vsa_bwd_order": (ctypes.c_int, [_p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                     _p, _p]),
    "vsa_bwd_noalloc": (ctypes.c_int, [ctypes.POINTER(_BwdArgs), _p]),
}
NOALLOC_SCRATCH_BYTES = 512 << 20  # VSA_NOALLOC_SCRATCH_BYTES


def library_path() -> str:
    return _LIB_PATH


def is_built() -> bool:
    return os.path.exists(_LIB_PATH)


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it is not built (there is no fallback)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is not built; run `python -m "
                               "block_sparse_attention_attn_amd.build` (needs hipcc)")
        handle = ctypes.CDLL(_LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def _check(status: int, what: str) -> None:
    if status != 0:
        L = lib()
        msg = L.vsa_last_error().decode()
        raise RuntimeError(f"{what}: {L.vsa_status_string(status).decode()}: {msg}")


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _need_gpu(t: torch.Tensor, name: str) -> None:
    if not t.is_cuda:
        raise RuntimeError(f"{name} must be a GPU tensor (this library has no CPU path)")


def _act(t: torch.Tensor, name: str, shape) -> None:
    _need_gpu(t, name)
    if t.dtype != torch.bfloat16:
        raise RuntimeError(f"{name} must be bfloat16, got {t.dtype}")
    if t.dim() != 4 or tuple(t.shape) != tuple(shape):
        raise RuntimeError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise RuntimeError(f"{name} must be contiguous")


def _same_device(t: torch.Tensor, name: str, device: torch.device) -> None:
    _need_gpu(t, name)
    if t.device != device:
        raise RuntimeError(f"{name} is on {t.device}, expected {device}")


def _out(t: torch.Tensor, name: str, shape, dtype, device: torch.device) -> torch.Tensor:
    """A caller-supplied output: on the device, of the dtype and shape, contiguous (the kernels
    write it through a raw pointer, so anything else would be written out of bounds)."""
    _same_device(t, name, device)
    if t.dtype != dtype:
        raise RuntimeError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise RuntimeError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise RuntimeError(f"{name} must be contiguous")
    return t


def _workspace(t: Optional[torch.Tensor], need: int, device: torch.device,
               what: str) -> torch.Tensor:
    """The caller's workspace (a contiguous uint8 tensor of at least `need` bytes on the device),
    or a new one."""
    if t is None:
        return torch.empty(max(need, 1), dtype=torch.uint8, device=device)
    _same_device(t, f"{what} workspace", device)
    if t.dtype != torch.uint8 or not t.is_contiguous():
        raise RuntimeError(f"{what} workspace must be a contiguous uint8 tensor, got {t.dtype}"
                           f"{'' if t.is_contiguous() else ' (not contiguous)'}")
    if t.numel() < need:
        raise RuntimeError(f"{what} workspace holds {t.numel()} bytes, needs {need}")
    return t


def _idx(t: torch.Tensor, name: str) -> torch.Tensor:
    """Metadata: an integer GPU tensor, converted to contiguous int32 (value-preserving)."""
    _need_gpu(t, name)
    if t.dtype not in (torch.int32, torch.int64):
        raise RuntimeError(f"{name} must be int32 or int64, got {t.dtype}")
    return t.to(torch.int32).contiguous()


def is_supported(q: torch.Tensor, variable_block_sizes: torch.Tensor) -> bool:
    """Static facts only (never tensor contents): built, GPU tensors, bf16, 4-D, head_dim 128,
    contiguous, integer vbs, S == 64 * num_kv_blocks. Any block count >= 1 is allowed."""
    if not is_built() or not q.is_cuda or not variable_block_sizes.is_cuda:
        return False
    if q.dtype != torch.bfloat16 or q.dim() != 4 or q.shape[-1] != HEAD_DIM:
        return False
    if not q.is_contiguous():
        return False
    if variable_block_sizes.dtype not in (torch.int32, torch.int64):
        return False
    nb = variable_block_sizes.numel()
    return nb > 0 and q.shape[2] == BLOCK * nb


def invert_workspace_bytes(batch: int, heads: int, nq: int, nkv: int) -> int:
    return int(lib().vsa_invert_workspace_bytes(batch, heads, nq, nkv))


def invert_indices(q2k_idx: torch.Tensor, q2k_num: torch.Tensor, num_kv_blocks: int,
                   workspace: Optional[torch.Tensor] = None,
                   out: Optional[Tuple[torch.Tensor, torch.Tensor]] = None):
    """q2k ``[B, H, nq, topk]`` / ``[B, H, nq]`` -> k2q ``[B, H, nkv, nq]`` (ascending, 0-padded)
    and ``[B, H, nkv]``, int32, bit-exact."""
    idx = _idx(q2k_idx, "q2k_idx")
    num = _idx(q2k_num, "q2k_num")
    if idx.dim() != 4 or num.dim() != 3 or tuple(num.shape) != tuple(idx.shape[:3]):
        raise RuntimeError(f"q2k_idx {tuple(idx.shape)} / q2k_num {tuple(num.shape)}: expected "
                           "[B, H, nq, topk] and [B, H, nq]")
    B, H, nq, topk = idx.shape
    dev = idx.device
    _same_device(num, "q2k_num", dev)
    if out is None:
        k2q_idx = torch.empty((B, H, num_kv_blocks, nq), dtype=torch.int32, device=dev)
        k2q_num = torch.empty((B, H, num_kv_blocks), dtype=torch.int32, device=dev)
    else:
        k2q_idx = _out(out[0], "k2q_idx out", (B, H, num_kv_blocks, nq), torch.int32, dev)
        k2q_num = _out(out[1], "k2q_num out", (B, H, num_kv_blocks), torch.int32, dev)
    need = invert_workspace_bytes(B, H, nq, num_kv_blocks)
    workspace = _workspace(workspace, need, dev, "invert_indices")
    st = lib().vsa_invert_indices(idx.data_ptr(), num.data_ptr(), B, H, nq, topk, num_kv_blocks,
                                  k2q_idx.data_ptr(), k2q_num.data_ptr(), workspace.data_ptr(),
                                  workspace.numel() * workspace.element_size(), _stream(dev))
    _check(st, "vsa_invert_indices")
    return k2q_idx, k2q_num


def fwd_workspace_bytes(batch: int, heads: int, seqlen: int, kv_chunk_blocks: int = 0) -> int:
    """Forward workspace bytes: the fp16 copy of v (2 bytes per element) and, with kv-range chunks,
    the chunk bounds and per-wave state."""
    return int(lib().vsa_fwd_workspace_bytes(batch, heads, seqlen, kv_chunk_blocks))


def forward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, q2k_idx: torch.Tensor,
            q2k_num: torch.Tensor, variable_block_sizes: torch.Tensor,
            sm_scale: Optional[float] = None,
            out: Optional[Tuple[torch.Tensor, torch.Tensor]] = None,
            kv_chunk_blocks: int = 0, workspace: Optional[torch.Tensor] = None):
    """Block-sparse forward: returns ``(o bf16 [B,H,S,128], lse fp32 [B,H,S] M form)``.
    ``kv_chunk_blocks``: kv blocks per kv-range chunk (0: the library's choice, chunks of
    FWD_CHUNK_KV_BLOCKS from FWD_CHUNK_MIN_KV_BLOCKS kv blocks on; negative: one launch). The
    workspace (``fwd_workspace_bytes``: the fp16 copy of v, and the chunk state) is allocated
    here unless given."""
    _need_gpu(q, "q")
    if q.dim() != 4:
        raise RuntimeError(f"q must be 4-D, got {q.dim()} dims")
    B, H, S, D = q.shape
    dev = q.device
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _act(t, n, (B, H, S, D))
        _same_device(t, n, dev)
    idx = _idx(q2k_idx, "q2k_idx")
    num = _idx(q2k_num, "q2k_num")
    vbs = _idx(variable_block_sizes, "variable_block_sizes")
    for t, n in ((idx, "q2k_idx"), (num, "q2k_num"), (vbs, "variable_block_sizes")):
        _same_device(t, n, dev)
    nb = vbs.numel()
    if idx.dim() != 4:
        idx = idx.view(B, H, -1, idx.shape[-1])
    if num.dim() != 3:
        num = num.view(B, H, -1)
    if idx.shape[2] != nb or num.shape[2] != nb:
        raise RuntimeError(f"q2k metadata must have num_kv_blocks = {nb} q blocks per (b, h)")
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(D)
    if out is None:
        o = torch.empty_like(q)
        lse = torch.empty((B, H, S), dtype=torch.float32, device=dev)
    else:
        o = _out(out[0], "o out", (B, H, S, D), torch.bfloat16, dev)
        lse = _out(out[1], "lse out", (B, H, S), torch.float32, dev)
    need = fwd_workspace_bytes(B, H, S, kv_chunk_blocks)
    workspace = _workspace(workspace, need, dev, "forward")
    a = _FwdArgs(q.data_ptr(), k.data_ptr(), v.data_ptr(), idx.data_ptr(), num.data_ptr(),
                 vbs.data_ptr(), o.data_ptr(), lse.data_ptr(), B, H, S, D, nb, idx.shape[-1],
                 float(sm_scale), _ptr(workspace),
                 workspace.numel() * workspace.element_size() if workspace is not None else 0,
                 int(kv_chunk_blocks))
    _check(lib().vsa_fwd(ctypes.byref(a), _stream(q.device)), "vsa_fwd")
    return o, lse


def bwd_workspace_bytes(batch: int, heads: int, seqlen: int, q2k_stride: int = 0,
                        dq_mode: int = DQ_RECOMPUTE, chunk_blocks: int = 0) -> int:
    """Workspace bytes of a backward call; ``q2k_stride`` is the row width of the q2k lists the
    call passes, 0 when the library derives them; ``chunk_blocks`` as for ``BwdPlan``."""
    return int(lib().vsa_bwd_workspace_bytes(batch, heads, seqlen, q2k_stride, dq_mode,
                                             chunk_blocks))


def bwd_workspace_offset(batch: int, heads: int, seqlen: int, region: int, q2k_stride: int = 0,
                         dq_mode: int = DQ_RECOMPUTE, chunk_blocks: int = 0) -> int:
    """Byte offset of a backward workspace region (WS_LSE_DELTA, WS_KV_ORDER, ...)."""
    return int(lib().vsa_bwd_workspace_offset(batch, heads, seqlen, q2k_stride, dq_mode,
                                              chunk_blocks, region))


def default_dq_mode(batch: int, heads: int, seqlen: int, q2k_stride: int = 0,
                    chunk_blocks: int = 0, device=None) -> int:
    """The dQ mode a backward call uses when the caller names none: DQ_SPILL (dQ from the dS
    tiles the kv-major kernel writes: one GEMM per pair, the faster mode) when its workspace --
    8 KiB per possible pair, B*H*nb*K tiles for q2k rows of width K (nb when the library derives
    them; with chunks of R q blocks, B*H*R*K: the spill then holds one chunk's tiles) plus the
    slot tables and the rest -- takes at most 1/3 of the device's memory and the spill's size
    limits hold (at most 65535 kv blocks, nb*K below 2^31); DQ_RECOMPUTE otherwise. The choice
    depends only on the shape and the device (not on the memory free at the time), so a given
    call always runs the same kernels and gives the same bits. On MI355X (288 GB): 32768 tokens
    with top-k 128 spill into 4 GiB, 65536 tokens into 8 GiB, 524288 tokens with top-k 2048
    (B*H = 8) into 72 GiB in chunks of SPILL_CHUNK_BLOCKS (the whole spill would need 1 TiB)."""
    nb = seqlen // BLOCK
    kq = q2k_stride if q2k_stride > 0 else nb
    if nb > 65535 or nb * kq >= 1 << 31:
        return DQ_RECOMPUTE
    need = bwd_workspace_bytes(batch, heads, seqlen, q2k_stride, DQ_SPILL, chunk_blocks)
    total = _total_memory(device)
    return DQ_SPILL if 0 < need <= total // 3 else DQ_RECOMPUTE


_TOTAL_MEMORY = {}


def _total_memory(device) -> int:
    dev = torch.device(device if device is not None else "cuda")
    idx = dev.index if dev.index is not None else torch.cuda.current_device()
    if idx not in _TOTAL_MEMORY:
        _TOTAL_MEMORY[idx] = torch.cuda.get_device_properties(idx).total_memory
    return _TOTAL_MEMORY[idx]


def bwd_order(k2q_num: torch.Tensor, bin_width: int = ORDER_BIN_WIDTH,
              out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Length-binned work order ``[B*H*nb]`` int32 of item ids (b*H + h)*nb + kv."""
    num = _idx(k2q_num, "k2q_num")
    if num.dim() != 3:
        raise RuntimeError("k2q_num must be [B, H, nb]")
    B, H, nb = num.shape
    order = (_out(out, "order out", (B * H * nb,), torch.int32, num.device) if out is not None
             else torch.empty(B * H * nb, dtype=torch.int32, device=num.device))
    _check(lib().vsa_bwd_order(num.data_ptr(), B, H, nb, bin_width, order.data_ptr(),
                               _stream(num.device)), "vsa_bwd_order")
    return order


class BwdPlan:
    """A checked, ready-to-launch backward call over fixed tensors (argument marshalling only).

    ``run()`` enqueues the whole backward (``vsa_bwd``); ``stage(i)`` enqueues one of its stages
    (``vsa_bwd_stage``: PREPROCESS=0, INDEX=1, DKDV=2, DQ=3), all on the current stream. With
    ``q2k_idx``/``q2k_num`` (the forward's metadata, the same selection as k2q) the library skips
    deriving them. ``chunk_blocks``: blocks per chunk of the main kernels, q blocks of each k2q
    list for the kv-major kernel and kv blocks of each q2k list for the recomputing q-major one
    (0: the library's choice, chunks of CHUNK_BLOCKS -- SPILL_CHUNK_BLOCKS in DQ_SPILL mode --
    for the kv-major kernel alone from CHUNK_MIN_KV_BLOCKS kv blocks on; negative: one launch
    each). In DQ_SPILL mode with chunks the spill holds one chunk's dS tiles and the dQ kernel runs
    after each chunk's kv-major launch, inside stage DKDV (stage DQ then enqueues nothing). The
    plan keeps references to every tensor it points at.
    """

    PREPROCESS, INDEX, DKDV, DQ = 0, 1, 2, 3

    def __init__(self, grad_o, q, k, v, o, lse, k2q_idx, k2q_num, variable_block_sizes,
                 sm_scale=None, order=None, workspace=None, out=None, q2k_idx=None,
                 q2k_num=None, dq_mode=None, chunk_blocks=0):
        _need_gpu(q, "q")
        if q.dim() != 4:
            raise RuntimeError(f"q must be 4-D, got {q.dim()} dims")
        B, H, S, D = q.shape
        dev = q.device
        for t, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o"), (grad_o, "grad_o")):
            _act(t, n, (B, H, S, D))
            _same_device(t, n, dev)
        _same_device(lse, "lse", dev)
        if lse.dtype != torch.float32 or not lse.is_contiguous() or lse.numel() != B * H * S:
            raise RuntimeError(f"lse must be contiguous float32 holding [B, H, S] = {B * H * S} "
                               f"values, got {lse.dtype} with {lse.numel()}")
        idx = _idx(k2q_idx, "k2q_idx")
        num = _idx(k2q_num, "k2q_num")
        vbs = _idx(variable_block_sizes, "variable_block_sizes")
        for t, n in ((idx, "k2q_idx"), (num, "k2q_num"), (vbs, "variable_block_sizes")):
            _same_device(t, n, dev)
        nb = vbs.numel()
        if S != BLOCK * nb:
            raise RuntimeError(f"seqlen {S} must equal num_kv_blocks ({nb}) * {BLOCK}")
        if idx.dim() not in (2, 4) or idx.numel() != B * H * nb * idx.shape[-1]:
            raise RuntimeError(f"k2q_idx has shape {tuple(idx.shape)}, expected "
                               f"[{B},{H},{nb},max_q] or [{B * H * nb},max_q]")
        if num.numel() != B * H * nb:
            raise RuntimeError(f"k2q_num must hold {B * H * nb} counts, got {num.numel()}")
        if order is not None:
            order = _idx(order, "order")
            _same_device(order, "order", dev)
            if order.numel() != B * H * nb:
                raise RuntimeError(f"order must hold {B * H * nb} item ids")
        qidx = qnum = None
        if (q2k_idx is None) != (q2k_num is None):
            raise RuntimeError("give both q2k_idx and q2k_num, or neither")
        if q2k_idx is not None:
            qidx = _idx(q2k_idx, "q2k_idx")
            qnum = _idx(q2k_num, "q2k_num")
            _same_device(qidx, "q2k_idx", dev)
            _same_device(qnum, "q2k_num", dev)
            if qidx.numel() != B * H * nb * qidx.shape[-1] or qnum.numel() != B * H * nb:
                raise RuntimeError(f"q2k metadata must be [{B},{H},{nb},stride] and [{B},{H},{nb}]")
        if sm_scale is None:
            sm_scale = 1.0 / math.sqrt(D)
        kq = qidx.shape[-1] if qidx is not None else 0
        if dq_mode is None:
            dq_mode = default_dq_mode(B, H, S, kq, chunk_blocks, dev)
        if out is None:
            out = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
        else:
            out = tuple(_out(t, f"{n} out", (B, H, S, D), torch.bfloat16, dev)
                        for t, n in zip(out, ("dq", "dk", "dv")))
        workspace = _workspace(workspace, bwd_workspace_bytes(B, H, S, kq, dq_mode, chunk_blocks),
                               dev, "backward")
        self.dq_mode = dq_mode
        self.dq, self.dk, self.dv = out
        self.workspace = workspace
        self.device = q.device
        self._keep = (grad_o, q, k, v, o, lse, idx, num, qidx, qnum, vbs, order)
        self.args = _BwdArgs(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                             grad_o.data_ptr(), lse.data_ptr(), idx.data_ptr(), num.data_ptr(),
                             _ptr(qidx), _ptr(qnum), vbs.data_ptr(), _ptr(order),
                             self.dq.data_ptr(), self.dk.data_ptr(), self.dv.data_ptr(),
                             workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                             B, H, S, D, nb, idx.shape[-1],
                             kq, float(sm_scale), int(dq_mode), int(chunk_blocks))
        self._ref = ctypes.byref(self.args)
        _check(lib().vsa_bwd_check(self._ref), "vsa_bwd")

    def run(self):
        _check(lib().vsa_bwd(self._ref, _stream(self.device)), "vsa_bwd")
        return self.dq, self.dk, self.dv

    def stage(self, i: int):
        _check(lib().vsa_bwd_stage(self._ref, i, _stream(self.device)), "vsa_bwd_stage")

    def region(self, r: int, count: int, dtype=torch.int32) -> torch.Tensor:
        """``count`` elements of workspace region ``r`` (WS_LSE_DELTA, WS_KV_ORDER, ...)."""
        a = self.args
        off = bwd_workspace_offset(a.batch, a.heads, a.seqlen, r, a.q2k_stride if a.q2k_idx else 0,
                                   a.dq_mode, a.chunk_blocks)
        nbytes = count * torch.empty(0, dtype=dtype).element_size()
        return self.workspace[off:off + nbytes].view(dtype)

    def lse_delta(self) -> torch.Tensor:
        """The workspace's per-q-block statistics records as fp32 [B, H, nb, 2, 64] (valid after
        PREPROCESS): (pp - lse) / c of the block's 64 rows, then -Delta * 2^-(eo + ev) of its 64
        rows, with the head's words of ``scales()``."""
        a = self.args
        nb = a.seqlen // BLOCK
        n = a.batch * a.heads * a.seqlen * 2
        return self.region(WS_LSE_DELTA, n, torch.float32).view(a.batch, a.heads, nb, 2, BLOCK)

    def scales(self) -> torch.Tensor:
        """The per-head operand scales as int32 [B, H, 8] (valid after PREPROCESS): words SC_EQ,
        SC_EK, SC_EV, SC_EO, SC_PP, SC_ES, then SC_C (fp32 bits) and 0."""
        a = self.args
        return self.region(WS_SCALES, a.batch * a.heads * 8, torch.int32).view(a.batch, a.heads, 8)


def backward_from_k2q(grad_o: torch.Tensor, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                      o: torch.Tensor, lse: torch.Tensor, k2q_idx: torch.Tensor,
                      k2q_num: torch.Tensor, variable_block_sizes: torch.Tensor,
                      sm_scale: Optional[float] = None, order: Optional[torch.Tensor] = None,
                      workspace: Optional[torch.Tensor] = None,
                      out: Optional[Tuple[torch.Tensor, torch.Tensor, torch.Tensor]] = None,
                      q2k_idx: Optional[torch.Tensor] = None,
                      q2k_num: Optional[torch.Tensor] = None, dq_mode: Optional[int] = None,
                      chunk_blocks: int = 0):
    """Backward from k2q metadata (``[B, H, nb, max_q_blocks]`` or ``[B*H*nb, max_q_blocks]``
    plus ``[B, H, nb]`` counts). Returns ``(dq, dk, dv)`` bf16. ``dq_mode`` None picks
    ``default_dq_mode`` (the dS spill when its workspace fits)."""
    return BwdPlan(grad_o, q, k, v, o, lse, k2q_idx, k2q_num, variable_block_sizes,
                   sm_scale=sm_scale, order=order, workspace=workspace, out=out,
                   q2k_idx=q2k_idx, q2k_num=q2k_num, dq_mode=dq_mode,
                   chunk_blocks=chunk_blocks).run()


def backward(grad_o, q, k, v, o, lse, q2k_idx, q2k_num, variable_block_sizes,
             sm_scale: Optional[float] = None, dq_mode: Optional[int] = None,
             chunk_blocks: int = 0):
    """Backward from the forward's q2k metadata: inverts to k2q on the GPU, then runs the
    backward with both lists (the q-major dQ kernel walks q2k, the kv-major kernel k2q). The q2k
    rows must not repeat a kv block. ``dq_mode`` None picks ``default_dq_mode``: with the q2k
    rows given, the dS spill needs 8 KiB per (q block, q2k slot), 4 GiB at 32768 tokens with
    top-k 128. Returns ``(dq, dk, dv)``."""
    B, H = q.shape[0], q.shape[1]
    idx = _idx(q2k_idx, "q2k_idx")
    num = _idx(q2k_num, "q2k_num")
    if idx.dim() != 4:
        idx = idx.view(B, H, -1, idx.shape[-1])
    if num.dim() != 3:
        num = num.view(B, H, -1)
    nb = variable_block_sizes.numel()
    k2q_idx, k2q_num = invert_indices(idx, num, nb)
    return backward_from_k2q(grad_o, q, k, v, o, lse, k2q_idx, k2q_num, variable_block_sizes,
                             sm_scale=sm_scale, q2k_idx=idx, q2k_num=num, dq_mode=dq_mode,
                             chunk_blocks=chunk_blocks)


def backward_noalloc(grad_o, q, k, v, o, lse, k2q_idx, k2q_num, variable_block_sizes, out,
                     sm_scale: Optional[float] = None, q2k_idx: Optional[torch.Tensor] = None,
                     q2k_num: Optional[torch.Tensor] = None, dq_mode: int = DQ_RECOMPUTE,
                     chunk_blocks: int = 0):
    """``vsa_bwd_noalloc``: the backward with its workspace in the library's static scratch
    (NOALLOC_SCRATCH_BYTES per GPU), for callers that cannot allocate. ``out`` = (dq, dk, dv) must
    be given; the metadata must already be contiguous int32 on the device (nothing is converted
    or allocated here). Calls on one GPU share the scratch, so calls that overlap there race.
    Raises if the call's workspace would not fit the scratch."""
    B, H, S, D = q.shape
    dev = q.device
    for t, n in ((k2q_idx, "k2q_idx"), (k2q_num, "k2q_num"), (variable_block_sizes, "vbs"),
                 (q2k_idx, "q2k_idx"), (q2k_num, "q2k_num")):
        if t is not None and (t.dtype != torch.int32 or not t.is_contiguous()):
            raise RuntimeError(f"{n} must be contiguous int32 for backward_noalloc")
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o"), (grad_o, "grad_o")):
        _act(t, n, (B, H, S, D))
        _same_device(t, n, dev)
    _same_device(lse, "lse", dev)
    if lse.dtype != torch.float32 or not lse.is_contiguous() or lse.numel() != B * H * S:
        raise RuntimeError("lse must be contiguous float32 holding [B, H, S] values")
    dq, dk, dv = (_out(t, f"{n} out", (B, H, S, D), torch.bfloat16, dev)
                  for t, n in zip(out, ("dq", "dk", "dv")))
    for t, n in ((k2q_idx, "k2q_idx"), (k2q_num, "k2q_num"), (variable_block_sizes, "vbs")):
        _same_device(t, n, dev)
    nb = variable_block_sizes.numel()
    if (q2k_idx is None) != (q2k_num is None):
        raise RuntimeError("give both q2k_idx and q2k_num, or neither")
    kq = q2k_idx.shape[-1] if q2k_idx is not None else 0
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(D)
    a = _BwdArgs(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), grad_o.data_ptr(),
                 lse.data_ptr(), k2q_idx.data_ptr(), k2q_num.data_ptr(), _ptr(q2k_idx),
                 _ptr(q2k_num), variable_block_sizes.data_ptr(), None, dq.data_ptr(),
                 dk.data_ptr(), dv.data_ptr(), None, 0, B, H, S, D, nb, k2q_idx.shape[-1], kq,
                 float(sm_scale), int(dq_mode), int(chunk_blocks))
    _check(lib().vsa_bwd_noalloc(ctypes.byref(a), _stream(dev)), "vsa_bwd_noalloc")
    return dq, dk, dv
