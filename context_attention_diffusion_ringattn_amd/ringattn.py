"""Python surface of the ring-shard attention library (torch tensors in, out).

PyTorch only provides device memory and the stream; every computation runs in
the HIP library through the C ABI (``include/ringattn.h``).  Tensors are BSHD
(``[batch, seq, heads, head_dim]``, contiguous): Q/K/V bf16 on a ROCm device,
outputs float32; LSE is ``[batch, heads, q_len]`` float32 (natural log).
"""

from __future__ import annotations

import ctypes
import dataclasses
import math
from typing import List, Optional, Sequence, Tuple

import torch

from . import _lib
from ._lib import Plan, RingAttnError, Shape, check, lib, offsets_array


# ------------------------------------------------------------------ config --

@dataclasses.dataclass(frozen=True)
class RingConfig:
    """The subset of ``ContextParallelConfig`` (Parallelism API page) that maps
    onto one GPU's share of ring attention, with the pages' rules checked:

    * ``ring_degree``: number of K/V chunks (ring ranks), >= 1;
    * ``ulysses_degree``: head groups; with ring_degree = 1 this GPU's share is
      full-sequence attention over heads / ulysses_degree heads;
    * ``convert_to_fp32``: output and LSE merged in float32 (default True, the
      mode of every forward call; the bf16 state exists only per ring step,
      ``step_bf16``, to measure the error it causes);
    * ``rotate_method``: only ``"allgather"`` is supported (as on the page);
    * ``ring_anything``: uneven chunks; needs ring_degree > 1 and
      ulysses_degree == 1, inference only, no attention mask (guide, variant
      table and section "Ring Anything Attention");
    * ``ulysses_anything``: uneven sequence and head split over Ulysses; needs
      ulysses_degree > 1 and ring_degree == 1 (section "Ulysses Anything
      Attention").
    ``share(seq_len, heads, rank)`` gives a rank's layout (``cp_share``).
    """

    ring_degree: int = 1
    ulysses_degree: int = 1
    convert_to_fp32: bool = True
    rotate_method: str = "allgather"
    ring_anything: bool = False
    ulysses_anything: bool = False

    def __post_init__(self):
        if self.ring_degree < 1 or self.ulysses_degree < 1:
            raise ValueError("ring_degree and ulysses_degree must be >= 1")
        if not self.convert_to_fp32:
            raise ValueError("convert_to_fp32=False: the forward path always merges in float32 "
                             "(step_bf16 runs the bf16 state per ring step, for measuring its error)")
        if self.rotate_method != "allgather":
            raise ValueError(f"rotate_method {self.rotate_method!r} is not supported; only 'allgather'")
        if self.ring_anything and (self.ring_degree <= 1 or self.ulysses_degree != 1):
            raise ValueError("ring_anything needs ring_degree > 1 and ulysses_degree == 1")
        if self.ulysses_anything and (self.ulysses_degree <= 1 or self.ring_degree != 1):
            raise ValueError("ulysses_anything needs ulysses_degree > 1 and ring_degree == 1")
        if self.ring_anything and self.ulysses_anything:
            raise ValueError("ring_anything and ulysses_anything do not combine")
        if self.ring_degree > _lib.RINGATTN_MAX_CHUNKS:
            raise ValueError(f"ring_degree above {_lib.RINGATTN_MAX_CHUNKS} is not supported")

    def share(self, seq_len: int, heads: int, rank: int) -> dict:
        """The layout of `rank` in this configuration's ring x Ulysses grid."""
        return cp_share(seq_len, heads, ring_degree=self.ring_degree, ulysses_degree=self.ulysses_degree,
                        ring_anything=self.ring_anything, ulysses_anything=self.ulysses_anything, rank=rank)


# ------------------------------------------------------------- marshalling --

def _stream_handle(device: torch.device, stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


def _check_bf16(t: torch.Tensor, name: str) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != torch.bfloat16:
        raise TypeError(f"{name} must be bfloat16 (got {t.dtype})")
    if t.dim() != 4:
        raise ValueError(f"{name} must be [batch, seq, heads, head_dim] (got {tuple(t.shape)})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous BSHD")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a ROCm device (got {t.device})")


def _check_f32(t: torch.Tensor, name: str, shape: Tuple[int, ...], device: torch.device) -> None:
    if t.dtype != torch.float32 or tuple(t.shape) != tuple(shape) or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous float32 tensor of shape {tuple(shape)} "
                         f"(got {t.dtype} {tuple(t.shape)})")
    if t.device != device:
        raise ValueError(f"{name} must be on {device} (got {t.device})")


def _check_device(t: torch.Tensor, name: str, device: torch.device) -> None:
    if t.device != device:
        raise ValueError(f"{name} must be on {device}, the device of q (got {t.device})")


def _shape(q: torch.Tensor, kv_len: int) -> Shape:
    B, Sq, H, D = q.shape
    return Shape(batch=B, heads=H, head_dim=D, reserved=0, q_len=Sq, kv_len=kv_len)


def _ptr(t: Optional[torch.Tensor]) -> ctypes.c_void_p:
    return ctypes.c_void_p(t.data_ptr() if t is not None else 0)


def default_scale(head_dim: int) -> float:
    """1/sqrt(head_dim) as a float32 value."""
    return float(torch.tensor(1.0 / math.sqrt(head_dim), dtype=torch.float32).item())


# ------------------------------------------------------------------- calls --

def chunk_offsets(seq_len: int, n_chunks: int, ring_anything: bool = False) -> List[int]:
    """Chunk partition computed by the library (host code)."""
    arr = (ctypes.c_int64 * (n_chunks + 1))() if n_chunks >= 0 else None
    if arr is None:
        raise ValueError("n_chunks must be >= 0")
    check(lib().ringattn_chunk_offsets(int(seq_len), int(n_chunks), int(bool(ring_anything)), arr),
          "ringattn_chunk_offsets")
    return list(arr)


_library_chunk_offsets = chunk_offsets


def acc_init(out_acc: torch.Tensor, lse_acc: torch.Tensor, stream=None) -> None:
    """Set accumulators to the empty state (out = 0, lse = -inf)."""
    if not isinstance(out_acc, torch.Tensor) or out_acc.dim() != 4:
        raise ValueError("out_acc must be a [batch, seq, heads, head_dim] tensor")
    if out_acc.device.type != "cuda":
        raise ValueError(f"out_acc must be on a ROCm device (got {out_acc.device})")
    B, Sq, H, D = out_acc.shape
    _check_f32(out_acc, "out_acc", (B, Sq, H, D), out_acc.device)
    _check_f32(lse_acc, "lse_acc", (B, H, Sq), out_acc.device)
    shape = Shape(batch=B, heads=H, head_dim=D, reserved=0, q_len=Sq, kv_len=0)
    check(lib().ringattn_acc_init(_ptr(out_acc), _ptr(lse_acc), ctypes.byref(shape),
                                  _stream_handle(out_acc.device, stream)), "ringattn_acc_init")


def new_accumulators(q: torch.Tensor, stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Allocate float32 accumulators for q and set them to the empty state."""
    B, Sq, H, D = q.shape
    out = torch.empty((B, Sq, H, D), dtype=torch.float32, device=q.device)
    lse = torch.empty((B, H, Sq), dtype=torch.float32, device=q.device)
    acc_init(out, lse, stream)
    return out, lse


def new_workspace(nbytes: int, device) -> Optional[torch.Tensor]:
    """A split workspace of ``nbytes`` bytes (None when no workspace is
    needed); its contents on entry do not matter."""
    if not nbytes:
        return None
    return torch.empty((int(nbytes),), dtype=torch.uint8, device=device)


def _workspace_args(workspace: Optional[torch.Tensor], device):
    if workspace is None:
        return _ptr(None), 0
    if not isinstance(workspace, torch.Tensor) or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor")
    _check_device(workspace, "workspace", device)
    return _ptr(workspace), workspace.numel() * workspace.element_size()


def step_plan(q_shape: Sequence[int], kv_len: int, n_splits: int = 0, block_m: int = 0) -> Tuple[int, int, int]:
    """(n_splits, block_m, workspace_bytes) of the plan of a split ring step
    over a chunk of kv_len keys (the plan of a one-chunk forward)."""
    return forward_plan(q_shape, [0, int(kv_len)], n_splits, block_m)


def step(q: torch.Tensor, k_chunk: torch.Tensor, v_chunk: torch.Tensor, out_acc: torch.Tensor,
         lse_acc: torch.Tensor, scale: Optional[float] = None, stream=None, *, n_splits: int = 1,
         block_m: int = 0, workspace: Optional[torch.Tensor] = None) -> None:
    """One ring step: attend q to one K/V chunk and LSE-merge into the float32
    accumulators in place (the merge is fused into the kernel epilogue).

    ``n_splits`` = 1 (default): ``ringattn_step``, one workgroup per query
    tile over the whole chunk.  Otherwise ``ringattn_step_split`` with that
    many key splits (0 = the library's plan); ``workspace`` as from
    ``new_workspace(step_plan(...)[2])``, allocated here when not given."""
    _check_bf16(q, "q")
    _check_bf16(k_chunk, "k_chunk")
    _check_bf16(v_chunk, "v_chunk")
    B, Sq, H, D = q.shape
    if k_chunk.shape != v_chunk.shape or k_chunk.shape[0] != B or k_chunk.shape[2:] != q.shape[2:]:
        raise ValueError(f"k/v chunk shapes {tuple(k_chunk.shape)} / {tuple(v_chunk.shape)} do not match q")
    _check_device(k_chunk, "k_chunk", q.device)
    _check_device(v_chunk, "v_chunk", q.device)
    _check_f32(out_acc, "out_acc", (B, Sq, H, D), q.device)
    _check_f32(lse_acc, "lse_acc", (B, H, Sq), q.device)
    if scale is None:
        scale = default_scale(D)
    shape = _shape(q, k_chunk.shape[1])
    if int(n_splits) == 1 and workspace is None and int(block_m) == 0:
        check(lib().ringattn_step(_ptr(q), _ptr(k_chunk), _ptr(v_chunk), _ptr(out_acc), _ptr(lse_acc),
                                  ctypes.c_float(scale), ctypes.byref(shape), _stream_handle(q.device, stream)),
              "ringattn_step")
        return
    plan = Plan(n_splits=int(n_splits), block_m=int(block_m), workspace_bytes=0)
    if workspace is None:
        workspace = new_workspace(step_plan(q.shape, k_chunk.shape[1], n_splits, block_m)[2], q.device)
    ws_ptr, ws_len = _workspace_args(workspace, q.device)
    check(lib().ringattn_step_split(_ptr(q), _ptr(k_chunk), _ptr(v_chunk), _ptr(out_acc), _ptr(lse_acc),
                                    ctypes.c_float(scale), ctypes.byref(shape), ctypes.byref(plan), ws_ptr, ws_len,
                                    _stream_handle(q.device, stream)), "ringattn_step_split")


def new_accumulators_bf16(q: torch.Tensor, stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """bf16 accumulators for q (the convert_to_fp32=False mode) set to the
    empty state by ``ringattn_acc_init_bf16``."""
    B, Sq, H, D = q.shape
    out = torch.empty((B, Sq, H, D), dtype=torch.bfloat16, device=q.device)
    lse = torch.empty((B, H, Sq), dtype=torch.bfloat16, device=q.device)
    shape = Shape(batch=B, heads=H, head_dim=D, reserved=0, q_len=Sq, kv_len=0)
    check(lib().ringattn_acc_init_bf16(_ptr(out), _ptr(lse), ctypes.byref(shape), _stream_handle(q.device, stream)),
          "ringattn_acc_init_bf16")
    return out, lse


def step_bf16(q: torch.Tensor, k_chunk: torch.Tensor, v_chunk: torch.Tensor, out_acc: torch.Tensor,
              lse_acc: torch.Tensor, scale: Optional[float] = None, stream=None) -> None:
    """One ring step with bf16 accumulators (``ringattn_step_bf16``): the
    partial is rounded to bf16, merged, and the state stored as bf16."""
    _check_bf16(q, "q")
    _check_bf16(k_chunk, "k_chunk")
    _check_bf16(v_chunk, "v_chunk")
    B, Sq, H, D = q.shape
    if k_chunk.shape != v_chunk.shape or k_chunk.shape[0] != B or k_chunk.shape[2:] != q.shape[2:]:
        raise ValueError(f"k/v chunk shapes {tuple(k_chunk.shape)} / {tuple(v_chunk.shape)} do not match q")
    _check_device(k_chunk, "k_chunk", q.device)
    _check_device(v_chunk, "v_chunk", q.device)
    for t, name, shp in ((out_acc, "out_acc", (B, Sq, H, D)), (lse_acc, "lse_acc", (B, H, Sq))):
        if t.dtype != torch.bfloat16 or tuple(t.shape) != shp or not t.is_contiguous() or t.device != q.device:
            raise ValueError(f"{name} must be a contiguous bf16 tensor of shape {shp} on {q.device}")
    if scale is None:
        scale = default_scale(D)
    shape = _shape(q, k_chunk.shape[1])
    check(lib().ringattn_step_bf16(_ptr(q), _ptr(k_chunk), _ptr(v_chunk), _ptr(out_acc), _ptr(lse_acc),
                                   ctypes.c_float(scale), ctypes.byref(shape), _stream_handle(q.device, stream)),
          "ringattn_step_bf16")


def merge(out_acc: torch.Tensor, lse_acc: torch.Tensor, out_part: torch.Tensor, lse_part: torch.Tensor,
          stream=None) -> None:
    """LSE-merge a float32 partial into the accumulators in place."""
    if not isinstance(out_acc, torch.Tensor) or out_acc.dim() != 4:
        raise ValueError("out_acc must be a [batch, seq, heads, head_dim] tensor")
    if out_acc.device.type != "cuda":
        raise ValueError(f"out_acc must be on a ROCm device (got {out_acc.device})")
    B, Sq, H, D = out_acc.shape
    _check_f32(out_acc, "out_acc", (B, Sq, H, D), out_acc.device)
    _check_f32(out_part, "out_part", (B, Sq, H, D), out_acc.device)
    _check_f32(lse_acc, "lse_acc", (B, H, Sq), out_acc.device)
    _check_f32(lse_part, "lse_part", (B, H, Sq), out_acc.device)
    shape = Shape(batch=B, heads=H, head_dim=D, reserved=0, q_len=Sq, kv_len=0)
    check(lib().ringattn_merge(_ptr(out_acc), _ptr(lse_acc), _ptr(out_part), _ptr(lse_part),
                               ctypes.byref(shape), _stream_handle(out_acc.device, stream)), "ringattn_merge")


def forward_plan(q_shape: Sequence[int], offsets: Sequence[int], n_splits: int = 0, block_m: int = 0,
                 kv_chunk_stride: int = 0) -> Tuple[int, int, int]:
    """(n_splits, block_m, workspace_bytes) of the plan the library uses for a
    forward call; n_splits / block_m = 0 let the library choose."""
    B, Sq, H, D = q_shape
    shape = Shape(batch=B, heads=H, head_dim=D, reserved=0, q_len=Sq, kv_len=int(offsets[-1]))
    plan = Plan(n_splits=int(n_splits), block_m=int(block_m), workspace_bytes=0)
    arr = offsets_array(offsets)
    check(lib().ringattn_forward_plan(ctypes.byref(shape), arr, len(offsets) - 1, int(kv_chunk_stride),
                                      ctypes.byref(plan)), "ringattn_forward_plan")
    return plan.n_splits, plan.block_m, plan.workspace_bytes


def forward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *,
            chunk_offsets: Optional[Sequence[int]] = None,
            ring_degree: Optional[int] = None,
            ring_anything: bool = False,
            kv_chunk_stride: int = 0,
            scale: Optional[float] = None,
            n_splits: int = 0,
            block_m: int = 0,
            out: Optional[torch.Tensor] = None,
            lse: Optional[torch.Tensor] = None,
            workspace: Optional[torch.Tensor] = None,
            convert_to_fp32: bool = True,
            stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """The whole shard: q attends to every K/V chunk; returns (out fp32, lse fp32).

    Give either ``chunk_offsets`` (n_chunks + 1 host integers) or
    ``ring_degree`` (+ ``ring_anything``) to partition the K/V rows.  With
    ``kv_chunk_stride`` > 0, k/v are the padded all-gather buffer of Ring
    Anything (chunk c at rows ``c * kv_chunk_stride``, true lengths from the
    offsets).  Buffers not passed in are allocated with torch on q's device.
    """
    if not convert_to_fp32:
        raise ValueError("convert_to_fp32=False: the forward path always merges in float32 "
                         "(step_bf16 runs the bf16 state per ring step, for measuring its error)")
    _check_bf16(q, "q")
    _check_bf16(k, "k")
    _check_bf16(v, "v")
    B, Sq, H, D = q.shape
    if k.shape != v.shape or k.shape[0] != B or k.shape[2:] != q.shape[2:]:
        raise ValueError(f"k/v shapes {tuple(k.shape)} / {tuple(v.shape)} do not match q {tuple(q.shape)}")
    _check_device(k, "k", q.device)
    _check_device(v, "v", q.device)
    if chunk_offsets is None:
        if ring_degree is None:
            ring_degree = 1
        n = int(ring_degree)
        if kv_chunk_stride:
            raise ValueError("kv_chunk_stride needs explicit chunk_offsets")
        chunk_offsets = _library_chunk_offsets(k.shape[1], n, ring_anything)
    offs = [int(x) for x in chunk_offsets]
    n_chunks = len(offs) - 1
    rows_needed = n_chunks * int(kv_chunk_stride) if kv_chunk_stride else offs[-1]
    if k.shape[1] != rows_needed:
        raise ValueError(f"k/v hold {k.shape[1]} rows per batch, the chunk layout needs {rows_needed}")
    if scale is None:
        scale = default_scale(D)
    if out is None:
        out = torch.empty((B, Sq, H, D), dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty((B, H, Sq), dtype=torch.float32, device=q.device)
    _check_f32(out, "out", (B, Sq, H, D), q.device)
    _check_f32(lse, "lse", (B, H, Sq), q.device)
    shape = Shape(batch=B, heads=H, head_dim=D, reserved=0, q_len=Sq, kv_len=offs[-1])
    arr = offsets_array(offs)
    plan = Plan(n_splits=int(n_splits), block_m=int(block_m), workspace_bytes=0)
    if workspace is None:
        check(lib().ringattn_forward_plan(ctypes.byref(shape), arr, n_chunks, int(kv_chunk_stride),
                                          ctypes.byref(plan)), "ringattn_forward_plan")
        workspace = new_workspace(plan.workspace_bytes, q.device)
    ws_ptr, ws_len = _workspace_args(workspace, q.device)
    check(lib().ringattn_forward(_ptr(q), _ptr(k), _ptr(v), arr, n_chunks, int(kv_chunk_stride), _ptr(out), _ptr(lse),
                                 ctypes.c_float(scale), ctypes.byref(shape), ctypes.byref(plan), ws_ptr, ws_len,
                                 _stream_handle(q.device, stream)), "ringattn_forward")
    return out, lse


def ring_sweep(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *,
               chunk_offsets: Optional[Sequence[int]] = None,
               ring_degree: Optional[int] = None,
               ring_anything: bool = False,
               kv_chunk_stride: int = 0,
               scale: Optional[float] = None,
               out: Optional[torch.Tensor] = None,
               lse: Optional[torch.Tensor] = None,
               stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Every rank of the ring on this GPU (``ringattn_ring_sweep``).

    ``q`` is the full sequence ``[B, S, H, D]`` (rank r's shard is rows
    ``[offsets[r], offsets[r+1])``); each rank visits the chunks in the order
    r, r+1, ... (mod N) with a float32 LSE merge after every step.  Returns
    (out ``[B, S, H, D]`` fp32, lse ``[B, H, S]`` fp32) for all ranks' rows.
    """
    _check_bf16(q, "q")
    _check_bf16(k, "k")
    _check_bf16(v, "v")
    B, S, H, D = q.shape
    if k.shape != v.shape or k.shape[0] != B or k.shape[2:] != q.shape[2:]:
        raise ValueError(f"k/v shapes {tuple(k.shape)} / {tuple(v.shape)} do not match q {tuple(q.shape)}")
    _check_device(k, "k", q.device)
    _check_device(v, "v", q.device)
    if chunk_offsets is None:
        if kv_chunk_stride:
            raise ValueError("kv_chunk_stride needs explicit chunk_offsets")
        chunk_offsets = _library_chunk_offsets(S, int(ring_degree or 1), ring_anything)
    offs = [int(x) for x in chunk_offsets]
    n_chunks = len(offs) - 1
    rows_needed = n_chunks * int(kv_chunk_stride) if kv_chunk_stride else offs[-1]
    if k.shape[1] != rows_needed:
        raise ValueError(f"k/v hold {k.shape[1]} rows per batch, the chunk layout needs {rows_needed}")
    if scale is None:
        scale = default_scale(D)
    if out is None:
        out = torch.empty((B, S, H, D), dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty((B, H, S), dtype=torch.float32, device=q.device)
    _check_f32(out, "out", (B, S, H, D), q.device)
    _check_f32(lse, "lse", (B, H, S), q.device)
    shape = Shape(batch=B, heads=H, head_dim=D, reserved=0, q_len=S, kv_len=offs[-1])
    check(lib().ringattn_ring_sweep(_ptr(q), _ptr(k), _ptr(v), offsets_array(offs), n_chunks, int(kv_chunk_stride),
                                    _ptr(out), _ptr(lse), ctypes.c_float(scale), ctypes.byref(shape),
                                    _stream_handle(q.device, stream)), "ringattn_ring_sweep")
    return out, lse


def cp_share(seq_len: int, heads: int, *, ring_degree: int = 1, ulysses_degree: int = 1,
             ring_anything: bool = False, ulysses_anything: bool = False, rank: int = 0) -> dict:
    """Layout of `rank` in the ring x Ulysses grid (``ringattn_cp_layout``):
    ``ring_index``, ``ulysses_index``, its tokens before the Ulysses
    all-to-all (``token_begin``/``token_end``) and the query rows
    (``q_begin``/``q_end``) and heads (``head_begin``/``head_end``) of its
    attention share, which attends to the ring chunks of the same heads."""
    cfg = _lib.CpConfig(seq_len=int(seq_len), heads=int(heads), ring_degree=int(ring_degree),
                        ulysses_degree=int(ulysses_degree), ring_anything=int(bool(ring_anything)),
                        ulysses_anything=int(bool(ulysses_anything)), reserved=0)
    out = _lib.CpShare()
    check(lib().ringattn_cp_layout(ctypes.byref(cfg), int(rank), ctypes.byref(out)), "ringattn_cp_layout")
    return {k: getattr(out, k) for k, _ in _lib.CpShare._fields_}


def ring_shard(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, config: RingConfig, *,
               scale: Optional[float] = None, **kw) -> Tuple[torch.Tensor, torch.Tensor]:
    """Forward for one GPU's share under a ``RingConfig``: ring_degree chunks
    of the K/V sequence (Ring Anything if set).  For the Ulysses share pass
    the head subset as q/k/v and ring_degree = 1."""
    return forward(q, k, v, ring_degree=config.ring_degree, ring_anything=config.ring_anything,
                   scale=scale, convert_to_fp32=config.convert_to_fp32, **kw)
