"""MoE token dispatch / combine for one MI355X (gfx950).

A thin binding over the C ABI in include/ep_mi355x.h: each function checks
that the torch tensors it is handed are contiguous device tensors of the
right dtype and shape, allocates outputs with torch (device memory is the
only thing torch provides here), and calls the library entry point of the
same name on torch's current stream.  Every step of the path runs in the HIP
kernels; there is no CPU or PyTorch fallback.
"""
from __future__ import annotations

import ctypes
import dataclasses

import torch

from . import _lib
from ._lib import (  # noqa: F401
    EP_COMBINE_FLAT,
    EP_COMBINE_GROUPED,
    EP_FORMAT_BF16,
    EP_FORMAT_FP8_PACKED,
    EP_ROWS_EXPERT,
    EP_ROWS_GROUP,
    EP_STATUS_COMBINE_OOB,
    EP_STATUS_DISPATCH_OVERFLOW,
    EP_STATUS_EXPERT_LIST_OVERFLOW,
    EP_STATUS_GENERATION,
    EP_STATUS_STALE,
    EP_STATUS_INVALID_IDS,
    EP_STATUS_SELECTIONS,
    EP_STATUS_LIST_OVERFLOW,
    EP_STATUS_ROWS_EXPERT,
    EP_STATUS_ROWS_GROUP,
    EP_STATUS_WORDS,
    EPError,
)

__all__ = [
    "Layout",
    "LayoutHandle",
    "StaleLayoutError",
    "ep_fp8_row_bytes",
    "fp8_row_pitch",
    "ep_layout_workspace_bytes",
    "ep_layout",
    "ep_layout_noalloc",
    "alloc_layout",
    "ep_dispatch",
    "ep_combine",
    "ep_expert_gemm",
    "PackedExpertWeights",
    "ep_expert_weights_packed_bytes",
    "ep_pack_expert_weights",
    "ep_strerror",
    "EPError",
]


def _ptr(t: torch.Tensor | None) -> int | None:
    return None if t is None else t.data_ptr()


def _dev(t: torch.Tensor, name: str, dtype: torch.dtype, shape=None) -> torch.Tensor:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor, got {t.device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return t


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _problem(T: int, H: int, K: int, E: int, G: int, A: int = 0, flags: int = 0) -> _lib.Problem:
    return _lib.Problem(T, H, K, E, G, A, flags)


def ep_fp8_row_bytes(hidden: int) -> int:
    """Bytes of one packed fp8 row (H payload bytes, H/128 fp32 scales, 16-byte pad)."""
    return int(_lib.lib().ep_fp8_row_bytes(hidden))


def fp8_row_pitch(hidden: int, align: int = 128) -> int:
    """The packed fp8 row size rounded up to `align` bytes: a receive-row
    pitch that keeps every row on an aligned boundary (7424 for hidden 7168)."""
    rb = ep_fp8_row_bytes(hidden)
    return -1 if rb < 0 else (rb + align - 1) // align * align


def ep_layout_workspace_bytes(num_tokens: int, topk: int, num_experts: int, num_groups: int = 0) -> int:
    p = _problem(num_tokens, 1, topk, num_experts, num_groups)
    return int(_lib.lib().ep_layout_workspace_bytes(ctypes.byref(p)))


def ep_strerror(code: int) -> str:
    return _lib.lib().ep_strerror(code).decode()


class StaleLayoutError(RuntimeError):
    """A LayoutHandle was used after its Layout's buffers were recomputed."""


@dataclasses.dataclass
class Layout:
    """Device outputs of ep_layout plus the shape they were computed for.

    ``generation`` is the value the library's ep_layout stamped on these
    buffers (unique in the process, 0 before the first layout).  A
    LayoutHandle taken with ``handle()`` remembers it, so a dispatch replayed
    from a cached handle is rejected once the buffers hold another routing
    (the PR's cached ``handle=`` dispatch and its stale-layout guard): on the
    host by ``LayoutHandle.get()``, and on the device by the kernels, which
    compare the handle's generation with the one stamped in the status words
    and write nothing on a mismatch (so a replayed HIP graph is guarded too)."""

    num_tokens: int
    topk: int
    num_experts: int
    num_groups: int
    counts: torch.Tensor
    offsets: torch.Tensor
    slot: torch.Tensor
    status: torch.Tensor
    group_counts: torch.Tensor | None = None
    group_offsets: torch.Tensor | None = None
    grow: torch.Tensor | None = None
    row_src: torch.Tensor | None = None
    row_topk_idx: torch.Tensor | None = None
    row_topk_weights: torch.Tensor | None = None
    row_capacity: int = 0
    workspace: torch.Tensor | None = None
    expert_alignment: int = 0
    expert_row_src: torch.Tensor | None = None
    expert_row_capacity: int = 0
    recv_stats: torch.Tensor | None = None
    generation: int = 0

    def struct(self, generation: int | None = None) -> _lib.LayoutStruct:
        """The C struct over these buffers, carrying ``generation`` (default:
        the buffers' current one) for the kernels' stale-layout check."""
        return _lib.LayoutStruct(
            _ptr(self.counts),
            _ptr(self.offsets),
            _ptr(self.slot),
            _ptr(self.status),
            _ptr(self.group_counts),
            _ptr(self.group_offsets),
            _ptr(self.grow),
            _ptr(self.row_src),
            _ptr(self.row_topk_idx),
            _ptr(self.row_topk_weights),
            self.row_capacity,
            _ptr(self.expert_row_src),
            self.expert_row_capacity,
            _ptr(self.recv_stats),
            self.generation if generation is None else int(generation),
        )

    def max_expert_rows(self) -> int:
        pad = self.num_experts * (self.expert_alignment - 1) if self.expert_alignment > 1 else 0
        return self.num_tokens * self.topk + pad

    def max_group_rows(self) -> int:
        return min(self.num_tokens * self.num_groups, self.num_tokens * self.topk)

    def num_rows(self, rows: int = EP_ROWS_EXPERT) -> int:
        """Rows the layout needs (synchronises the stream)."""
        w = EP_STATUS_ROWS_EXPERT if rows == EP_ROWS_EXPERT else EP_STATUS_ROWS_GROUP
        return int(self.status[w].item())

    def handle(self) -> "LayoutHandle":
        return LayoutHandle(self, self.generation)

    def status_word(self, word: int) -> int:
        """One device status word (synchronises the stream)."""
        return int(self.status[word].item())

    def dispatch_overflowed(self) -> bool:
        """Whether the last ep_dispatch on this layout needed more rows than
        its capacity (it then wrote no row).  Synchronises."""
        return self.status_word(EP_STATUS_DISPATCH_OVERFLOW) != 0

    def stale_call_seen(self) -> bool:
        """Whether a call since the last ep_layout was handed a stale
        generation (it then wrote nothing).  Synchronises."""
        return self.status_word(EP_STATUS_STALE) != 0


@dataclasses.dataclass(frozen=True)
class LayoutHandle:
    """A Layout as it was at one generation (see Layout)."""

    layout: Layout
    generation: int

    def get(self) -> Layout:
        if self.layout.generation != self.generation:
            raise StaleLayoutError(
                f"layout recomputed since this handle was taken (generation {self.generation} -> "
                f"{self.layout.generation})"
            )
        return self.layout


def _resolve(layout) -> tuple[Layout, int]:
    """The Layout and the generation a call on it must carry."""
    if isinstance(layout, LayoutHandle):
        return layout.get(), layout.generation
    return layout, layout.generation


def _check_layout_args(topk_idx, num_experts, num_groups, topk_weights, recv_stats):
    if topk_idx.dim() != 2:
        raise ValueError("topk_idx must be [T, K]")
    T, K = topk_idx.shape
    _dev(topk_idx, "topk_idx", torch.int64)
    if topk_weights is not None:
        _dev(topk_weights, "topk_weights", torch.float32, (T, K))
    elif int(num_groups) > 0:
        raise ValueError("grouped layout needs topk_weights for the per-row weight lists")
    if recv_stats is not None:
        if recv_stats.dtype not in (torch.int32, torch.uint32):
            raise TypeError("recv_stats must be a 32-bit integer tensor")
        _dev(recv_stats, "recv_stats", recv_stats.dtype, (num_experts,))
    return T, K


def _alloc_layout(T, K, num_experts, G, A, dev, row_capacity, expert_row_src, recv_stats) -> Layout:
    """A Layout's output buffers for this shape (no workspace)."""
    i32 = dict(dtype=torch.int32, device=dev)
    L = Layout(
        num_tokens=T,
        topk=K,
        num_experts=num_experts,
        num_groups=G,
        counts=torch.empty(num_experts, **i32),
        offsets=torch.empty(num_experts + 1, **i32),
        slot=torch.empty(T, K, **i32),
        status=torch.empty(_lib.EP_STATUS_WORDS, **i32),
        expert_alignment=A,
        recv_stats=recv_stats,
    )
    if expert_row_src:
        L.expert_row_capacity = L.max_expert_rows()
        L.expert_row_src = torch.empty(max(L.expert_row_capacity, 1), **i32)
    if G > 0:
        cap = L.max_group_rows() if row_capacity is None else int(row_capacity)
        L.row_capacity = cap
        L.group_counts = torch.empty(G, **i32)
        L.group_offsets = torch.empty(G + 1, **i32)
        L.grow = torch.empty(T, K, **i32)
        L.row_src = torch.empty(max(cap, 1), **i32)
        L.row_topk_idx = torch.empty(max(cap, 1), K, **i32)
        L.row_topk_weights = torch.empty(max(cap, 1), K, dtype=torch.float32, device=dev)
    return L


def _check_out_shape(out: Layout, T, K, num_experts, G, A) -> None:
    if (out.num_tokens, out.topk, out.num_experts, out.num_groups, out.expert_alignment) != (
        T,
        K,
        num_experts,
        G,
        A,
    ):
        raise ValueError("out was allocated for a different problem shape")


def ep_layout(
    topk_idx: torch.Tensor,
    num_experts: int,
    num_groups: int = 0,
    topk_weights: torch.Tensor | None = None,
    row_capacity: int | None = None,
    out: Layout | None = None,
    expert_alignment: int = 0,
    expert_row_src: bool = False,
    recv_stats: torch.Tensor | None = None,
) -> Layout:
    """Count, scan and place every selection of topk_idx (int64 [T, K]).

    ``expert_alignment`` rounds each expert segment up to a multiple of that
    many rows; ``expert_row_src`` also returns each expert-major row's source
    token (-1 on padding rows); ``recv_stats`` (uint32 as int32 [E]) gets the
    per-expert counts added to it.  ``out`` reuses the buffers of an earlier
    Layout of the same shape (nothing is allocated then; its generation
    advances)."""
    T, K = _check_layout_args(topk_idx, num_experts, num_groups, topk_weights, recv_stats)
    G = int(num_groups)
    A = int(expert_alignment)
    if out is not None:
        _check_out_shape(out, T, K, num_experts, G, A)
        out.recv_stats = recv_stats
        _run_layout(out, topk_idx, topk_weights)
        return out
    L = _alloc_layout(T, K, num_experts, G, A, topk_idx.device, row_capacity, expert_row_src, recv_stats)
    p = _problem(T, 1, K, num_experts, G, A)
    nbytes = int(_lib.lib().ep_layout_workspace_bytes(ctypes.byref(p)))
    if nbytes == 0:
        raise _lib.EPError("ep_layout_workspace_bytes", _lib.EP_EINVAL, "invalid problem shape")
    L.workspace = torch.empty(nbytes, dtype=torch.uint8, device=topk_idx.device)
    _run_layout(L, topk_idx, topk_weights)
    return L


def _run_layout(L: Layout, topk_idx: torch.Tensor, topk_weights: torch.Tensor | None) -> None:
    p = _problem(L.num_tokens, 1, L.topk, L.num_experts, L.num_groups, L.expert_alignment)
    s = L.struct()
    if L.workspace is None:
        raise ValueError("this Layout has no workspace (made by ep_layout_noalloc); pass it to "
                         "ep_layout_noalloc, or make one with ep_layout")
    rc = _lib.lib().ep_layout(
        ctypes.byref(p),
        _ptr(topk_idx),
        _ptr(topk_weights),
        ctypes.byref(s),
        _ptr(L.workspace),
        L.workspace.numel(),
        _stream(topk_idx.device),
    )
    _lib.check("ep_layout", rc)
    L.generation = int(s.generation)


def ep_layout_noalloc(
    topk_idx: torch.Tensor,
    num_experts: int,
    out: Layout,
    topk_weights: torch.Tensor | None = None,
    recv_stats: torch.Tensor | None = None,
) -> Layout:
    """ep_layout into the buffers of ``out`` (a Layout of the same shape, from
    ep_layout or ``alloc_layout``) with no device allocation at all: the
    library keeps the per-block tallies in its own fixed per-GPU scratch
    (EP_LAYOUT_SCRATCH_BYTES), so this call suits code that must not
    allocate (graph capture, serving loops).  Calls on one GPU share that
    scratch and must not overlap in time.  Raises EPError (EP_ESCRATCH) for
    a problem whose tallies do not fit it."""
    T, K = _check_layout_args(topk_idx, num_experts, out.num_groups, topk_weights, recv_stats)
    _check_out_shape(out, T, K, num_experts, out.num_groups, out.expert_alignment)
    out.recv_stats = recv_stats
    p = _problem(T, 1, K, num_experts, out.num_groups, out.expert_alignment)
    s = out.struct()
    rc = _lib.lib().ep_layout_noalloc(
        ctypes.byref(p), _ptr(topk_idx), _ptr(topk_weights), ctypes.byref(s), _stream(topk_idx.device)
    )
    _lib.check("ep_layout_noalloc", rc)
    out.generation = int(s.generation)
    return out


def alloc_layout(
    num_tokens: int,
    topk: int,
    num_experts: int,
    num_groups: int = 0,
    row_capacity: int | None = None,
    expert_alignment: int = 0,
    expert_row_src: bool = False,
    device: torch.device | str = "cuda",
) -> Layout:
    """The output buffers of a layout of this shape, without a workspace, for
    ``ep_layout_noalloc`` (allocate once, outside the code that must not)."""
    return _alloc_layout(int(num_tokens), int(topk), int(num_experts), int(num_groups),
                         int(expert_alignment), torch.device(device), row_capacity, expert_row_src, None)


def ep_dispatch(
    x: torch.Tensor,
    layout: Layout,
    fp8: bool = False,
    rows: int = EP_ROWS_EXPERT,
    capacity: int | None = None,
    out: torch.Tensor | None = None,
    row_stride: int | None = None,
    zero_padding: bool = False,
    check: bool = False,
) -> torch.Tensor:
    """Scatter token rows x (bf16 [T, H]) to their receive rows.

    Returns ``out``: bf16 [capacity, H], or uint8 [capacity, ep_fp8_row_bytes(H)]
    with ``fp8``.  The receive-row pitch is the row size of ``out`` (one row
    of the 2-D tensor per receive row); when ``out`` is allocated here it is
    ``row_stride`` bytes (default: the row size, rows packed back to back).
    Only the first row-size bytes of each row are written, except that fp8
    rows on 128-byte lines (``out`` and the pitch multiples of 128 bytes,
    as with ``fp8_row_pitch``) are zero-filled from their end to the next
    128-byte boundary, so every line is written whole.  The default
    capacity is the worst case (T*K expert rows, min(T*G, T*K) group rows),
    so no host synchronisation is needed.  With a smaller ``capacity`` the
    rows needed may exceed it: the call then writes no row and sets the
    status word EP_STATUS_DISPATCH_OVERFLOW (``layout.dispatch_overflowed()``;
    ``check=True`` synchronises and raises EPError instead).  ``layout`` may
    be a LayoutHandle (checked against its generation, on the host and on
    the device).  ``zero_padding`` also zeroes the expert alignment padding
    rows."""
    layout, gen = _resolve(layout)
    if x.dim() != 2 or x.shape[0] != layout.num_tokens:
        raise ValueError("x must be [T, H] with the layout's T")
    _dev(x, "x", torch.bfloat16)
    T, H = x.shape
    if capacity is None:
        capacity = layout.max_expert_rows() if rows == EP_ROWS_EXPERT else layout.max_group_rows()
    fmt = EP_FORMAT_FP8_PACKED if fp8 else EP_FORMAT_BF16
    if fp8:
        rb = ep_fp8_row_bytes(H)
        if rb < 0:
            raise _lib.EPError("ep_dispatch", _lib.EP_ENOTSUP, "fp8 rows need hidden % 128 == 0")
        dtype, esize = torch.uint8, 1
    else:
        rb = 2 * H
        dtype, esize = torch.bfloat16, 2
    if out is None:
        pitch = rb if row_stride is None else int(row_stride)
        if pitch < rb or pitch % esize:
            raise ValueError(f"row_stride must be a multiple of {esize} and >= {rb}")
        out = torch.empty(max(capacity, 1), pitch // esize, dtype=dtype, device=x.device)
    else:
        _dev(out, "out", dtype)
        if out.dim() != 2 or out.shape[1] * esize < rb or out.shape[0] < capacity:
            raise ValueError(f"out must be {dtype} [>= capacity, >= {rb // esize}]")
        if row_stride is not None and row_stride != out.shape[1] * esize:
            raise ValueError("row_stride disagrees with out's row size")
    pitch = out.shape[1] * esize
    flags = _lib.EP_FLAG_ZERO_PADDING if zero_padding else 0
    p = _problem(T, H, layout.topk, layout.num_experts, layout.num_groups, layout.expert_alignment, flags)
    s = layout.struct(gen)
    rc = _lib.lib().ep_dispatch(
        ctypes.byref(p),
        ctypes.byref(s),
        _ptr(x),
        _ptr(out),
        int(capacity),
        int(pitch),
        int(rows),
        fmt,
        _stream(x.device),
    )
    _lib.check("ep_dispatch", rc)
    if check and T > 0:
        if layout.stale_call_seen():
            raise StaleLayoutError("the layout buffers were recomputed before this dispatch ran")
        if layout.dispatch_overflowed():
            need = layout.num_rows(rows)
            raise _lib.EPError("ep_dispatch", _lib.EP_EINVAL,
                               f"{need} receive rows needed, capacity {capacity}: nothing written")
    return out


def ep_combine(
    y: torch.Tensor,
    layout: Layout,
    topk_weights: torch.Tensor,
    topk_idx: torch.Tensor | None = None,
    order: int = EP_COMBINE_FLAT,
    out: torch.Tensor | None = None,
    bias0: torch.Tensor | None = None,
    bias1: torch.Tensor | None = None,
) -> torch.Tensor:
    """Weighted reduction of each token's expert-output rows y (bf16 [rows, H],
    expert-major) into out (bf16 [T, H]); bias0 / bias1 (bf16 [T, H]) seed the
    accumulator."""
    layout, gen = _resolve(layout)
    if y.dim() != 2:
        raise ValueError("y must be [rows, H]")
    _dev(y, "y", torch.bfloat16)
    T, K = layout.num_tokens, layout.topk
    H = y.shape[1]
    _dev(topk_weights, "topk_weights", torch.float32, (T, K))
    if topk_idx is not None:
        _dev(topk_idx, "topk_idx", torch.int64, (T, K))
    if order == EP_COMBINE_GROUPED and topk_idx is None:
        raise ValueError("grouped order needs topk_idx")
    for name, b in (("bias0", bias0), ("bias1", bias1)):
        if b is not None:
            _dev(b, name, torch.bfloat16, (T, H))
    if out is None:
        out = torch.empty(T, H, dtype=torch.bfloat16, device=y.device)
    else:
        _dev(out, "out", torch.bfloat16, (T, H))
    p = _problem(T, H, K, layout.num_experts, layout.num_groups, layout.expert_alignment)
    s = layout.struct(gen)
    rc = _lib.lib().ep_combine(
        ctypes.byref(p),
        ctypes.byref(s),
        _ptr(topk_idx),
        _ptr(topk_weights),
        _ptr(y),
        int(y.shape[0]),
        _ptr(bias0),
        _ptr(bias1),
        _ptr(out),
        int(order),
        _stream(y.device),
    )
    _lib.check("ep_combine", rc)
    return out


@dataclasses.dataclass(frozen=True)
class PackedExpertWeights:
    """Expert weights bf16 [E, N, H] packed once into the grouped GEMM's tile
    order (``ep_pack_expert_weights``); pass it to ``ep_expert_gemm`` in
    place of the [E, N, H] tensor."""

    data: torch.Tensor  # bf16, ep_expert_weights_packed_bytes(E, N, H) / 2 elements
    num_experts: int
    n_out: int
    hidden: int


def ep_expert_weights_packed_bytes(num_experts: int, n_out: int, hidden: int) -> int:
    return int(_lib.lib().ep_expert_weights_packed_bytes(int(num_experts), int(n_out), int(hidden)))


def ep_pack_expert_weights(w: torch.Tensor) -> PackedExpertWeights:
    """Pack bf16 [E, N, H] expert weights for ``ep_expert_gemm``: every
    (expert, 256-column tile, 32-wide reduction step) block becomes 16 KiB
    contiguous, rows past N zero."""
    _dev(w, "w", torch.bfloat16)
    if w.dim() != 3:
        raise ValueError("w must be [E, N, H]")
    E, N, H = w.shape
    nbytes = ep_expert_weights_packed_bytes(E, N, H)
    if nbytes < 0:
        raise ValueError("packed weights need N % 128 == 0 and H % 64 == 0")
    data = torch.empty(nbytes // 2, dtype=torch.bfloat16, device=w.device)
    rc = _lib.lib().ep_pack_expert_weights(_ptr(w), int(E), int(N), int(H), _ptr(data), _stream(w.device))
    _lib.check("ep_pack_expert_weights", rc)
    return PackedExpertWeights(data, int(E), int(N), int(H))


def ep_expert_gemm(
    x: torch.Tensor,
    layout: Layout,
    w: torch.Tensor | PackedExpertWeights,
    out: torch.Tensor | None = None,
    gather: bool = False,
) -> torch.Tensor:
    """Grouped GEMM over the expert-major segments: y[r] = x_r @ w[e]^T for
    each receive row r of expert e; w: bf16 [E, N, H], or those weights
    packed by ``ep_pack_expert_weights``; returns y bf16 [rows, N] (rows
    outside the experts' selections are left as they were).

    x_r is row r of x (bf16 [rows, >= H], the dispatched receive rows), or,
    with ``gather``, row expert_row_src[r] of the token matrix x (bf16
    [T, >= H]): the dispatch folded into the GEMM's loads, which needs a
    layout computed with ``expert_row_src=True``."""
    layout, gen = _resolve(layout)
    packed = isinstance(w, PackedExpertWeights)
    if packed:
        E, N, H = w.num_experts, w.n_out, w.hidden
        _dev(w.data, "w.data", torch.bfloat16)
        if w.data.numel() * 2 != ep_expert_weights_packed_bytes(E, N, H):
            raise ValueError("packed weights of the wrong size")
        wt = w.data
    else:
        if w.dim() != 3:
            raise ValueError("w must be [E, N, H]")
        E, N, H = w.shape
        _dev(w, "w", torch.bfloat16)
        wt = w
    if x.dim() != 2:
        raise ValueError("x must be [rows, H]")
    _dev(x, "x", torch.bfloat16)
    if E != layout.num_experts:
        raise ValueError("w must hold one [N, H] matrix per expert")
    if x.shape[1] < H:
        raise ValueError("x rows are shorter than H")
    rows = layout.max_expert_rows()
    if gather:
        if x.shape[0] != layout.num_tokens:
            raise ValueError("with gather, x must be the [T, H] token matrix")
        if layout.expert_row_src is None or layout.expert_row_capacity < rows:
            raise ValueError("gather needs a layout computed with expert_row_src=True")
    elif x.shape[0] < rows:
        raise ValueError("x must hold the layout's worst-case expert rows")
    if out is None:
        out = torch.empty(rows if gather else x.shape[0], N, dtype=torch.bfloat16, device=x.device)
    else:
        _dev(out, "out", torch.bfloat16)
        if out.dim() != 2 or out.shape[1] < N or out.shape[0] < rows:
            raise ValueError("out must be bf16 [>= expert rows, >= N]")
    flags = (_lib.EP_FLAG_GATHER_ROWS if gather else 0) | (_lib.EP_FLAG_PACKED_WEIGHTS if packed else 0)
    p = _problem(layout.num_tokens, H, layout.topk, layout.num_experts, layout.num_groups,
                 layout.expert_alignment, flags)
    s = layout.struct(gen)
    rc = _lib.lib().ep_expert_gemm(
        ctypes.byref(p), ctypes.byref(s), _ptr(x), int(x.shape[1]), _ptr(wt), int(N), _ptr(out), int(out.shape[1]),
        _stream(x.device),
    )
    _lib.check("ep_expert_gemm", rc)
    return out
