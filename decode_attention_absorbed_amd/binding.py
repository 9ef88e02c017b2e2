"""Thin ctypes binding over libmla_decode.so (argument marshalling only).

Every step of the decode runs in the HIP library; this module checks torch
tensors against the plan, passes raw device pointers and the current stream,
and turns status codes into exceptions.  It never falls back to another
implementation: if the library is missing, importing the symbols fails.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence, Tuple

import numpy as np

# torch first: it loads the HIP runtime (libamdhip64.so.7) that the library
# then shares, so device pointers and streams mean the same thing on both sides.
import torch  # noqa: E402

from .build import LIB_PATH

MLA_OK = 0
MLA_ERR_INVALID_ARGUMENT = 1
MLA_ERR_UNSUPPORTED = 2
MLA_ERR_WORKSPACE_TOO_SMALL = 3
MLA_ERR_HIP = 4
MLA_ERR_OUT_OF_MEMORY = 5

MLA_Q_NUM_SEGMENTS = 0
MLA_Q_NUM_WORKGROUPS = 1
MLA_Q_NUM_PARTIALS = 2
MLA_Q_ROWS_PER_BLOCK = 3
MLA_Q_TILE_TOKENS = 4
MLA_Q_NUM_ROW_BLOCKS = 5
MLA_Q_NUM_COMBINE_WGS = 6

#: every symbol include/mla_decode.h declares
EXPORTED = (
    "mla_decode_plan",
    "mla_decode_plan_host",
    "mla_decode_workspace_bytes",
    "mla_decode",
    "mla_decode_partials",
    "mla_decode_combine",
    "mla_decode_plan_destroy",
    "mla_status_string",
    "mla_last_error",
    "mla_plan_query",
    "mla_plan_copy",
    "mla_plan_copy_combine",
    "mla_decode_fp8_plan",
    "mla_decode_fp8_plan_host",
    "mla_decode_fp8",
    "mla_decode_fp8_partials",
    "mla_prolog",
    "mla_up_project",
    "mla_o_project_workspace_bytes",
    "mla_o_project",
    "mla_decode_noalloc",
    "mla_decode_variant",
    "mla_decode_plan_update",
)

#: values of mla_decode_variant's `variant` (include/mla_decode.h)
MLA_RESCALE_LAZY = 0
MLA_RESCALE_POW2 = 1

#: kv_format values of mla_prolog
MLA_KV_BF16 = 0
MLA_KV_FP8 = 1


class MLAError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{message} (status {status})")
        self.status = status


_lib = None


def library_path() -> str:
    return os.environ.get("MLA_DECODE_LIB", LIB_PATH)


def lib() -> ctypes.CDLL:
    """Load the library once; raises loudly if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise ImportError(f"{path} not found: build it with `python -m decode_attention_absorbed_amd.build`")
    L = ctypes.CDLL(path)
    i32p = ctypes.POINTER(ctypes.c_int32)
    vp = ctypes.c_void_p
    L.mla_decode_plan.argtypes = [i32p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.POINTER(vp)]
    L.mla_decode_plan.restype = ctypes.c_int
    L.mla_decode_plan_host.argtypes = L.mla_decode_plan.argtypes
    L.mla_decode_plan_update.argtypes = [vp, i32p, vp]
    L.mla_decode_plan_update.restype = ctypes.c_int
    L.mla_decode_plan_host.restype = ctypes.c_int
    L.mla_decode_workspace_bytes.argtypes = [vp]
    L.mla_decode_workspace_bytes.restype = ctypes.c_size_t
    L.mla_decode.argtypes = [
        vp, vp, vp, vp, ctypes.c_int64, vp, ctypes.c_int32, vp, ctypes.c_float, vp, vp, vp, ctypes.c_size_t, vp,
    ]
    L.mla_decode.restype = ctypes.c_int
    L.mla_decode_noalloc.argtypes = L.mla_decode.argtypes[:11] + [vp]
    L.mla_decode_noalloc.restype = ctypes.c_int
    L.mla_decode_partials.argtypes = L.mla_decode.argtypes
    L.mla_decode_partials.restype = ctypes.c_int
    L.mla_decode_variant.argtypes = L.mla_decode.argtypes[:13] + [ctypes.c_int32, vp, vp]
    L.mla_decode_variant.restype = ctypes.c_int
    L.mla_decode_combine.argtypes = [vp, vp, vp, vp, ctypes.c_size_t, vp]
    L.mla_decode_combine.restype = ctypes.c_int
    L.mla_decode_plan_destroy.argtypes = [vp]
    L.mla_decode_plan_destroy.restype = None
    L.mla_status_string.argtypes = [ctypes.c_int]
    L.mla_status_string.restype = ctypes.c_char_p
    L.mla_last_error.argtypes = []
    L.mla_last_error.restype = ctypes.c_char_p
    L.mla_plan_query.argtypes = [vp, ctypes.c_int32]
    L.mla_plan_query.restype = ctypes.c_int64
    L.mla_plan_copy.argtypes = [vp, i32p, i32p]
    L.mla_plan_copy.restype = ctypes.c_int
    L.mla_plan_copy_combine.argtypes = [vp, i32p]
    L.mla_plan_copy_combine.restype = ctypes.c_int
    L.mla_decode_fp8_plan.argtypes = L.mla_decode_plan.argtypes
    L.mla_decode_fp8_plan.restype = ctypes.c_int
    L.mla_decode_fp8_plan_host.argtypes = L.mla_decode_plan.argtypes
    L.mla_decode_fp8_plan_host.restype = ctypes.c_int
    L.mla_decode_fp8.argtypes = [
        vp, vp, vp, vp, vp, ctypes.c_int64, vp, ctypes.c_int32, vp, ctypes.c_float, vp, vp, vp, ctypes.c_size_t, vp,
    ]
    L.mla_decode_fp8.restype = ctypes.c_int
    L.mla_decode_fp8_partials.argtypes = L.mla_decode_fp8.argtypes
    L.mla_decode_fp8_partials.restype = ctypes.c_int
    L.mla_prolog.argtypes = [
        ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, vp, vp, vp, vp, vp, ctypes.c_float, vp, vp, ctypes.c_int32,
        vp, vp, ctypes.c_int32, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, vp, vp, vp, vp, vp,
    ]
    L.mla_prolog.restype = ctypes.c_int
    L.mla_up_project.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, vp, vp, vp, vp]
    L.mla_up_project.restype = ctypes.c_int
    L.mla_o_project_workspace_bytes.argtypes = [ctypes.c_int32] * 4
    L.mla_o_project_workspace_bytes.restype = ctypes.c_size_t
    L.mla_o_project.argtypes = [ctypes.c_int32] * 4 + [vp, vp, vp, vp, ctypes.c_size_t, vp]
    L.mla_o_project.restype = ctypes.c_int
    _lib = L
    return L


def _check(status: int) -> None:
    if status != MLA_OK:
        L = lib()
        raise MLAError(status, f"{L.mla_status_string(status).decode()}: {L.mla_last_error().decode()}")


class Plan:
    """Owns an mla_plan*; destroyed with the object (or explicitly)."""

    def __init__(self, handle: int, seq_lens: np.ndarray, q_len: int, num_heads: int, page_size: int, on_device: bool):
        self.handle = handle
        self.seq_lens = seq_lens
        self.q_len = q_len
        self.num_heads = num_heads
        self.page_size = page_size
        self.on_device = on_device

    @property
    def batch(self) -> int:
        return int(self.seq_lens.shape[0])

    def query(self, key: int) -> int:
        return int(lib().mla_plan_query(self.handle, key))

    @property
    def workspace_bytes(self) -> int:
        return int(lib().mla_decode_workspace_bytes(self.handle))

    def segments(self) -> np.ndarray:
        """int32 [num_segments, 4]: request, first key, end key, partial id (-1 = whole)."""
        n = self.query(MLA_Q_NUM_SEGMENTS)
        seg = np.zeros((max(n, 1), 4), dtype=np.int32)
        _check(lib().mla_plan_copy(self.handle, seg.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), None))
        return seg[:n]

    def workgroups(self) -> np.ndarray:
        """int32 [grid, 4]: first segment, end segment, row block, 0."""
        n = self.query(MLA_Q_NUM_WORKGROUPS)
        wg = np.zeros((max(n, 1), 4), dtype=np.int32)
        _check(lib().mla_plan_copy(self.handle, None, wg.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))))
        return wg[:n]

    def combine_units(self) -> np.ndarray:
        """int32 [combine grid, 4]: request, first partial, pieces (0 = empty), first row."""
        n = self.query(MLA_Q_NUM_COMBINE_WGS)
        cu = np.zeros((max(n, 1), 4), dtype=np.int32)
        _check(lib().mla_plan_copy_combine(self.handle, cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))))
        return cu[:n]

    def update(self, seq_lens: Sequence[int], stream: Optional["torch.cuda.Stream"] = None) -> None:
        """mla_decode_plan_update: new lengths for the same batch shape, copied
        to the device schedule on `stream` (default: the current stream)."""
        lens = np.ascontiguousarray(np.asarray(seq_lens, dtype=np.int32))
        if lens.shape != (self.batch,):
            raise ValueError(f"seq_lens: shape {lens.shape}, expected ({self.batch},)")
        if stream is None and self.on_device:
            stream = torch.cuda.current_stream()
        st = stream.cuda_stream if stream is not None else None
        _check(lib().mla_decode_plan_update(self.handle, lens.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), st))
        self.seq_lens = lens

    def destroy(self) -> None:
        if self.handle:
            lib().mla_decode_plan_destroy(self.handle)
            self.handle = 0

    def __del__(self):
        try:
            self.destroy()
        except Exception:
            pass


def _make_plan(fn_name: str, seq_lens: Sequence[int], q_len: int, num_heads: int, page_size: int, num_cus: int) -> Plan:
    lens = np.ascontiguousarray(np.asarray(seq_lens, dtype=np.int32))
    h = ctypes.c_void_p()
    fn = getattr(lib(), fn_name)
    _check(fn(lens.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), int(lens.shape[0]), int(q_len), int(num_heads), int(page_size), int(num_cus), ctypes.byref(h)))
    return Plan(h.value, lens, q_len, num_heads, page_size, fn_name in ("mla_decode_plan", "mla_decode_fp8_plan"))


def mla_decode_plan(seq_lens: Sequence[int], q_len: int, num_heads: int, page_size: int, num_cus: int = 0) -> Plan:
    """Plan the split for one decode step (uploads the schedule to the current device)."""
    return _make_plan("mla_decode_plan", seq_lens, q_len, num_heads, page_size, num_cus)


def mla_decode_plan_host(seq_lens: Sequence[int], q_len: int, num_heads: int, page_size: int, num_cus: int) -> Plan:
    """Host-only plan (no HIP call): for inspection and argument checks."""
    return _make_plan("mla_decode_plan_host", seq_lens, q_len, num_heads, page_size, num_cus)


def mla_decode_fp8_plan(seq_lens: Sequence[int], q_len: int, num_heads: int, page_size: int, num_cus: int = 0) -> Plan:
    """Plan for the FP8-cache decode (64-key tiles; uploads the schedule)."""
    return _make_plan("mla_decode_fp8_plan", seq_lens, q_len, num_heads, page_size, num_cus)


def mla_decode_fp8_plan_host(seq_lens: Sequence[int], q_len: int, num_heads: int, page_size: int, num_cus: int) -> Plan:
    """Host-only FP8 plan (no HIP call)."""
    return _make_plan("mla_decode_fp8_plan_host", seq_lens, q_len, num_heads, page_size, num_cus)


def mla_decode_workspace_bytes(plan: Plan) -> int:
    return plan.workspace_bytes


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _expect(t: torch.Tensor, name: str, dtype: torch.dtype, shape: Tuple[int, ...]) -> None:
    if t.dtype != dtype:
        raise TypeError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on the GPU")


def _decode_args(plan, q_nope_absorbed, q_pe, kv_cache, block_table, seq_lens, softmax_scale, out, lse, workspace,
                 stream):
    """Checks the tensors, allocates out/lse/workspace where not given, and
    returns (mla_decode's argument list, out, lse)."""
    B, qlen, H = plan.batch, plan.q_len, plan.num_heads
    dev = q_nope_absorbed.device
    _expect(q_nope_absorbed, "q_nope_absorbed", torch.bfloat16, (B, qlen, H, 512))
    _expect(q_pe, "q_pe", torch.bfloat16, (B, qlen, H, 64))
    if kv_cache.dim() != 3 or kv_cache.shape[1] != plan.page_size or kv_cache.shape[2] != 576:
        raise ValueError(f"kv_cache: shape {tuple(kv_cache.shape)}, expected [num_pages, {plan.page_size}, 576]")
    _expect(kv_cache, "kv_cache", torch.bfloat16, tuple(kv_cache.shape))
    if block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError(f"block_table: shape {tuple(block_table.shape)}, expected [{B}, *]")
    _expect(block_table, "block_table", torch.int32, tuple(block_table.shape))
    _expect(seq_lens, "seq_lens", torch.int32, (B,))
    if out is None:
        out = torch.empty((B, qlen, H, 512), dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty((B, qlen, H), dtype=torch.float32, device=dev)
    _expect(out, "out", torch.float32, (B, qlen, H, 512))
    _expect(lse, "lse", torch.float32, (B, qlen, H))
    need = plan.workspace_bytes
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    args = [
        plan.handle,
        _ptr(q_nope_absorbed),
        _ptr(q_pe),
        _ptr(kv_cache),
        int(kv_cache.shape[0]),
        _ptr(block_table),
        int(block_table.shape[1]),
        _ptr(seq_lens),
        float(softmax_scale),
        _ptr(out),
        _ptr(lse),
        _ptr(workspace),
        int(ws_bytes),
    ]
    return args, stream.cuda_stream, out, lse


def mla_decode(
    plan: Plan,
    q_nope_absorbed: torch.Tensor,
    q_pe: torch.Tensor,
    kv_cache: torch.Tensor,
    block_table: torch.Tensor,
    seq_lens: torch.Tensor,
    softmax_scale: float,
    out: Optional[torch.Tensor] = None,
    lse: Optional[torch.Tensor] = None,
    workspace: Optional[torch.Tensor] = None,
    stream: Optional[torch.cuda.Stream] = None,
) -> Tuple[torch.Tensor, torch.Tensor]:
    """Enqueue the decode on `stream` (default: the current stream); returns (out, lse)."""
    args, st, out, lse = _decode_args(plan, q_nope_absorbed, q_pe, kv_cache, block_table, seq_lens, softmax_scale,
                                      out, lse, workspace, stream)
    _check(lib().mla_decode(*args, st))
    return out, lse


def mla_decode_variant(
    plan: Plan,
    q_nope_absorbed: torch.Tensor,
    q_pe: torch.Tensor,
    kv_cache: torch.Tensor,
    block_table: torch.Tensor,
    seq_lens: torch.Tensor,
    softmax_scale: float,
    variant: int = MLA_RESCALE_LAZY,
    rescale_events: Optional[torch.Tensor] = None,
    out: Optional[torch.Tensor] = None,
    lse: Optional[torch.Tensor] = None,
    workspace: Optional[torch.Tensor] = None,
    stream: Optional[torch.cuda.Stream] = None,
) -> Tuple[torch.Tensor, torch.Tensor]:
    """mla_decode with the O-rescale form `variant` (MLA_RESCALE_LAZY or
    MLA_RESCALE_POW2); `rescale_events` (a 1-element int32 device tensor the
    caller zeroes, or None) is incremented once per (wave, tile) rescale of O."""
    if rescale_events is not None:
        _expect(rescale_events, "rescale_events", torch.int32, (1,))
    args, st, out, lse = _decode_args(plan, q_nope_absorbed, q_pe, kv_cache, block_table, seq_lens, softmax_scale,
                                      out, lse, workspace, stream)
    _check(lib().mla_decode_variant(*args, int(variant), _ptr(rescale_events), st))
    return out, lse


def mla_decode_noalloc(
    plan: Plan,
    q_nope_absorbed: torch.Tensor,
    q_pe: torch.Tensor,
    kv_cache: torch.Tensor,
    block_table: torch.Tensor,
    seq_lens: torch.Tensor,
    softmax_scale: float,
    out: torch.Tensor,
    lse: torch.Tensor,
    stream: Optional[torch.cuda.Stream] = None,
) -> Tuple[torch.Tensor, torch.Tensor]:
    """mla_decode without a workspace: the library's per-GPU scratch holds the
    partials (no allocation in the call; out and lse come from the caller)."""
    B, qlen, H = plan.batch, plan.q_len, plan.num_heads
    _expect(q_nope_absorbed, "q_nope_absorbed", torch.bfloat16, (B, qlen, H, 512))
    _expect(q_pe, "q_pe", torch.bfloat16, (B, qlen, H, 64))
    _expect(kv_cache, "kv_cache", torch.bfloat16, tuple(kv_cache.shape))
    _expect(block_table, "block_table", torch.int32, tuple(block_table.shape))
    _expect(seq_lens, "seq_lens", torch.int32, (B,))
    _expect(out, "out", torch.float32, (B, qlen, H, 512))
    _expect(lse, "lse", torch.float32, (B, qlen, H))
    if stream is None:
        stream = torch.cuda.current_stream(q_nope_absorbed.device)
    _check(
        lib().mla_decode_noalloc(
            plan.handle, _ptr(q_nope_absorbed), _ptr(q_pe), _ptr(kv_cache), int(kv_cache.shape[0]), _ptr(block_table),
            int(block_table.shape[1]), _ptr(seq_lens), float(softmax_scale), _ptr(out), _ptr(lse), stream.cuda_stream,
        )
    )
    return out, lse


def mla_decode_fp8(
    plan: Plan,
    q_nope_absorbed: torch.Tensor,
    q_pe: torch.Tensor,
    kv_codes: torch.Tensor,
    kv_scales: torch.Tensor,
    block_table: torch.Tensor,
    seq_lens: torch.Tensor,
    softmax_scale: float,
    out: Optional[torch.Tensor] = None,
    lse: Optional[torch.Tensor] = None,
    workspace: Optional[torch.Tensor] = None,
    stream: Optional[torch.cuda.Stream] = None,
    partials_only: bool = False,
) -> Tuple[torch.Tensor, torch.Tensor]:
    """Enqueue the FP8-cache decode (E4M3 codes [num_pages, page, 576] uint8 and
    E8M0 token scales [num_pages, page] uint8); returns (out, lse).  With
    ``partials_only`` only the decode kernel runs (mla_decode_fp8_partials)."""
    B, qlen, H = plan.batch, plan.q_len, plan.num_heads
    dev = q_nope_absorbed.device
    _expect(q_nope_absorbed, "q_nope_absorbed", torch.bfloat16, (B, qlen, H, 512))
    _expect(q_pe, "q_pe", torch.bfloat16, (B, qlen, H, 64))
    if kv_codes.dim() != 3 or kv_codes.shape[1] != plan.page_size or kv_codes.shape[2] != 576:
        raise ValueError(f"kv_codes: shape {tuple(kv_codes.shape)}, expected [num_pages, {plan.page_size}, 576]")
    _expect(kv_codes, "kv_codes", torch.uint8, tuple(kv_codes.shape))
    _expect(kv_scales, "kv_scales", torch.uint8, tuple(kv_codes.shape[:2]))
    if block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError(f"block_table: shape {tuple(block_table.shape)}, expected [{B}, *]")
    _expect(block_table, "block_table", torch.int32, tuple(block_table.shape))
    _expect(seq_lens, "seq_lens", torch.int32, (B,))
    if out is None:
        out = torch.empty((B, qlen, H, 512), dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty((B, qlen, H), dtype=torch.float32, device=dev)
    _expect(out, "out", torch.float32, (B, qlen, H, 512))
    _expect(lse, "lse", torch.float32, (B, qlen, H))
    need = plan.workspace_bytes
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    fn = lib().mla_decode_fp8_partials if partials_only else lib().mla_decode_fp8
    _check(
        fn(
            plan.handle,
            _ptr(q_nope_absorbed),
            _ptr(q_pe),
            _ptr(kv_codes),
            _ptr(kv_scales),
            int(kv_codes.shape[0]),
            _ptr(block_table),
            int(block_table.shape[1]),
            _ptr(seq_lens),
            float(softmax_scale),
            _ptr(out),
            _ptr(lse),
            _ptr(workspace),
            int(ws_bytes),
            stream.cuda_stream,
        )
    )
    return out, lse


def mla_prolog(
    q_nope128: torch.Tensor,
    q_pe_raw: torch.Tensor,
    w_uk_t: torch.Tensor,
    c_kv_raw: torch.Tensor,
    kv_norm_w: torch.Tensor,
    rms_eps: float,
    k_pe_raw: torch.Tensor,
    rope_cos_sin: torch.Tensor,
    seq_lens: torch.Tensor,
    block_table: torch.Tensor,
    kv_cache: torch.Tensor,
    kv_scales: Optional[torch.Tensor] = None,
    q_nope_absorbed: Optional[torch.Tensor] = None,
    q_pe: Optional[torch.Tensor] = None,
    stream: Optional[torch.cuda.Stream] = None,
) -> Tuple[torch.Tensor, torch.Tensor]:
    """Enqueue the prolog: absorbed query, RoPE'd q_pe, and the new tokens'
    rows written into ``kv_cache`` (bf16 [num_pages, page, 576], or uint8 E4M3
    codes with ``kv_scales`` uint8 [num_pages, page]); returns
    (q_nope_absorbed, q_pe)."""
    if q_nope128.dim() != 4 or q_nope128.shape[3] != 128:
        raise ValueError(f"q_nope128: shape {tuple(q_nope128.shape)}, expected [B, q_len, H, 128]")
    B, qlen, H = (int(v) for v in q_nope128.shape[:3])
    dev = q_nope128.device
    _expect(q_nope128, "q_nope128", torch.bfloat16, (B, qlen, H, 128))
    _expect(q_pe_raw, "q_pe_raw", torch.bfloat16, (B, qlen, H, 64))
    _expect(w_uk_t, "w_uk_t", torch.bfloat16, (H, 512, 128))
    _expect(c_kv_raw, "c_kv_raw", torch.bfloat16, (B, qlen, 512))
    _expect(kv_norm_w, "kv_norm_w", torch.bfloat16, (512,))
    _expect(k_pe_raw, "k_pe_raw", torch.bfloat16, (B, qlen, 64))
    if rope_cos_sin.dim() != 2 or rope_cos_sin.shape[1] != 64:
        raise ValueError(f"rope_cos_sin: shape {tuple(rope_cos_sin.shape)}, expected [max_pos, 64]")
    _expect(rope_cos_sin, "rope_cos_sin", torch.float32, tuple(rope_cos_sin.shape))
    _expect(seq_lens, "seq_lens", torch.int32, (B,))
    if block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError(f"block_table: shape {tuple(block_table.shape)}, expected [{B}, *]")
    _expect(block_table, "block_table", torch.int32, tuple(block_table.shape))
    if kv_cache.dim() != 3 or kv_cache.shape[2] != 576:
        raise ValueError(f"kv_cache: shape {tuple(kv_cache.shape)}, expected [num_pages, page, 576]")
    fp8 = kv_cache.dtype == torch.uint8
    _expect(kv_cache, "kv_cache", torch.uint8 if fp8 else torch.bfloat16, tuple(kv_cache.shape))
    if fp8:
        if kv_scales is None:
            raise ValueError("an FP8 cache needs kv_scales")
        _expect(kv_scales, "kv_scales", torch.uint8, tuple(kv_cache.shape[:2]))
    if q_nope_absorbed is None:
        q_nope_absorbed = torch.empty((B, qlen, H, 512), dtype=torch.bfloat16, device=dev)
    if q_pe is None:
        q_pe = torch.empty((B, qlen, H, 64), dtype=torch.bfloat16, device=dev)
    _expect(q_nope_absorbed, "q_nope_absorbed", torch.bfloat16, (B, qlen, H, 512))
    _expect(q_pe, "q_pe", torch.bfloat16, (B, qlen, H, 64))
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    _check(
        lib().mla_prolog(
            B, qlen, H,
            _ptr(q_nope128), _ptr(q_pe_raw), _ptr(w_uk_t), _ptr(c_kv_raw), _ptr(kv_norm_w), float(rms_eps),
            _ptr(k_pe_raw), _ptr(rope_cos_sin), int(rope_cos_sin.shape[0]),
            _ptr(seq_lens), _ptr(block_table), int(block_table.shape[1]),
            int(kv_cache.shape[0]), int(kv_cache.shape[1]), MLA_KV_FP8 if fp8 else MLA_KV_BF16,
            _ptr(kv_cache), _ptr(kv_scales if fp8 else None),
            _ptr(q_nope_absorbed), _ptr(q_pe), stream.cuda_stream,
        )
    )
    return q_nope_absorbed, q_pe


def mla_up_project(
    attn_out: torch.Tensor,
    w_uv: torch.Tensor,
    o: Optional[torch.Tensor] = None,
    stream: Optional[torch.cuda.Stream] = None,
) -> torch.Tensor:
    """Enqueue o[b, j, h] = W_UV[h] attn_out[b, j, h] (attn_out fp32 [B, q_len, H, 512],
    w_uv bf16 [H, 128, 512]); returns o (bf16 [B, q_len, H, 128])."""
    if attn_out.dim() != 4 or attn_out.shape[3] != 512:
        raise ValueError(f"attn_out: shape {tuple(attn_out.shape)}, expected [B, q_len, H, 512]")
    B, qlen, H = (int(v) for v in attn_out.shape[:3])
    _expect(attn_out, "attn_out", torch.float32, (B, qlen, H, 512))
    _expect(w_uv, "w_uv", torch.bfloat16, (H, 128, 512))
    if o is None:
        o = torch.empty((B, qlen, H, 128), dtype=torch.bfloat16, device=attn_out.device)
    _expect(o, "o", torch.bfloat16, (B, qlen, H, 128))
    if stream is None:
        stream = torch.cuda.current_stream(attn_out.device)
    _check(lib().mla_up_project(B, qlen, H, _ptr(attn_out), _ptr(w_uv), _ptr(o), stream.cuda_stream))
    return o


def mla_o_project_workspace_bytes(batch: int, q_len: int, k_in: int, n_out: int) -> int:
    return int(lib().mla_o_project_workspace_bytes(batch, q_len, k_in, n_out))


def mla_o_project(
    o: torch.Tensor,
    w_o: torch.Tensor,
    y: Optional[torch.Tensor] = None,
    workspace: Optional[torch.Tensor] = None,
    stream: Optional[torch.cuda.Stream] = None,
) -> torch.Tensor:
    """Enqueue y = W_O concat_h(o) for o bf16 [B, q_len, H, 128] (mla_up_project's
    output) and w_o bf16 [n_out, H * 128]; returns y (bf16 [B, q_len, n_out])."""
    if o.dim() != 4 or o.shape[3] != 128:
        raise ValueError(f"o: shape {tuple(o.shape)}, expected [B, q_len, H, 128]")
    B, qlen, H = (int(v) for v in o.shape[:3])
    K = H * 128
    _expect(o, "o", torch.bfloat16, (B, qlen, H, 128))
    if w_o.dim() != 2 or w_o.shape[1] != K:
        raise ValueError(f"w_o: shape {tuple(w_o.shape)}, expected [n_out, {K}]")
    _expect(w_o, "w_o", torch.bfloat16, tuple(w_o.shape))
    N = int(w_o.shape[0])
    if y is None:
        y = torch.empty((B, qlen, N), dtype=torch.bfloat16, device=o.device)
    _expect(y, "y", torch.bfloat16, (B, qlen, N))
    need = mla_o_project_workspace_bytes(B, qlen, K, N)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=o.device)
    if stream is None:
        stream = torch.cuda.current_stream(o.device)
    _check(
        lib().mla_o_project(
            B, qlen, K, N, _ptr(o), _ptr(w_o), _ptr(y), _ptr(workspace),
            workspace.numel() * workspace.element_size(), stream.cuda_stream,
        )
    )
    return y

