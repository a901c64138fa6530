"""Python binding of libflexmi (MI355X block-sparse attention, forward and backward).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI in ``include/flexmi.h``.  torch supplies device
memory and the current stream.  The binding exposes the C entry points under
the same names:

  flex_blockmask_build(mask, L, S, q_block, kv_block, ...) -> BlockMask
  flex_attn_fwd(q, k, v, score=..., mask=..., block_mask=..., ...) -> (out, lse)
  flex_attn_fwd_aux(q, k, v, ...) -> (out, lse, max_scores)
  flex_attn_fwd_paged(q, k_pool, v_pool, page_table, S=..., ...) -> (out, lse, max_scores)
  flex_attn_fwd_workspace_bytes(...)
  flex_blockmask_transpose(block_mask) -> BlockMaskQ
  flex_attn_fwd_noalloc(q, k, v, ...) -> (out, lse)
  flex_attn_bwd(q, k, v, out, dout, lse, ...) -> (dq, dk, dv)
  flex_attn_bwd_paged(q, k_pool, v_pool, page_table, out, dout, lse, S=..., ...) -> (dq, dk, dv)
  flex_attn_bwd_workspace_bytes(...)
  BlockMask.to_dense / grid / to_string / sparsity / [b, h, rows] / adjust
      (flex_blockmask_to_dense, _grid, _sparsity, _slice, _adjust)
  flex_status_string(code)

There is no fallback: if the native library is missing or cannot load, every
call raises.
"""
from __future__ import annotations

import ctypes
import dataclasses
import math
import os
from typing import Optional

import torch  # imported first so the library binds to torch's HIP runtime

__all__ = [
    "MaskSpec", "ScoreSpec", "BlockMask", "FlexError", "load_library", "library_path",
    "flex_blockmask_build", "flex_attn_fwd", "flex_attn_fwd_aux", "flex_attn_fwd_workspace_bytes",
    "BlockMaskQ", "flex_blockmask_transpose", "flex_attn_bwd", "flex_attn_bwd_workspace_bytes",
    "flex_attn_fwd_paged", "flex_attn_fwd_noalloc", "flex_attn_bwd_paged",
    "flex_status_string", "flex_last_error", "MASK_KINDS", "SCORE_KINDS", "PREDICATES", "EXPORTED_SYMBOLS",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
MASK_KINDS = {"noop": 0, "causal": 1, "causal_window_sinks": 2, "doc_causal": 3, "program": 4}
SCORE_KINDS = {"none": 0, "softcap": 1, "softcap_alibi": 2, "alibi": 3}
PREDICATES = {"causal": 0, "window": 1, "kv_lt": 2, "chunk": 3, "stride": 4, "doc": 5, "head_lt": 6}
MAX_CLAUSES, MAX_LITERALS = 4, 2
DTYPES = {torch.float32: 0, torch.bfloat16: 1}
EXPORTED_SYMBOLS = ("flex_blockmask_build", "flex_attn_fwd_workspace_bytes", "flex_attn_fwd", "flex_attn_fwd_aux",
                    "flex_blockmask_transpose", "flex_attn_bwd_workspace_bytes", "flex_attn_bwd",
                    "flex_attn_fwd_paged", "flex_attn_fwd_noalloc", "flex_attn_bwd_paged",
                    "flex_blockmask_to_dense", "flex_blockmask_grid", "flex_blockmask_sparsity",
                    "flex_blockmask_slice", "flex_blockmask_adjust",
                    "flex_status_string", "flex_last_error")


class flex_mask_pred(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("arg", ctypes.c_int32)]


class flex_mask_clause(ctypes.Structure):
    _fields_ = [("n", ctypes.c_int32), ("lit", flex_mask_pred * MAX_LITERALS)]


class flex_mask_params(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("window", ctypes.c_int32), ("sinks", ctypes.c_int32),
                ("reserved", ctypes.c_int32), ("q_offset", ctypes.c_int64), ("doc_id", ctypes.c_void_p),
                ("doc_len", ctypes.c_int64), ("n_clauses", ctypes.c_int32),
                ("clause", flex_mask_clause * MAX_CLAUSES), ("q_offsets", ctypes.c_void_p),
                ("kv_lens", ctypes.c_void_p)]


class flex_score_params(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("cap", ctypes.c_float), ("alibi_m", ctypes.c_float)]


class flex_block_mask(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("H", ctypes.c_int32), ("q_block", ctypes.c_int32),
                ("kv_block", ctypes.c_int32), ("num_q_blocks", ctypes.c_int32), ("num_kv_blocks", ctypes.c_int32),
                ("kv_num_blocks", ctypes.c_void_p), ("kv_indices", ctypes.c_void_p),
                ("full_kv_num_blocks", ctypes.c_void_p), ("full_kv_indices", ctypes.c_void_p)]


class flex_kv_pages(ctypes.Structure):
    _fields_ = [("page_table", ctypes.c_void_p), ("page_size", ctypes.c_int32), ("max_pages", ctypes.c_int32),
                ("num_pages", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class flex_block_mask_q(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("H", ctypes.c_int32), ("q_block", ctypes.c_int32),
                ("kv_block", ctypes.c_int32), ("num_q_blocks", ctypes.c_int32), ("num_kv_blocks", ctypes.c_int32),
                ("q_num_blocks", ctypes.c_void_p), ("q_indices", ctypes.c_void_p),
                ("full_q_num_blocks", ctypes.c_void_p), ("full_q_indices", ctypes.c_void_p)]


_LIB = None


def library_path() -> str:
    return os.environ.get("FLEXMI_LIBRARY", os.path.join(_HERE, "libflexmi.so"))


def load_library():
    """Load libflexmi.so (built by ``programmable_block_sparse_amd.build``); raises if absent."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(f"native library {path} is missing: run programmable_block_sparse_amd.build first")
    lib = ctypes.CDLL(path)
    P, I32, I64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    I64x3 = ctypes.POINTER(ctypes.c_int64)
    lib.flex_blockmask_build.argtypes = [ctypes.POINTER(flex_mask_params), I64, I64,
                                         ctypes.POINTER(flex_block_mask), P]
    lib.flex_blockmask_build.restype = ctypes.c_int
    lib.flex_attn_fwd_workspace_bytes.argtypes = [I32, I32, I32, I32, I64, I64, I32, ctypes.POINTER(flex_block_mask)]
    lib.flex_attn_fwd_workspace_bytes.restype = ctypes.c_size_t
    lib.flex_attn_fwd.argtypes = [P, P, P, I32, I32, I32, I32, I64, I64, I32, I64x3, I64x3, I64x3, ctypes.c_float,
                                  ctypes.POINTER(flex_score_params), ctypes.POINTER(flex_mask_params),
                                  ctypes.POINTER(flex_block_mask), P, P, P, ctypes.c_size_t, P]
    lib.flex_attn_fwd.restype = ctypes.c_int
    lib.flex_attn_fwd_aux.argtypes = [P, P, P, I32, I32, I32, I32, I64, I64, I32, I64x3, I64x3, I64x3,
                                      ctypes.c_float, ctypes.POINTER(flex_score_params),
                                      ctypes.POINTER(flex_mask_params), ctypes.POINTER(flex_block_mask), P, P, P,
                                      P, ctypes.c_size_t, P]
    lib.flex_attn_fwd_aux.restype = ctypes.c_int
    lib.flex_attn_fwd_paged.argtypes = [P, P, P, I32, I32, I32, I32, I64, I64, I32, I64x3, I64x3, I64x3,
                                        ctypes.c_float, ctypes.POINTER(flex_score_params),
                                        ctypes.POINTER(flex_mask_params), ctypes.POINTER(flex_block_mask),
                                        ctypes.POINTER(flex_kv_pages), P, P, P, P, ctypes.c_size_t, P]
    lib.flex_attn_fwd_paged.restype = ctypes.c_int
    lib.flex_attn_fwd_noalloc.argtypes = [P, P, P, I32, I32, I32, I32, I64, I64, I32, I64x3, I64x3, I64x3,
                                          ctypes.c_float, ctypes.POINTER(flex_score_params),
                                          ctypes.POINTER(flex_mask_params), ctypes.POINTER(flex_block_mask), P, P, P]
    lib.flex_attn_fwd_noalloc.restype = ctypes.c_int
    lib.flex_blockmask_transpose.argtypes = [ctypes.POINTER(flex_block_mask), ctypes.POINTER(flex_block_mask_q), P]
    lib.flex_blockmask_transpose.restype = ctypes.c_int
    lib.flex_attn_bwd_workspace_bytes.argtypes = [I32, I32, I32, I32, I64, I64, I32, ctypes.POINTER(flex_block_mask)]
    lib.flex_attn_bwd_workspace_bytes.restype = ctypes.c_size_t
    lib.flex_attn_bwd.argtypes = [P, P, P, P, P, P, I32, I32, I32, I32, I64, I64, I32, I64x3, I64x3, I64x3,
                                  ctypes.c_float, ctypes.POINTER(flex_score_params), ctypes.POINTER(flex_mask_params),
                                  ctypes.POINTER(flex_block_mask), ctypes.POINTER(flex_block_mask_q), P, P, P, P,
                                  ctypes.c_size_t, P]
    lib.flex_attn_bwd.restype = ctypes.c_int
    lib.flex_attn_bwd_paged.argtypes = [P, P, P, ctypes.POINTER(flex_kv_pages), P, P, P, I32, I32, I32, I32, I64, I64,
                                        I32, I64x3, I64x3, I64x3, ctypes.c_float, ctypes.POINTER(flex_score_params),
                                        ctypes.POINTER(flex_mask_params), ctypes.POINTER(flex_block_mask),
                                        ctypes.POINTER(flex_block_mask_q), P, P, P, P, ctypes.c_size_t, P]
    lib.flex_attn_bwd_paged.restype = ctypes.c_int
    BMP = ctypes.POINTER(flex_block_mask)
    lib.flex_blockmask_to_dense.argtypes = [BMP, P, P]
    lib.flex_blockmask_grid.argtypes = [BMP, I32, I32, P, P]
    lib.flex_blockmask_sparsity.argtypes = [BMP, P, P]
    lib.flex_blockmask_slice.argtypes = [BMP, ctypes.POINTER(ctypes.c_int32), BMP, P]
    lib.flex_blockmask_adjust.argtypes = [BMP, I64, I64, BMP, P]
    for name in ("flex_blockmask_to_dense", "flex_blockmask_grid", "flex_blockmask_sparsity", "flex_blockmask_slice",
                 "flex_blockmask_adjust"):
        getattr(lib, name).restype = ctypes.c_int
    lib.flex_status_string.argtypes = [I32]
    lib.flex_status_string.restype = ctypes.c_char_p
    lib.flex_last_error.argtypes = []
    lib.flex_last_error.restype = ctypes.c_char_p
    _LIB = lib
    return lib


class FlexError(RuntimeError):
    def __init__(self, status: int, detail: str):
        self.status = status
        super().__init__(f"{flex_status_string(status)}: {detail}")


def flex_status_string(status: int) -> str:
    return load_library().flex_status_string(int(status)).decode()


def flex_last_error() -> str:
    return load_library().flex_last_error().decode()


def _check(status: int):
    if status != 0:
        raise FlexError(status, flex_last_error())


@dataclasses.dataclass
class MaskSpec:
    """mask_mod menu entry.  ``q_offset=None`` means bottom-right alignment (S - L).

    kind "program": ``clauses`` is a sequence of clauses, each a sequence of
    (predicate, argument) pairs from PREDICATES; the mask is the AND of the
    clauses, a clause the OR of its predicates (and_masks / or_masks)."""
    kind: str = "noop"
    window: int = 0
    sinks: int = 0
    q_offset: Optional[int] = None
    doc_id: Optional[torch.Tensor] = None   # int32 device tensor for "doc_causal" / the "doc" predicate
    clauses: tuple = ()
    q_offsets: Optional[torch.Tensor] = None  # int32 device (B,): per-batch logical position of query row 0
    kv_lens: Optional[torch.Tensor] = None    # int32 device (B,): per-batch filled length of the cache

    def to_c(self, L: int, S: int) -> flex_mask_params:
        ptr = lambda t: None if t is None else t.data_ptr()
        key = (L, S, self.kind, self.window, self.sinks, self.q_offset,
               None if self.doc_id is None else (self.doc_id.data_ptr(), self.doc_id.numel()),
               tuple(tuple((str(n), int(a)) for n, a in c) for c in self.clauses),
               ptr(self.q_offsets), ptr(self.kv_lens))
        cached = self.__dict__.get("_c")
        if cached is not None and cached[0] == key:
            return cached[1]
        m = flex_mask_params()
        m.kind = MASK_KINDS[self.kind]
        m.window = int(self.window)
        m.sinks = int(self.sinks)
        m.q_offset = int(S - L if self.q_offset is None else self.q_offset)
        if self.doc_id is not None:
            if self.doc_id.dtype != torch.int32 or not self.doc_id.is_contiguous():
                raise ValueError("doc_id must be a contiguous int32 tensor")
            m.doc_id = self.doc_id.data_ptr()
            m.doc_len = self.doc_id.numel()
        for t in (self.q_offsets, self.kv_lens):
            if t is not None and (t.dtype != torch.int32 or not t.is_contiguous()):
                raise ValueError("q_offsets and kv_lens must be contiguous int32 tensors")
        m.q_offsets = ptr(self.q_offsets)
        m.kv_lens = ptr(self.kv_lens)
        clauses = key[-3]
        if len(clauses) > MAX_CLAUSES or any(len(c) > MAX_LITERALS for c in clauses):
            raise ValueError(f"at most {MAX_CLAUSES} clauses of at most {MAX_LITERALS} predicates")
        m.n_clauses = len(clauses)
        for i, c in enumerate(clauses):
            m.clause[i].n = len(c)
            for j, (name, arg) in enumerate(c):
                m.clause[i].lit[j].kind = PREDICATES[name]
                m.clause[i].lit[j].arg = arg
        self.__dict__["_c"] = (key, m)
        return m


@dataclasses.dataclass
class ScoreSpec:
    """score_mod menu entry."""
    kind: str = "none"
    cap: float = 0.0
    alibi_m: float = 8.0

    def to_c(self) -> flex_score_params:
        key = (self.kind, self.cap, self.alibi_m)
        cached = self.__dict__.get("_c")
        if cached is not None and cached[0] == key:
            return cached[1]
        s = flex_score_params()
        s.kind = SCORE_KINDS[self.kind]
        s.cap = float(self.cap)
        s.alibi_m = float(self.alibi_m)
        self.__dict__["_c"] = (key, s)
        return s


@dataclasses.dataclass
class BlockMask:
    """The four BlockMask arrays (int32 device tensors) and their dims."""
    kv_num_blocks: torch.Tensor
    kv_indices: torch.Tensor
    full_kv_num_blocks: torch.Tensor
    full_kv_indices: torch.Tensor
    q_block: int
    kv_block: int
    L: int
    S: int

    @property
    def B(self) -> int:
        return self.kv_num_blocks.shape[0]

    @property
    def H(self) -> int:
        return self.kv_num_blocks.shape[1]

    # -- utilities of the 2kiu guide, section 3.3 (each runs in a library kernel)
    @property
    def shape(self):
        """batch dims + sequence lengths: (B, H, L, S)."""
        return (self.B, self.H, self.L, self.S)

    def numel(self) -> int:
        """Elements of the mask, sparse ones included."""
        return self.B * self.H * self.L * self.S

    def _empty_like(self, B, H, nqb, nkb, L, S) -> "BlockMask":
        dev = self.kv_indices.device
        t = lambda *shape: torch.empty(shape, dtype=torch.int32, device=dev)
        return BlockMask(t(B, H, nqb), t(B, H, nqb, nkb), t(B, H, nqb), t(B, H, nqb, nkb), self.q_block,
                         self.kv_block, L, S)

    def to_dense(self) -> torch.Tensor:
        """int32 (B, H, nQB, nKB): 1 where a tile is computed (C: flex_blockmask_to_dense)."""
        dense = torch.empty(self.kv_indices.shape, dtype=torch.int32, device=self.kv_indices.device)
        _check(load_library().flex_blockmask_to_dense(ctypes.byref(self.to_c()), dense.data_ptr(), self._stream()))
        return dense

    def grid(self, grid_rows: int, grid_cols: int) -> torch.Tensor:
        """int8 tile classes pooled into windows: 2 all full, 0 all empty, 1 mixed (C: flex_blockmask_grid)."""
        B, H, nqb, nkb = self.kv_indices.shape
        wr, wc = -(-nqb // grid_rows), -(-nkb // grid_cols)
        out = torch.empty((B, H, -(-nqb // wr), -(-nkb // wc)), dtype=torch.int8, device=self.kv_indices.device)
        _check(load_library().flex_blockmask_grid(ctypes.byref(self.to_c()), grid_rows, grid_cols, out.data_ptr(),
                                                  self._stream()))
        return out

    def to_string(self, grid_size=(20, 20), limit: int = 4) -> str:
        """ASCII picture: '█' full, '░' partial, ' ' empty; grid_size=-1 draws every tile."""
        B, H, nqb, nkb = self.kv_indices.shape
        gr, gc = (nqb, nkb) if grid_size == -1 else grid_size
        g = self.grid(gr, gc).cpu().numpy()
        glyph = {0: " ", 1: "░", 2: "█"}
        lines, shown = [], 0
        for b in range(B):
            for h in range(H):
                if shown == limit:
                    break
                lines.append(f"b={b} h={h}")
                lines.extend("".join(glyph[int(c)] for c in row) for row in g[b, h])
                shown += 1
        return "\n".join(lines)

    def sparsity(self) -> float:
        """Percentage of tiles not computed (C: flex_blockmask_sparsity; waits for the result)."""
        out = torch.empty(1, dtype=torch.float64, device=self.kv_indices.device)
        _check(load_library().flex_blockmask_sparsity(ctypes.byref(self.to_c()), out.data_ptr(), self._stream()))
        return float(out.item())

    def __getitem__(self, index) -> "BlockMask":
        """Select batches, heads and Q-block rows (integers keep their dimension) (C: flex_blockmask_slice)."""
        if not isinstance(index, tuple):
            index = (index,)
        if len(index) > 3:
            raise IndexError("at most three indices: batch, head, Q-block row")
        B, H, nqb, nkb = self.kv_indices.shape
        ranges = []
        for i, n in zip(range(3), (B, H, nqb)):
            sel = index[i] if i < len(index) else slice(None)
            if isinstance(sel, int):
                sel = slice(sel % n, sel % n + 1) if -n <= sel < n else None
            if sel is None or not isinstance(sel, slice) or sel.step not in (None, 1):
                raise IndexError(f"index {index[i]!r} is not a unit-step range inside {n}")
            start, stop, _ = sel.indices(n)
            ranges.append((start, stop))
        (b0, b1), (h0, h1), (r0, r1) = ranges
        rows_L = max(0, min(self.L - r0 * self.q_block, (r1 - r0) * self.q_block))
        out = self._empty_like(b1 - b0, h1 - h0, r1 - r0, nkb, rows_L, self.S)
        arr = (ctypes.c_int32 * 6)(b0, b1, h0, h1, r0, r1)
        _check(load_library().flex_blockmask_slice(ctypes.byref(self.to_c()), arr, ctypes.byref(out.to_c()),
                                                   self._stream()))
        return out

    def adjust(self, new_L: int, new_S: int) -> "BlockMask":
        """Crop to the top-left new lengths (C: flex_blockmask_adjust)."""
        B, H = self.B, self.H
        out = self._empty_like(B, H, -(-new_L // self.q_block), -(-new_S // self.kv_block), new_L, new_S)
        _check(load_library().flex_blockmask_adjust(ctypes.byref(self.to_c()), new_L, new_S, ctypes.byref(out.to_c()),
                                                    self._stream()))
        return out

    _adjust = adjust

    def as_tuple(self):
        """The four arrays followed by (q_block, kv_block, L, S)."""
        return (self.kv_num_blocks, self.kv_indices, self.full_kv_num_blocks, self.full_kv_indices, self.q_block,
                self.kv_block, self.L, self.S)

    @classmethod
    def from_kv_blocks(cls, kv_num_blocks, kv_indices, full_kv_num_blocks, full_kv_indices, *, q_block: int,
                       kv_block: int, L: int, S: int) -> "BlockMask":
        """Wrap existing KV-side lists (int32 device tensors, (B, H, nQB[, nKB]))."""
        for t in (kv_num_blocks, kv_indices, full_kv_num_blocks, full_kv_indices):
            if t.dtype != torch.int32 or not t.is_contiguous():
                raise ValueError("block lists must be contiguous int32 tensors")
        return cls(kv_num_blocks, kv_indices, full_kv_num_blocks, full_kv_indices, q_block, kv_block, L, S)

    def to(self, device) -> "BlockMask":
        """A copy on another device (this mask is unchanged)."""
        return BlockMask(*(t.to(device) for t in self.as_tuple()[:4]), self.q_block, self.kv_block, self.L, self.S)

    def _stream(self):
        return ctypes.c_void_p(_stream_ptr(self.kv_indices.device))

    def _validate(self, device=None):
        """The four arrays: int32, contiguous, on ``device`` (default: the mask's
        own GPU), shapes (B, H, nQB) and (B, H, nQB, nKB) for this mask's L, S."""
        device = self.kv_indices.device if device is None else device
        if self.q_block < 1 or self.kv_block < 1:
            raise ValueError("block sizes must be positive")
        nqb, nkb = -(-self.L // self.q_block), -(-self.S // self.kv_block)
        B, H = self.kv_num_blocks.shape[:2] if self.kv_num_blocks.dim() == 3 else (-1, -1)
        for name, shape in (("kv_num_blocks", (B, H, nqb)), ("kv_indices", (B, H, nqb, nkb)),
                            ("full_kv_num_blocks", (B, H, nqb)), ("full_kv_indices", (B, H, nqb, nkb))):
            _require(getattr(self, name), f"block mask {name}", device, dtype=torch.int32, shape=shape)

    def to_c(self) -> flex_block_mask:
        self._validate()
        cached = self.__dict__.get("_c")
        if cached is not None:
            return cached
        c = flex_block_mask()
        c.B, c.H = self.B, self.H
        c.q_block, c.kv_block = self.q_block, self.kv_block
        c.num_q_blocks, c.num_kv_blocks = self.kv_indices.shape[2], self.kv_indices.shape[3]
        c.kv_num_blocks = self.kv_num_blocks.data_ptr()
        c.kv_indices = self.kv_indices.data_ptr()
        c.full_kv_num_blocks = self.full_kv_num_blocks.data_ptr()
        c.full_kv_indices = self.full_kv_indices.data_ptr()
        self.__dict__["_c"] = c
        return c


def _require(t, name: str, device, *, dtype=None, shape=None, contiguous: bool = True):
    """Raise ValueError unless ``t`` is a tensor on ``device`` (a GPU) with the
    given dtype, exact shape and contiguity.  Runs before any pointer is handed
    to the library, so a wrong buffer is an error, never a stray address."""
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch tensor")
    if t.device.type != "cuda" or (device is not None and t.device != device):
        raise ValueError(f"{name} must be on {device} (it is on {t.device})")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype} (it is {t.dtype})")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)} (it has {tuple(t.shape)})")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _require_workspace(ws, ws_bytes: int, device):
    if ws is None:
        return
    _require(ws, "workspace", device)
    if ws.numel() * ws.element_size() < ws_bytes:
        raise ValueError(f"workspace holds {ws.numel() * ws.element_size()} bytes, {ws_bytes} needed")


def _require_mask_tensors(mask: "MaskSpec", device, B: Optional[int]):
    if mask.doc_id is not None:
        _require(mask.doc_id, "doc_id", device, dtype=torch.int32)
        if mask.doc_id.dim() != 1:
            raise ValueError("doc_id must be 1-D")
    for name in ("q_offsets", "kv_lens"):
        t = getattr(mask, name)
        if t is not None:
            _require(t, name, device, dtype=torch.int32, shape=None if B is None else (B,))


def _require_qkv(q, k, v, names=("q", "k", "v")):
    """q, k, v (or q and the pools): GPU tensors on one device, last dim
    contiguous (other strides are passed to the library)."""
    for t, name in zip((q, k, v), names):
        if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
            raise ValueError(f"{name} must be a GPU tensor")
        if t.device != q.device:
            raise ValueError(f"{name} is on {t.device}, q on {q.device}")
        if t.stride(3) != 1:
            raise ValueError("the last dimension must be contiguous")


def _stream_ptr(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def flex_blockmask_build(mask: MaskSpec, L: int, S: int, q_block: int, kv_block: int, *, B: int = 1, H: int = 1,
                         device="cuda", out: Optional[BlockMask] = None) -> BlockMask:
    """Fill a BlockMask on the GPU (C: flex_blockmask_build).

    Allocates the four int32 tensors unless ``out`` (a BlockMask of the same dims)
    is given, in which case it is refilled in place.
    """
    lib = load_library()
    if out is None:
        nqb, nkb = -(-L // q_block), -(-S // kv_block)
        dev = torch.device(device)
        t = lambda *shape: torch.empty(shape, dtype=torch.int32, device=dev)
        out = BlockMask(t(B, H, nqb), t(B, H, nqb, nkb), t(B, H, nqb), t(B, H, nqb, nkb), q_block, kv_block, L, S)
    elif (out.L, out.S, out.q_block, out.kv_block, out.B, out.H) != (L, S, q_block, kv_block, B, H):
        raise ValueError("out BlockMask has different dims")
    out._validate()
    _require_mask_tensors(mask, out.kv_indices.device, None)
    cm = mask.to_c(L, S)
    cbm = out.to_c()
    _check(lib.flex_blockmask_build(ctypes.byref(cm), L, S, ctypes.byref(cbm),
                                    ctypes.c_void_p(_stream_ptr(out.kv_num_blocks.device))))
    return out


def flex_attn_fwd_workspace_bytes(dtype: torch.dtype, B: int, Hq: int, Hkv: int, L: int, S: int, D: int,
                                  block_mask: BlockMask) -> int:
    lib = load_library()
    cbm = block_mask.to_c()
    return int(lib.flex_attn_fwd_workspace_bytes(DTYPES[dtype], B, Hq, Hkv, L, S, D, ctypes.byref(cbm)))


def flex_attn_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, block_mask: BlockMask,
                  score: Optional[ScoreSpec] = None, mask: Optional[MaskSpec] = None,
                  scale: Optional[float] = None, return_lse: bool = True,
                  out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                  workspace: Optional[torch.Tensor] = None):
    """Block-sparse attention forward (C: flex_attn_fwd).

    q (B, Hq, L, D), k and v (B, Hkv, S, D) device tensors of one dtype (float32 or
    bfloat16) with a contiguous last dim.  Returns (out, lse); lse is None when
    ``return_lse`` is false.  ``scale=None`` selects 1/sqrt(D).
    """
    out, lse, _ = _fwd(q, k, v, block_mask, score, mask, scale, return_lse, False, out, lse, None, workspace)
    return out, lse


def flex_attn_fwd_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, block_mask: BlockMask,
                          out: torch.Tensor, lse: Optional[torch.Tensor] = None,
                          score: Optional[ScoreSpec] = None, mask: Optional[MaskSpec] = None,
                          scale: Optional[float] = None):
    """flex_attn_fwd that allocates nothing (C: flex_attn_fwd_noalloc).

    ``out`` (and ``lse``, if wanted) are the caller's; the split-KV scratch is
    the library's per-GPU array.  Calls that overlap in time on one GPU race.
    Returns (out, lse)."""
    lib = load_library()
    score = score or ScoreSpec()
    mask = mask or MaskSpec()
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k and v must be 4-D (B, H, seq, D)")
    B, Hq, L, D = q.shape
    Hkv, S = k.shape[1], k.shape[2]
    if k.shape[0] != B or v.shape[:3] != k.shape[:3] or k.shape[3] != D or v.shape[3] != D:
        raise ValueError(f"shape mismatch: q {tuple(q.shape)} k {tuple(k.shape)} v {tuple(v.shape)}")
    if not (q.dtype == k.dtype == v.dtype) or q.dtype not in DTYPES:
        raise ValueError("q, k, v must share a dtype, float32 or bfloat16")
    _require_qkv(q, k, v)
    dev = q.device
    _require(out, "out", dev, dtype=q.dtype, shape=(B, Hq, L, D))
    if lse is not None:
        _require(lse, "lse", dev, dtype=torch.float32, shape=(B, Hq, L))
    block_mask._validate(dev)
    _require_mask_tensors(mask, dev, B)
    st = lambda t: (ctypes.c_int64 * 3)(t.stride(0), t.stride(1), t.stride(2))
    cs, cm, cbm = score.to_c(), mask.to_c(L, S), block_mask.to_c()
    _check(lib.flex_attn_fwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), DTYPES[q.dtype], B, Hq, Hkv, L, S, D,
                                     st(q), st(k), st(v), ctypes.c_float(0.0 if scale is None else float(scale)),
                                     ctypes.byref(cs), ctypes.byref(cm), ctypes.byref(cbm), out.data_ptr(),
                                     None if lse is None else lse.data_ptr(),
                                     ctypes.c_void_p(_stream_ptr(dev))))
    return out, lse


def flex_attn_fwd_aux(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, block_mask: BlockMask,
                      score: Optional[ScoreSpec] = None, mask: Optional[MaskSpec] = None,
                      scale: Optional[float] = None, return_lse: bool = True, return_max_scores: bool = True,
                      out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                      max_scores: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None):
    """flex_attn_fwd plus the per-row maximum visible score (C: flex_attn_fwd_aux).

    Returns (out, lse, max_scores); an output not requested is None."""
    return _fwd(q, k, v, block_mask, score, mask, scale, return_lse, return_max_scores, out, lse, max_scores,
                workspace)


def _fwd(q, k, v, block_mask, score, mask, scale, return_lse, return_max, out, lse, max_scores, workspace):
    lib = load_library()
    score = score or ScoreSpec()
    mask = mask or MaskSpec()
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k and v must be 4-D (B, H, seq, D)")
    B, Hq, L, D = q.shape
    Hkv, S = k.shape[1], k.shape[2]
    if k.shape[0] != B or v.shape[:3] != k.shape[:3] or k.shape[3] != D or v.shape[3] != D:
        raise ValueError(f"shape mismatch: q {tuple(q.shape)} k {tuple(k.shape)} v {tuple(v.shape)}")
    if not (q.dtype == k.dtype == v.dtype) or q.dtype not in DTYPES:
        raise ValueError("q, k, v must share a dtype, float32 or bfloat16")
    _require_qkv(q, k, v)
    dev = q.device
    if out is None:
        out = torch.empty((B, Hq, L, D), dtype=q.dtype, device=dev)
    _require(out, "out", dev, dtype=q.dtype, shape=(B, Hq, L, D))
    if return_lse and lse is None:
        lse = torch.empty((B, Hq, L), dtype=torch.float32, device=dev)
    if not return_lse:
        lse = None
    if lse is not None:
        _require(lse, "lse", dev, dtype=torch.float32, shape=(B, Hq, L))
    if return_max and max_scores is None:
        max_scores = torch.empty((B, Hq, L), dtype=torch.float32, device=dev)
    if not return_max:
        max_scores = None
    if max_scores is not None:
        _require(max_scores, "max_scores", dev, dtype=torch.float32, shape=(B, Hq, L))
    block_mask._validate(dev)
    _require_mask_tensors(mask, dev, B)
    cbm = block_mask.to_c()
    ws_bytes = int(lib.flex_attn_fwd_workspace_bytes(DTYPES[q.dtype], B, Hq, Hkv, L, S, D, ctypes.byref(cbm)))
    _require_workspace(workspace, ws_bytes, dev)
    if ws_bytes and workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    st = lambda t: (ctypes.c_int64 * 3)(t.stride(0), t.stride(1), t.stride(2))
    cs, cm = score.to_c(), mask.to_c(L, S)
    args = [q.data_ptr(), k.data_ptr(), v.data_ptr(), DTYPES[q.dtype], B, Hq, Hkv, L, S, D, st(q), st(k), st(v),
            ctypes.c_float(0.0 if scale is None else float(scale)), ctypes.byref(cs), ctypes.byref(cm),
            ctypes.byref(cbm), out.data_ptr(), None if lse is None else lse.data_ptr()]
    tail = [None if not ws_bytes else workspace.data_ptr(), ws_bytes, ctypes.c_void_p(_stream_ptr(q.device))]
    if max_scores is None:
        status = lib.flex_attn_fwd(*args, *tail)
    else:
        status = lib.flex_attn_fwd_aux(*args, max_scores.data_ptr(), *tail)
    _check(status)
    return out, lse, max_scores


@dataclasses.dataclass
class BlockMaskQ:
    """The Q-side (transposed) lists of a BlockMask (int32 device tensors)."""
    q_num_blocks: torch.Tensor
    q_indices: torch.Tensor
    full_q_num_blocks: torch.Tensor
    full_q_indices: torch.Tensor
    q_block: int
    kv_block: int
    L: int
    S: int

    def _validate(self, device, block_mask: "BlockMask"):
        """int32, contiguous, on ``device``, transposed dims of ``block_mask``."""
        B, H, nqb, nkb = block_mask.kv_indices.shape
        for name, shape in (("q_num_blocks", (B, H, nkb)), ("q_indices", (B, H, nkb, nqb)),
                            ("full_q_num_blocks", (B, H, nkb)), ("full_q_indices", (B, H, nkb, nqb))):
            _require(getattr(self, name), f"Q-side block mask {name}", device, dtype=torch.int32, shape=shape)

    def to_c(self) -> flex_block_mask_q:
        cached = self.__dict__.get("_c")
        if cached is not None:
            return cached
        c = flex_block_mask_q()
        c.B, c.H = self.q_num_blocks.shape[0], self.q_num_blocks.shape[1]
        c.q_block, c.kv_block = self.q_block, self.kv_block
        c.num_kv_blocks, c.num_q_blocks = self.q_indices.shape[2], self.q_indices.shape[3]
        c.q_num_blocks = self.q_num_blocks.data_ptr()
        c.q_indices = self.q_indices.data_ptr()
        c.full_q_num_blocks = self.full_q_num_blocks.data_ptr()
        c.full_q_indices = self.full_q_indices.data_ptr()
        self.__dict__["_c"] = c
        return c


def flex_blockmask_transpose(block_mask: BlockMask, out: Optional[BlockMaskQ] = None) -> BlockMaskQ:
    """Fill the Q-side lists of a BlockMask on the GPU (C: flex_blockmask_transpose)."""
    lib = load_library()
    B, H, nqb, nkb = block_mask.kv_indices.shape
    if out is None:
        dev = block_mask.kv_indices.device
        t = lambda *shape: torch.empty(shape, dtype=torch.int32, device=dev)
        out = BlockMaskQ(t(B, H, nkb), t(B, H, nkb, nqb), t(B, H, nkb), t(B, H, nkb, nqb), block_mask.q_block,
                         block_mask.kv_block, block_mask.L, block_mask.S)
    block_mask._validate()
    out._validate(block_mask.kv_indices.device, block_mask)
    cbm, cq = block_mask.to_c(), out.to_c()
    _check(lib.flex_blockmask_transpose(ctypes.byref(cbm), ctypes.byref(cq),
                                        ctypes.c_void_p(_stream_ptr(block_mask.kv_indices.device))))
    return out


def flex_attn_bwd_workspace_bytes(dtype: torch.dtype, B: int, Hq: int, Hkv: int, L: int, S: int, D: int,
                                  block_mask: BlockMask) -> int:
    cbm = block_mask.to_c()
    return int(load_library().flex_attn_bwd_workspace_bytes(DTYPES[dtype], B, Hq, Hkv, L, S, D, ctypes.byref(cbm)))


def flex_attn_bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, out: torch.Tensor, dout: torch.Tensor,
                  lse: torch.Tensor, *, block_mask: BlockMask, block_mask_q: BlockMaskQ,
                  score: Optional[ScoreSpec] = None, mask: Optional[MaskSpec] = None, scale: Optional[float] = None,
                  dq: Optional[torch.Tensor] = None, dk: Optional[torch.Tensor] = None,
                  dv: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None):
    """Gradients of sum(out * dout) with respect to q, k, v (C: flex_attn_bwd).

    q, k, v, score, mask, scale and block_mask as for the flex_attn_fwd call
    that returned out and lse; dout like out.  Returns (dq, dk, dv)."""
    B, Hkv, S = q.shape[0], k.shape[1], k.shape[2]
    if q.dim() != 4 or k.dim() != 4 or k.shape[0] != B or v.shape[:3] != k.shape[:3]:
        raise ValueError(f"shape mismatch: q {tuple(q.shape)} k {tuple(k.shape)} v {tuple(v.shape)}")
    return _bwd(q, k, v, None, S, out, dout, lse, block_mask, block_mask_q, score, mask, scale, dq, dk, dv,
                workspace)


def flex_attn_bwd_paged(q: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor, page_table: torch.Tensor,
                        out: torch.Tensor, dout: torch.Tensor, lse: torch.Tensor, *, S: int, block_mask: BlockMask,
                        block_mask_q: BlockMaskQ, score: Optional[ScoreSpec] = None,
                        mask: Optional[MaskSpec] = None, scale: Optional[float] = None,
                        dq: Optional[torch.Tensor] = None, dk: Optional[torch.Tensor] = None,
                        dv: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None):
    """Backward of flex_attn_fwd_paged (C: flex_attn_bwd_paged): pools, page
    table and S as for that call.  Returns (dq, dk, dv) with dk, dv the
    gradients of the logical keys and values, (B, Hkv, S, D)."""
    if k_pool.dim() != 4 or v_pool.shape != k_pool.shape:
        raise ValueError(f"pool shapes {tuple(k_pool.shape)} / {tuple(v_pool.shape)} differ or are not 4-D")
    B = q.shape[0]
    if page_table.dtype != torch.int32 or not page_table.is_contiguous() or page_table.dim() != 2 \
            or page_table.shape[0] != B:
        raise ValueError("page_table must be a contiguous int32 (B, max_pages) tensor")
    _require(page_table, "page_table", q.device, dtype=torch.int32)
    pages = flex_kv_pages()
    pages.page_table = page_table.data_ptr()
    pages.page_size, pages.max_pages, pages.num_pages = k_pool.shape[2], page_table.shape[1], k_pool.shape[0]
    return _bwd(q, k_pool, v_pool, pages, int(S), out, dout, lse, block_mask, block_mask_q, score, mask, scale, dq,
                dk, dv, workspace)


def _bwd(q, k, v, pages, S, out, dout, lse, block_mask, block_mask_q, score, mask, scale, dq, dk, dv, workspace):
    lib = load_library()
    score = score or ScoreSpec()
    mask = mask or MaskSpec()
    B, Hq, L, D = q.shape
    Hkv = k.shape[1]
    if k.shape[3] != D or v.shape[3] != D:
        raise ValueError(f"head dims differ: q {tuple(q.shape)} k {tuple(k.shape)} v {tuple(v.shape)}")
    if not (q.dtype == k.dtype == v.dtype == out.dtype == dout.dtype) or q.dtype not in DTYPES:
        raise ValueError("q, k, v, out, dout must share a dtype, float32 or bfloat16")
    _require_qkv(q, k, v)
    dev = q.device
    for t, name in ((out, "out"), (dout, "dout")):
        _require(t, name, dev, dtype=q.dtype, shape=(B, Hq, L, D))
    _require(lse, "lse", dev, dtype=torch.float32, shape=(B, Hq, L))
    if dq is None:
        dq = torch.empty((B, Hq, L, D), dtype=q.dtype, device=dev)
    if dk is None:
        dk = torch.empty((B, Hkv, S, D), dtype=q.dtype, device=dev)
    if dv is None:
        dv = torch.empty((B, Hkv, S, D), dtype=q.dtype, device=dev)
    _require(dq, "dq", dev, dtype=q.dtype, shape=(B, Hq, L, D))
    _require(dk, "dk", dev, dtype=q.dtype, shape=(B, Hkv, S, D))
    _require(dv, "dv", dev, dtype=q.dtype, shape=(B, Hkv, S, D))
    block_mask._validate(dev)
    block_mask_q._validate(dev, block_mask)
    _require_mask_tensors(mask, dev, B)
    cbm, cq = block_mask.to_c(), block_mask_q.to_c()
    ws_bytes = int(lib.flex_attn_bwd_workspace_bytes(DTYPES[q.dtype], B, Hq, Hkv, L, S, D, ctypes.byref(cbm)))
    _require_workspace(workspace, ws_bytes, dev)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    st = lambda t: (ctypes.c_int64 * 3)(t.stride(0), t.stride(1), t.stride(2))
    cs, cm = score.to_c(), mask.to_c(L, S)
    c_scale = ctypes.c_float(0.0 if scale is None else float(scale))
    tail = (DTYPES[q.dtype], B, Hq, Hkv, L, S, D, st(q), st(k), st(v), c_scale, ctypes.byref(cs), ctypes.byref(cm),
            ctypes.byref(cbm), ctypes.byref(cq), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), workspace.data_ptr(),
            ws_bytes, ctypes.c_void_p(_stream_ptr(q.device)))
    if pages is None:
        _check(lib.flex_attn_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), dout.data_ptr(),
                                 lse.data_ptr(), *tail))
    else:
        _check(lib.flex_attn_bwd_paged(q.data_ptr(), k.data_ptr(), v.data_ptr(), ctypes.byref(pages), out.data_ptr(),
                                       dout.data_ptr(), lse.data_ptr(), *tail))
    return dq, dk, dv


def flex_attn_fwd_paged(q: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor, page_table: torch.Tensor, *,
                        S: int, block_mask: BlockMask, score: Optional[ScoreSpec] = None,
                        mask: Optional[MaskSpec] = None, scale: Optional[float] = None, return_lse: bool = True,
                        return_max_scores: bool = False, out: Optional[torch.Tensor] = None,
                        lse: Optional[torch.Tensor] = None, max_scores: Optional[torch.Tensor] = None,
                        workspace: Optional[torch.Tensor] = None):
    """Forward over a paged K/V cache (C: flex_attn_fwd_paged).

    k_pool, v_pool: (num_pages, Hkv, page_size, D) device tensors, last dim
    contiguous; page_table: int32 (B, max_pages) device tensor; S: the logical
    capacity per batch.  Returns (out, lse, max_scores) as flex_attn_fwd_aux."""
    lib = load_library()
    score = score or ScoreSpec()
    mask = mask or MaskSpec()
    B, Hq, L, D = q.shape
    num_pages, Hkv, page_size = k_pool.shape[0], k_pool.shape[1], k_pool.shape[2]
    if v_pool.shape != k_pool.shape or k_pool.shape[3] != D:
        raise ValueError(f"pool shapes {tuple(k_pool.shape)} / {tuple(v_pool.shape)} do not match q {tuple(q.shape)}")
    if not (q.dtype == k_pool.dtype == v_pool.dtype) or q.dtype not in DTYPES:
        raise ValueError("q and the pools must share a dtype, float32 or bfloat16")
    if page_table.dtype != torch.int32 or not page_table.is_contiguous() or page_table.dim() != 2 \
            or page_table.shape[0] != B:
        raise ValueError("page_table must be a contiguous int32 (B, max_pages) tensor")
    _require_qkv(q, k_pool, v_pool, ("q", "k_pool", "v_pool"))
    dev = q.device
    _require(page_table, "page_table", dev, dtype=torch.int32)
    if out is None:
        out = torch.empty((B, Hq, L, D), dtype=q.dtype, device=dev)
    _require(out, "out", dev, dtype=q.dtype, shape=(B, Hq, L, D))
    lse = (lse if lse is not None else torch.empty((B, Hq, L), dtype=torch.float32, device=dev)) \
        if return_lse else None
    max_scores = (max_scores if max_scores is not None else
                  torch.empty((B, Hq, L), dtype=torch.float32, device=dev)) if return_max_scores else None
    for t, name in ((lse, "lse"), (max_scores, "max_scores")):
        if t is not None:
            _require(t, name, dev, dtype=torch.float32, shape=(B, Hq, L))
    block_mask._validate(dev)
    _require_mask_tensors(mask, dev, B)
    cbm = block_mask.to_c()
    ws_bytes = int(lib.flex_attn_fwd_workspace_bytes(DTYPES[q.dtype], B, Hq, Hkv, L, S, D, ctypes.byref(cbm)))
    _require_workspace(workspace, ws_bytes, dev)
    if ws_bytes and workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    pages = flex_kv_pages()
    pages.page_table = page_table.data_ptr()
    pages.page_size, pages.max_pages, pages.num_pages = page_size, page_table.shape[1], num_pages
    st = lambda t: (ctypes.c_int64 * 3)(t.stride(0), t.stride(1), t.stride(2))
    cs, cm = score.to_c(), mask.to_c(L, S)
    _check(lib.flex_attn_fwd_paged(q.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(), DTYPES[q.dtype], B, Hq, Hkv,
                                   L, S, D, st(q), st(k_pool), st(v_pool),
                                   ctypes.c_float(0.0 if scale is None else float(scale)), ctypes.byref(cs),
                                   ctypes.byref(cm), ctypes.byref(cbm), ctypes.byref(pages), out.data_ptr(),
                                   None if lse is None else lse.data_ptr(),
                                   None if max_scores is None else max_scores.data_ptr(),
                                   None if not ws_bytes else workspace.data_ptr(), ws_bytes,
                                   ctypes.c_void_p(_stream_ptr(q.device))))
    return out, lse, max_scores


def default_scale(D: int) -> float:
    """1/sqrt(D) rounded to float32, the value the library uses for scale <= 0."""
    import numpy as np
    return float(np.float32(1.0) / np.sqrt(np.float32(D)))
