"""Python binding of libmi_sparse.so: MInference-style dynamic sparse prefill
attention on MI355X (gfx950).

Argument marshalling only.  Every step of the computation runs in the HIP
kernels behind the C ABI declared in include/mi_sparse.h; torch provides
device memory (outputs, workspaces) and the current stream.  There is no CPU
or torch fallback: if the library is missing, every call raises.

Tensors: q [B, Hq, N, d], k and v [B, Hkv, N, d], float32 or bfloat16, on the
GPU, last dimension contiguous.  Query head h reads kv head h // (Hq // Hkv).
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional, Sequence

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmi_sparse.so")

MI_BLOCK = 64
MI_MAX_HEADS = 256
MI_F32, MI_BF16 = 0, 1
ASHAPE, VSLASH, BSPARSE, DENSE, VSLASH_EXACT = 0, 1, 2, 3, 4
VS_PATTERNS = (VSLASH, VSLASH_EXACT)
OP_VS_ESTIMATE, OP_BLOCK_ESTIMATE, OP_SPARSE_PREFILL, OP_ANTIDIAG_ESTIMATE = 0, 1, 2, 3
STATUS = {0: "MI_OK", 1: "MI_ERR_NULL", 2: "MI_ERR_SHAPE", 3: "MI_ERR_BUDGET", 4: "MI_ERR_DTYPE",
          5: "MI_ERR_WORKSPACE", 6: "MI_ERR_LAUNCH", 7: "MI_ERR_PATTERN"}

EXPORTS = ("mi_workspace_bytes", "mi_vs_estimate", "mi_block_estimate", "mi_antidiag_estimate", "mi_build_index",
           "mi_sparse_prefill", "mi_sparse_prefill_noalloc", "mi_attn_schedule", "mi_status_str",
           "mi_last_error")
NOALLOC_SCHEDULE_ENTRIES = 1 << 18


class MiError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS.get(status, status)}: {msg}")
        self.status = status


class MiAttnDesc(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("heads_q", ctypes.c_int32), ("heads_kv", ctypes.c_int32),
                ("seq_len", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("scale", ctypes.c_float),
                ("q_stride", ctypes.c_int64 * 3), ("k_stride", ctypes.c_int64 * 3),
                ("v_stride", ctypes.c_int64 * 3), ("o_stride", ctypes.c_int64 * 3)]


class MiIndex(ctypes.Structure):
    _fields_ = [("block_count", ctypes.c_void_p), ("block_idx", ctypes.c_void_p),
                ("col_count", ctypes.c_void_p), ("col_idx", ctypes.c_void_p),
                ("block_cap", ctypes.c_int32), ("col_cap", ctypes.c_int32), ("vs_bits", ctypes.c_void_p)]


_lib = None

_P = ctypes.c_void_p
_I = ctypes.c_int32
_SIGS = {
    "mi_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(MiAttnDesc), _I, _I, _I]),
    "mi_vs_estimate": (_I, [ctypes.POINTER(MiAttnDesc), _P, _P, _P, _I, _I, _I, _I, _I, _I,
                            _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "mi_block_estimate": (_I, [ctypes.POINTER(MiAttnDesc), _P, _P, _P, _I, _I, _P, _P, _P, _P,
                               ctypes.c_size_t, _P]),
    "mi_antidiag_estimate": (_I, [ctypes.POINTER(MiAttnDesc), _P, _P, _P, _I, _I, _P, _P, _P, _P,
                                  ctypes.c_size_t, _P]),
    "mi_build_index": (_I, [ctypes.POINTER(MiAttnDesc), _P, _P, _I, _P, _I, _P, _P, _I, _I, _I,
                            ctypes.POINTER(MiIndex), _P]),
    "mi_sparse_prefill": (_I, [ctypes.POINTER(MiAttnDesc), _P, _P, _P, _P, ctypes.POINTER(MiIndex),
                               _I, _I, _P, _P, _P, ctypes.c_size_t, _P]),
    "mi_sparse_prefill_noalloc": (_I, [ctypes.POINTER(MiAttnDesc), _P, _P, _P, _P, ctypes.POINTER(MiIndex),
                                       _I, _I, _P, _P, _P]),
    "mi_attn_schedule": (_I, [ctypes.POINTER(MiAttnDesc), _P, _I, _I, _I, _P, _I]),
    "mi_status_str": (ctypes.c_char_p, [_I]),
    "mi_last_error": (ctypes.c_char_p, []),
}


def lib():
    """The loaded native library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                              "(or python dynamic_sparse_attention_amd/build.py)")
        l = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(l, name)
            f.restype = res
            f.argtypes = args
        _lib = l
    return _lib


def _check(status: int):
    if status != 0:
        raise MiError(status, lib().mi_last_error().decode())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return MI_F32
    if t.dtype == torch.bfloat16:
        return MI_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _strides(t: Optional[torch.Tensor]):
    if t is None:
        return (0, 0, 0)
    if t.dim() != 4 or t.stride(3) != 1:
        raise ValueError("tensors must be 4-D [B, H, N, d] with a contiguous last dimension")
    return tuple(int(s) for s in t.stride()[:3])


def make_desc(q: torch.Tensor, k: torch.Tensor, v: Optional[torch.Tensor] = None,
              o: Optional[torch.Tensor] = None, scale: Optional[float] = None) -> MiAttnDesc:
    B, Hq, N, d = q.shape
    d_ = MiAttnDesc()
    d_.batch, d_.heads_q, d_.heads_kv, d_.seq_len, d_.head_dim = B, Hq, k.shape[1], N, d
    d_.dtype = _dtype_code(q)
    d_.scale = float(scale) if scale is not None else float(d) ** -0.5
    for name, t in (("q_stride", q), ("k_stride", k), ("v_stride", v), ("o_stride", o)):
        getattr(d_, name)[:] = _strides(t)
    return d_


def _stream(stream=None) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return int(s.cuda_stream)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _heads_arr(heads: Sequence[int]):
    arr = (ctypes.c_int32 * len(heads))(*[int(h) for h in heads])
    return arr


def workspace_bytes(desc: MiAttnDesc, op: int, p0: int = 0, p1: int = 0) -> int:
    return int(lib().mi_workspace_bytes(ctypes.byref(desc), op, p0, p1))


def _workspace(nbytes: int, device) -> torch.Tensor:
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


# ----------------------------------------------------------------------------
# The four calls
# ----------------------------------------------------------------------------

def vs_estimate(q, k, heads: Sequence[int], last_q: int = 64, n_vertical: int = 1000,
                n_slash: int = 6096, force_vertical: int = 1, force_slash: int = 1,
                scale: Optional[float] = None, return_scores: bool = True, outputs=None,
                stream=None):
    """Vertical-Slash estimate.  Returns (vertical_idx [B,Hq,n_vertical],
    slash_idx [B,Hq,n_slash], vertical_score [B,Hq,N] | None, slash_score | None);
    rows of heads not listed are left as allocated (zero)."""
    desc = make_desc(q, k, scale=scale)
    B, Hq, N, _ = q.shape
    dev = q.device
    if outputs is None:
        vidx = torch.zeros((B, Hq, n_vertical), dtype=torch.int32, device=dev)
        sidx = torch.zeros((B, Hq, n_slash), dtype=torch.int32, device=dev)
        vsc = torch.zeros((B, Hq, N), dtype=torch.float32, device=dev) if return_scores else None
        ssc = torch.zeros((B, Hq, N), dtype=torch.float32, device=dev) if return_scores else None
    else:
        vidx, sidx, vsc, ssc = outputs
    need = lib().mi_workspace_bytes(ctypes.byref(desc), OP_VS_ESTIMATE, len(heads), 0)
    ws = _workspace(need, dev)
    hs = _heads_arr(heads)
    _check(lib().mi_vs_estimate(ctypes.byref(desc), _ptr(q), _ptr(k), ctypes.cast(hs, _P), len(heads),
                                last_q, n_vertical, n_slash, force_vertical, force_slash,
                                _ptr(vidx), _ptr(sidx), _ptr(vsc), _ptr(ssc), _ptr(ws), ws.numel(),
                                _stream(stream)))
    return vidx, sidx, vsc, ssc


def block_estimate(q, k, heads: Sequence[int], top_blocks: int = 100, scale: Optional[float] = None,
                   return_scores: bool = True, outputs=None, stream=None):
    """Block-Sparse estimate.  Returns (block_idx [B,Hq,nb,top], block_count
    [B,Hq,nb], block_score [B,Hq,nb,nb] | None)."""
    desc = make_desc(q, k, scale=scale)
    B, Hq, N, _ = q.shape
    nb = N // MI_BLOCK
    dev = q.device
    if outputs is None:
        bidx = torch.zeros((B, Hq, nb, top_blocks), dtype=torch.int32, device=dev)
        bcnt = torch.zeros((B, Hq, nb), dtype=torch.int32, device=dev)
        w = torch.zeros((B, Hq, nb, nb), dtype=torch.float32, device=dev) if return_scores else None
    else:
        bidx, bcnt, w = outputs
    need = lib().mi_workspace_bytes(ctypes.byref(desc), OP_BLOCK_ESTIMATE, len(heads), 0)
    ws = _workspace(need, dev)
    hs = _heads_arr(heads)
    _check(lib().mi_block_estimate(ctypes.byref(desc), _ptr(q), _ptr(k), ctypes.cast(hs, _P), len(heads),
                                   top_blocks, _ptr(bidx), _ptr(bcnt), _ptr(w), _ptr(ws), ws.numel(),
                                   _stream(stream)))
    return bidx, bcnt, w


def antidiag_estimate(q, k, heads: Sequence[int], top_blocks: int = 100, scale: Optional[float] = None,
                   return_scores: bool = True, outputs=None, stream=None):
    """Block-Sparse lists from antidiagonal block scores (see
    mi_antidiag_estimate).  Returns (block_idx [B,Hq,nb,top], block_count
    [B,Hq,nb], block_score [B,Hq,nb,nb] | None)."""
    desc = make_desc(q, k, scale=scale)
    B, Hq, N, _ = q.shape
    nb = N // MI_BLOCK
    dev = q.device
    if outputs is None:
        bidx = torch.zeros((B, Hq, nb, top_blocks), dtype=torch.int32, device=dev)
        bcnt = torch.zeros((B, Hq, nb), dtype=torch.int32, device=dev)
        w = torch.zeros((B, Hq, nb, nb), dtype=torch.float32, device=dev) if return_scores else None
    else:
        bidx, bcnt, w = outputs
    need = lib().mi_workspace_bytes(ctypes.byref(desc), OP_ANTIDIAG_ESTIMATE, len(heads), 0)
    ws = _workspace(need, dev)
    hs = _heads_arr(heads)
    _check(lib().mi_antidiag_estimate(ctypes.byref(desc), _ptr(q), _ptr(k), ctypes.cast(hs, _P), len(heads),
                                      top_blocks, _ptr(bidx), _ptr(bcnt), _ptr(w), _ptr(ws), ws.numel(),
                                      _stream(stream)))
    return bidx, bcnt, w


@dataclass
class Index:
    block_count: torch.Tensor  # [B, Hq, nb]
    block_idx: torch.Tensor    # [B, Hq, nb, block_cap]
    col_count: torch.Tensor    # [B, Hq, nb]
    col_idx: torch.Tensor      # [B, Hq, nb, col_cap]
    vs_bits: Optional[torch.Tensor] = None  # [B, Hq, 2, N/32 + 4] int32 maps of exact VS heads

    @property
    def block_cap(self):
        return int(self.block_idx.shape[-1])

    @property
    def col_cap(self):
        return int(self.col_idx.shape[-1])

    def c_struct(self) -> MiIndex:
        s = MiIndex()
        s.block_count, s.block_idx = self.block_count.data_ptr(), self.block_idx.data_ptr()
        s.col_count, s.col_idx = self.col_count.data_ptr(), self.col_idx.data_ptr()
        s.block_cap, s.col_cap = self.block_cap, self.col_cap
        s.vs_bits = self.vs_bits.data_ptr() if self.vs_bits is not None else None
        return s


def index_caps(n: int, patterns, n_vertical: int = 0, n_slash: int = 0, top_blocks: int = 0,
               sink: int = 128, local: int = 4096):
    """Smallest list capacities that mi_build_index accepts for these patterns."""
    nb = n // MI_BLOCK
    pats = set(int(p) for p in patterns)
    bcap, ccap = 1, 1
    if pats & set(VS_PATTERNS):
        bcap = max(bcap, min(nb, 2 * n_slash))
        ccap = max(ccap, min(n_vertical, n))
    if BSPARSE in pats:
        bcap = max(bcap, min(top_blocks, nb))
    if ASHAPE in pats:
        bcap = max(bcap, min(nb, (sink + 63) // 64 + (local + 126) // 64))
    return bcap, ccap


def alloc_index(B: int, Hq: int, n: int, block_cap: int, col_cap: int, device, exact: bool = False) -> Index:
    """Index buffers; exact=True adds the membership maps of exact
    Vertical-Slash heads."""
    nb = n // MI_BLOCK
    return Index(
        torch.zeros((B, Hq, nb), dtype=torch.int32, device=device),
        torch.zeros((B, Hq, nb, block_cap), dtype=torch.int32, device=device),
        torch.zeros((B, Hq, nb), dtype=torch.int32, device=device),
        torch.zeros((B, Hq, nb, max(col_cap, 1)), dtype=torch.int32, device=device),
        torch.zeros((B, Hq, 2, n // 32 + 4), dtype=torch.int32, device=device) if exact else None)


def build_index(q, k, head_pattern: Sequence[int], vertical_idx=None, slash_idx=None,
                bs_block_idx=None, bs_block_count=None, top_blocks: int = 100, sink: int = 128,
                local: int = 4096, index: Optional[Index] = None, stream=None) -> Index:
    """Per-query-block work lists for every head (see mi_build_index)."""
    desc = make_desc(q, k)
    B, Hq, N, _ = q.shape
    nv = int(vertical_idx.shape[-1]) if vertical_idx is not None else 0
    ns = int(slash_idx.shape[-1]) if slash_idx is not None else 0
    if index is None:
        bcap, ccap = index_caps(N, head_pattern, nv, ns, top_blocks, sink, local)
        index = alloc_index(B, Hq, N, bcap, ccap, q.device, exact=VSLASH_EXACT in [int(p) for p in head_pattern])
    pat = (ctypes.c_int32 * Hq)(*[int(p) for p in head_pattern])
    st = index.c_struct()
    _check(lib().mi_build_index(ctypes.byref(desc), ctypes.cast(pat, _P), _ptr(vertical_idx), nv,
                                _ptr(slash_idx), ns, _ptr(bs_block_idx), _ptr(bs_block_count),
                                top_blocks, sink, local, ctypes.byref(st), _stream(stream)))
    return index


def sparse_prefill(q, k, v, head_pattern: Optional[Sequence[int]], index: Optional[Index],
                   sink: int = 128, local: int = 4096, scale: Optional[float] = None, out=None,
                   lse=None, return_lse: bool = True, stream=None, schedule: bool = False,
                   workspace: Optional[torch.Tensor] = None):
    """Sparse attention per head pattern; head_pattern=None runs dense causal
    attention on every head.  schedule=True (or a uint8 `workspace` tensor)
    passes a workspace in which the library builds the item schedule
    (grouping the heads of a kv group by pattern class).  Returns
    (o, lse | None)."""
    B, Hq, N, d = q.shape
    if out is None:
        out = torch.empty_like(q)
    if lse is None and return_lse:
        lse = torch.empty((B, Hq, N), dtype=torch.float32, device=q.device)
    desc = make_desc(q, k, v, out, scale=scale)
    pat = None if head_pattern is None else (ctypes.c_int32 * Hq)(*[int(p) for p in head_pattern])
    st = index.c_struct() if index is not None else None
    ws = workspace
    if ws is None and schedule:
        ws = _workspace(workspace_bytes(desc, OP_SPARSE_PREFILL), q.device)
    _check(lib().mi_sparse_prefill(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v),
                                   None if pat is None else ctypes.cast(pat, _P),
                                   None if st is None else ctypes.byref(st), sink, local,
                                   _ptr(out), _ptr(lse), None if ws is None else _ptr(ws),
                                   0 if ws is None else ws.numel(), _stream(stream)))
    return out, lse


def sparse_prefill_noalloc(q, k, v, head_pattern: Optional[Sequence[int]], index: Optional[Index],
                           sink: int = 128, local: int = 4096, scale: Optional[float] = None,
                           out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                           stream=None):
    """sparse_prefill with the item schedule in the library's built-in buffer
    (mi_sparse_prefill_noalloc): the caller passes preallocated out (and lse
    or None); nothing is allocated by the call.  Returns (out, lse)."""
    if out is None:
        raise ValueError("sparse_prefill_noalloc needs a preallocated out tensor")
    Hq = q.shape[1]
    desc = make_desc(q, k, v, out, scale=scale)
    pat = None if head_pattern is None else (ctypes.c_int32 * Hq)(*[int(p) for p in head_pattern])
    st = index.c_struct() if index is not None else None
    _check(lib().mi_sparse_prefill_noalloc(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v),
                                           None if pat is None else ctypes.cast(pat, _P),
                                           None if st is None else ctypes.byref(st), sink, local,
                                           _ptr(out), _ptr(lse), _stream(stream)))
    return out, lse


def attn_schedule(q, k, head_pattern: Optional[Sequence[int]], sink: int = 128, local: int = 4096,
                  block_cap: int = 1):
    """The attention item schedule for these shapes and patterns, built on the
    host (mi_attn_schedule): a list of packed items, -1 for padding."""
    desc = make_desc(q, k)
    Hq = q.shape[1]
    pat = None if head_pattern is None else (ctypes.c_int32 * Hq)(*[int(p) for p in head_pattern])
    cpat = None if pat is None else ctypes.cast(pat, _P)
    n = lib().mi_attn_schedule(ctypes.byref(desc), cpat, sink, local, block_cap, None, 0)
    if n < 0:
        raise MiError(7, "mi_attn_schedule rejected its arguments")
    buf = (ctypes.c_int32 * max(n, 1))()
    lib().mi_attn_schedule(ctypes.byref(desc), cpat, sink, local, block_cap, ctypes.cast(buf, _P), n)
    return list(buf[:n])


def layer_prefill(q, k, v, head_pattern: Sequence[int], *, last_q=64, n_vertical=1000, n_slash=6096,
                  force_vertical=1, force_slash=1, top_blocks=100, sink=128, local=4096,
                  scale=None, return_lse=False, stream=None):
    """One layer's whole hot path: estimates for the VS and BS heads, the
    index, and the sparse attention, all enqueued on one stream."""
    pat = [int(p) for p in head_pattern]
    vs_heads = [h for h, p in enumerate(pat) if p in VS_PATTERNS]
    bs_heads = [h for h, p in enumerate(pat) if p == BSPARSE]
    vidx = sidx = bidx = bcnt = None
    if vs_heads:
        vidx, sidx, _, _ = vs_estimate(q, k, vs_heads, last_q, n_vertical, n_slash, force_vertical,
                                       force_slash, scale=scale, return_scores=False, stream=stream)
    if bs_heads:
        bidx, bcnt, _ = block_estimate(q, k, bs_heads, top_blocks, scale=scale, return_scores=False,
                                       stream=stream)
    index = build_index(q, k, pat, vidx, sidx, bidx, bcnt, top_blocks, sink, local, stream=stream)
    o, lse = sparse_prefill(q, k, v, pat, index, sink, local, scale=scale, return_lse=return_lse,
                            stream=stream)
    return o, lse, dict(vertical_idx=vidx, slash_idx=sidx, bs_block_idx=bidx, bs_block_count=bcnt,
                        index=index)


class LayerPlan:
    """Buffers for one layer's hot path, allocated once; run() only enqueues
    the four library calls (estimates, index, attention) on one stream."""

    def __init__(self, q, k, v, head_pattern: Sequence[int], *, last_q=64, n_vertical=1000,
                 n_slash=6096, force_vertical=1, force_slash=1, top_blocks=100, sink=128,
                 local=4096, scale=None, with_lse=False):
        self.q, self.k, self.v = q, k, v
        self.pat = [int(p) for p in head_pattern]
        B, Hq, N, d = q.shape
        dev = q.device
        self.kw = dict(last_q=last_q, n_vertical=n_vertical, n_slash=n_slash,
                       force_vertical=force_vertical, force_slash=force_slash,
                       top_blocks=top_blocks, sink=sink, local=local)
        self.scale = scale
        self.vs_heads = [h for h, p in enumerate(self.pat) if p in VS_PATTERNS]
        self.bs_heads = [h for h, p in enumerate(self.pat) if p == BSPARSE]
        self.desc = make_desc(q, k, scale=scale)
        self.vidx = self.sidx = self.bidx = self.bcnt = None
        if self.vs_heads:
            self.vidx = torch.zeros((B, Hq, n_vertical), dtype=torch.int32, device=dev)
            self.sidx = torch.zeros((B, Hq, n_slash), dtype=torch.int32, device=dev)
            self.vs_ws = _workspace(workspace_bytes(self.desc, OP_VS_ESTIMATE, len(self.vs_heads)), dev)
            self.vs_heads_c = _heads_arr(self.vs_heads)
        if self.bs_heads:
            nb = N // MI_BLOCK
            self.bidx = torch.zeros((B, Hq, nb, top_blocks), dtype=torch.int32, device=dev)
            self.bcnt = torch.zeros((B, Hq, nb), dtype=torch.int32, device=dev)
            self.bs_ws = _workspace(workspace_bytes(self.desc, OP_BLOCK_ESTIMATE, len(self.bs_heads)), dev)
            self.bs_heads_c = _heads_arr(self.bs_heads)
        bcap, ccap = index_caps(N, self.pat, n_vertical, n_slash, top_blocks, sink, local)
        self.index = alloc_index(B, Hq, N, bcap, ccap, dev, exact=VSLASH_EXACT in self.pat)
        self.index_c = self.index.c_struct()
        self.pat_c = (ctypes.c_int32 * Hq)(*self.pat)
        self.o = torch.empty_like(q)
        self.lse = torch.empty((B, Hq, N), dtype=torch.float32, device=dev) if with_lse else None
        self.attn_desc = make_desc(q, k, v, self.o, scale=scale)
        # attention item schedule (chunks of one kv group and pattern class)
        self.attn_ws = _workspace(workspace_bytes(self.attn_desc, OP_SPARSE_PREFILL, 0), dev)

    def estimate(self, stream=None):
        kw, s, l = self.kw, _stream(stream), lib()
        if self.vs_heads:
            _check(l.mi_vs_estimate(ctypes.byref(self.desc), _ptr(self.q), _ptr(self.k),
                                    ctypes.cast(self.vs_heads_c, _P), len(self.vs_heads), kw["last_q"],
                                    kw["n_vertical"], kw["n_slash"], kw["force_vertical"],
                                    kw["force_slash"], _ptr(self.vidx), _ptr(self.sidx), None, None,
                                    _ptr(self.vs_ws), self.vs_ws.numel(), s))
        if self.bs_heads:
            _check(l.mi_block_estimate(ctypes.byref(self.desc), _ptr(self.q), _ptr(self.k),
                                       ctypes.cast(self.bs_heads_c, _P), len(self.bs_heads),
                                       kw["top_blocks"], _ptr(self.bidx), _ptr(self.bcnt), None,
                                       _ptr(self.bs_ws), self.bs_ws.numel(), s))

    def build_index(self, stream=None):
        kw = self.kw
        nv = kw["n_vertical"] if self.vs_heads else 0
        ns = kw["n_slash"] if self.vs_heads else 0
        _check(lib().mi_build_index(ctypes.byref(self.desc), ctypes.cast(self.pat_c, _P), _ptr(self.vidx),
                                    nv, _ptr(self.sidx), ns, _ptr(self.bidx), _ptr(self.bcnt),
                                    kw["top_blocks"], kw["sink"], kw["local"], ctypes.byref(self.index_c),
                                    _stream(stream)))

    def attention(self, stream=None, dense=False):
        kw = self.kw
        _check(lib().mi_sparse_prefill(ctypes.byref(self.attn_desc), _ptr(self.q), _ptr(self.k),
                                       _ptr(self.v), None if dense else ctypes.cast(self.pat_c, _P),
                                       None if dense else ctypes.byref(self.index_c), kw["sink"],
                                       kw["local"], _ptr(self.o), _ptr(self.lse), _ptr(self.attn_ws),
                                       self.attn_ws.numel(), _stream(stream)))

    def run(self, stream=None):
        self.estimate(stream)
        self.build_index(stream)
        self.attention(stream)
        return self.o
