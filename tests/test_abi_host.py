"""The C ABI on the host: the library loads, exports every declared entry
point, and rejects bad arguments before enqueuing anything.

No kernel is launched here: every call below fails validation, which runs
before any HIP call, so fake (never dereferenced) device addresses are used.
"""
import ctypes
import os
import re

import numpy as np
import pytest

import dynamic_sparse_attention_amd as mi

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "mi_sparse.h")
FAKE = 0x10000  # 16-byte aligned, never dereferenced


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^(?:mi_status|size_t|int32_t|const char\*)\s+(mi_\w+)\s*\(", text, re.M)))


def test_library_exports_every_declared_function():
    names = declared_functions()
    assert set(names) == set(mi.EXPORTS)
    l = mi.lib()
    for n in names:
        assert hasattr(l, n), n


def test_status_strings():
    l = mi.lib()
    for code in range(8):
        assert l.mi_status_str(code)
    assert l.mi_status_str(99) == b"unknown status"


def desc(**kw):
    d = mi.MiAttnDesc()
    d.batch, d.heads_q, d.heads_kv, d.seq_len, d.head_dim = 1, 4, 2, 1024, 128
    d.dtype, d.scale = mi.MI_BF16, 128 ** -0.5
    for name in ("q_stride", "k_stride", "v_stride", "o_stride"):
        getattr(d, name)[:] = (4 * 1024 * 128, 1024 * 128, 128)
    for k, v in kw.items():
        if k.endswith("_stride"):
            getattr(d, k)[:] = v
        else:
            setattr(d, k, v)
    return d


def heads(*h):
    return ctypes.cast((ctypes.c_int32 * len(h))(*h), ctypes.c_void_p)


def vs_call(d, hs=(0, 1), n_heads=None, last_q=64, nv=16, ns=32, fv=1, fs=1, ws=FAKE, ws_bytes=1 << 30,
            vidx=FAKE, sidx=FAKE, q=FAKE, vsc=None, ssc=None):
    l = mi.lib()
    return l.mi_vs_estimate(ctypes.byref(d), q, FAKE, heads(*hs), len(hs) if n_heads is None else n_heads,
                            last_q, nv, ns, fv, fs, vidx, sidx, vsc, ssc, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(seq_len=1000), 2), (dict(seq_len=0), 2), (dict(head_dim=96), 2), (dict(heads_kv=3), 2),
    (dict(heads_q=512, heads_kv=1), 2), (dict(dtype=7), 4), (dict(scale=0.0), 2),
    (dict(scale=float("nan")), 2), (dict(q_stride=(0, 1024 * 128, 100)), 2), (dict(batch=0), 2),
])
def test_bad_descriptor_rejected(kw, status):
    assert vs_call(desc(**kw)) == status
    assert mi.lib().mi_last_error()


@pytest.mark.parametrize("kw,status", [
    (dict(hs=(1, 0)), 7), (dict(hs=(0, 4)), 7), (dict(hs=(0, 0)), 7), (dict(n_heads=0), 7),
    (dict(last_q=0), 3), (dict(last_q=65), 3), (dict(nv=0), 3), (dict(fv=0), 3), (dict(fv=17), 3),
    (dict(fs=33), 3), (dict(ws_bytes=16), 5), (dict(ws=None), 5), (dict(vidx=None), 1),
    (dict(q=None), 1), (dict(q=FAKE + 4), 2), (dict(vsc=FAKE), 1),
])
def test_vs_estimate_validation(kw, status):
    assert vs_call(desc(), **kw) == status


def test_workspace_sizes():
    d = desc()
    l = mi.lib()
    vs = l.mi_workspace_bytes(ctypes.byref(d), mi.OP_VS_ESTIMATE, 2, 0)
    # per-chunk row statistics + row statistics + two score rows per listed head
    assert vs >= 2 * 2 * 1024 * 4 + 2 * 64 * 8
    bs = l.mi_workspace_bytes(ctypes.byref(d), mi.OP_BLOCK_ESTIMATE, 2, 0)
    nb = 1024 // 64
    # pooled query and key rows; rows of <= 512 blocks keep their scores on chip
    assert bs >= (2 * nb * 128 + 2 * nb * 128) * 4
    long = desc(seq_len=64 * 600, q_stride=(4 * 38400 * 128, 38400 * 128, 128),
                k_stride=(38400 * 128, 38400 * 128, 128))
    bs_long = l.mi_workspace_bytes(ctypes.byref(long), mi.OP_BLOCK_ESTIMATE, 2, 0)
    assert bs_long >= (2 * 600 * 128 + 2 * 600 * 128 + 2 * 600 * 600) * 4
    # attention item schedule: one int32 per (batch, head, run of 4 query blocks) plus padding
    pf = l.mi_workspace_bytes(ctypes.byref(d), mi.OP_SPARSE_PREFILL, 0, 0)
    assert pf >= 4 * 4 * (nb // 4) and pf % 256 == 0
    assert l.mi_workspace_bytes(ctypes.byref(desc(seq_len=10)), mi.OP_VS_ESTIMATE, 2, 0) == 0


def test_block_estimate_validation():
    l = mi.lib()
    d = desc()
    call = lambda top=4, ws_bytes=1 << 30, bidx=FAKE: l.mi_block_estimate(
        ctypes.byref(d), FAKE, FAKE, heads(0, 2), 2, top, bidx, FAKE, None, FAKE, ws_bytes, None)
    assert call(top=1) == 3
    assert call(ws_bytes=8) == 5
    assert call(bidx=None) == 1
    long = desc(seq_len=64 * 40000)
    assert l.mi_block_estimate(ctypes.byref(long), FAKE, FAKE, heads(0), 1, 4, FAKE, FAKE, None, FAKE,
                               1 << 40, None) == 2


def test_antidiag_estimate_validation():
    l = mi.lib()
    d = desc()
    # every call below fails validation, so nothing is launched on the fake pointers
    call = lambda top=4, ws_bytes=1 << 30, bidx=FAKE, q=FAKE: l.mi_antidiag_estimate(
        ctypes.byref(d), q, FAKE, heads(0, 2), 2, top, bidx, FAKE, None, FAKE, ws_bytes, None)
    assert call(top=1) == 3
    assert call(ws_bytes=8) == 5
    assert call(bidx=None) == 1
    assert call(q=FAKE + 8) == 2  # 16-byte alignment
    # the score rows live in the workspace unless the caller passes block_score
    nb = 1024 // 64
    need = l.mi_workspace_bytes(ctypes.byref(d), mi.OP_ANTIDIAG_ESTIMATE, 2, 0)
    assert need >= 2 * nb * nb * 4
    assert call(ws_bytes=need - 1) == 5
    long = desc(seq_len=64 * 40000)
    assert l.mi_antidiag_estimate(ctypes.byref(long), FAKE, FAKE, heads(0), 1, 4, FAKE, FAKE, None, FAKE,
                                  1 << 40, None) == 2


def index_struct(bcap=32, ccap=16, cols=True, bits=False):
    s = mi.MiIndex()
    s.block_count, s.block_idx = FAKE, FAKE
    s.col_count, s.col_idx = FAKE, (FAKE if cols else None)
    s.block_cap, s.col_cap = bcap, ccap
    s.vs_bits = FAKE if bits else None
    return s


def test_build_index_validation():
    l = mi.lib()
    d = desc()  # nb = 16
    pat = lambda *p: ctypes.cast((ctypes.c_int32 * 4)(*p), ctypes.c_void_p)

    def call(p, nv=16, ns=32, top=4, sink=128, local=256, out=None, vidx=FAKE, bs=FAKE):
        out = out or index_struct()
        return l.mi_build_index(ctypes.byref(d), p, vidx, nv, FAKE, ns, bs, FAKE, top, sink, local,
                                ctypes.byref(out), None)

    assert call(pat(0, 1, 2, 9)) == 7
    assert call(None) == 1
    assert call(pat(1, 1, 1, 1), vidx=None) == 1
    assert call(pat(1, 1, 1, 1), out=index_struct(bcap=15)) == 3       # min(nb, 2*32) = 16
    assert call(pat(1, 1, 1, 1), out=index_struct(ccap=15)) == 3       # min(16, 1024)
    assert call(pat(1, 1, 1, 1), out=index_struct(cols=False)) == 1
    assert call(pat(2, 2, 2, 2), top=40, out=index_struct(bcap=15)) == 3  # min(top, nb) = 16
    assert call(pat(2, 2, 2, 2), bs=None) == 1
    assert call(pat(0, 0, 0, 0), local=0) == 3
    assert call(pat(0, 0, 0, 0), sink=64, local=1000, out=index_struct(bcap=10)) == 3  # 1 + 17 -> 16
    assert call(pat(0, 0, 0, 0), sink=-1) == 3
    # exact Vertical-Slash heads: the same lists plus membership maps
    assert call(pat(4, 1, 1, 1), out=index_struct(bits=False)) == 1
    assert call(pat(4, 4, 4, 4), out=index_struct(bcap=15, bits=True)) == 3
    assert call(pat(4, 1, 1, 5)) == 7


def test_sparse_prefill_validation():
    l = mi.lib()
    d = desc()
    pat = lambda *p: ctypes.cast((ctypes.c_int32 * 4)(*p), ctypes.c_void_p)

    def call(p, idx=None, sink=128, local=256, o=FAKE):
        return l.mi_sparse_prefill(ctypes.byref(d), FAKE, FAKE, FAKE, p,
                                   None if idx is None else ctypes.byref(idx), sink, local, o, None,
                                   None, 0, None)

    assert call(pat(1, 1, 1, 1)) == 1                      # sparse heads need an index
    assert call(pat(1, 3, 3, 3), index_struct(cols=False)) == 1
    assert call(pat(0, 3, 3, 3), index_struct(), local=0) == 3
    assert call(pat(5, 3, 3, 3), index_struct()) == 7
    assert call(pat(4, 3, 3, 3), index_struct()) == 1       # exact heads need the maps
    assert call(pat(4, 3, 3, 3), index_struct(cols=False, bits=True)) == 1
    assert call(None, o=None) == 1
    assert call(None, o=FAKE + 8) == 2


def test_sparse_prefill_rejects_oversized_lds_and_strides():
    """The attention workgroup keeps its step list and the column lists of a
    run of query blocks in LDS: shapes beyond the 160 KiB an MI355X CU has are
    rejected on the host (MI_ERR_SHAPE) before any launch, as are K/V token
    strides whose 64-row span does not fit a 32-bit offset."""
    l = mi.lib()
    pat = ctypes.cast((ctypes.c_int32 * 4)(1, 1, 1, 1), ctypes.c_void_p)

    def call(d, idx, why):
        st = l.mi_sparse_prefill(ctypes.byref(d), FAKE, FAKE, FAKE, pat, ctypes.byref(idx), 128, 4096,
                                 FAKE, None, None, 0, None)
        assert why in ctypes.string_at(l.mi_last_error()).decode()
        return st
    # 2M tokens: the step list alone needs 128 KiB next to 64 KiB of staging tiles
    long = desc(seq_len=1 << 21)
    long.q_stride[:] = (4 << 21) * 128, (1 << 21) * 128, 128
    long.k_stride[:] = (2 << 21) * 128, (1 << 21) * 128, 128
    long.v_stride[:] = long.k_stride[:]
    long.o_stride[:] = long.q_stride[:]
    assert call(long, index_struct(), "bytes of LDS") == 2
    # 10000 columns per query block: 4 column lists of 40 KiB each
    big_cols = index_struct()
    big_cols.col_cap = 10000
    assert call(desc(), big_cols, "bytes of LDS") == 2
    # a token stride of 2^25 elements: 64 rows span 4 GiB
    wide = desc(k_stride=(1 << 40, 1 << 32, 1 << 25))
    assert call(wide, index_struct(), "strides too large") == 2
    # 256 rows of 16 MiB: a head's rows span 4 GiB (32-bit row offsets)
    far = desc(seq_len=256, v_stride=(1 << 40, 1 << 33, 1 << 23))
    assert call(far, index_struct(bcap=4, ccap=4), "span < 4 GiB") == 2



def test_attention_schedule_groups_heads_of_one_kv_group_and_class():
    """The attention item schedule is a permutation of every (b, h, run) item
    (plus -1 padding) in groups of four that share batch, kv group and
    pattern class, in run order within a group, ordered longest first."""
    l = mi.lib()
    B, Hq, Hkv, N = 2, 8, 2, 64 * 37  # 10 runs, the last one partial
    d = desc(batch=B, heads_q=Hq, heads_kv=Hkv, seq_len=N)
    pats = [1, 0, 2, 1, 3, 3, 0, 2]
    pat = ctypes.cast((ctypes.c_int32 * Hq)(*pats), ctypes.c_void_p)
    n = l.mi_attn_schedule(ctypes.byref(d), pat, 128, 256, 8, None, 0)
    buf = (ctypes.c_int32 * n)()
    assert l.mi_attn_schedule(ctypes.byref(d), pat, 128, 256, 8, buf, n) == n
    sched = np.array(buf[:], dtype=np.int64)
    assert n % 4 == 0 and n * 4 <= l.mi_workspace_bytes(ctypes.byref(d), mi.OP_SPARSE_PREFILL, 0, 0)
    nruns = (N // 64 + 3) // 4
    items = sched[sched >= 0]
    assert sorted(items.tolist()) == list(range(B * Hq * nruns))
    cls = lambda p: {0: 1, 2: 2}.get(p, 0)  # A-shape, Block-Sparse, else (VS / dense)
    group = Hq // Hkv
    prev_est = None
    for c in range(n // 4):
        chunk = [int(x) for x in sched[4 * c: 4 * c + 4] if x >= 0]
        assert chunk and all(x >= 0 for x in sched[4 * c: 4 * c + len(chunk)])  # padding only at the end
        bh = [x // nruns for x in chunk]
        runs = [x % nruns for x in chunk]
        keys = {(x // Hq, (x % Hq) // group, cls(pats[x % Hq])) for x in bh}
        assert len(keys) == 1
        assert runs == sorted(runs, reverse=True)
        first = runs[0]
        span = min(N // 64, 4 * (first + 1))
        k = cls(pats[bh[0] % Hq])
        est = span if k == 0 else min(span, (128 + 63) // 64 + (256 + 126) // 64 + 4) if k == 1 else min(span, 4 * 8)
        assert prev_est is None or est <= prev_est
        prev_est = est
    # dense comparator: every head in one class
    n2 = l.mi_attn_schedule(ctypes.byref(d), None, 128, 256, 8, None, 0)
    assert n2 == B * Hq * nruns


def test_noalloc_prefill_validation():
    """mi_sparse_prefill_noalloc validates like mi_sparse_prefill and rejects
    layers whose item schedule exceeds its built-in buffer, all before any
    HIP call."""
    l = mi.lib()
    pat = ctypes.cast((ctypes.c_int32 * 4)(1, 1, 1, 1), ctypes.c_void_p)
    d = desc()
    assert l.mi_sparse_prefill_noalloc(ctypes.byref(d), FAKE, FAKE, FAKE, pat, None, 128, 256, FAKE, None,
                                       None) == 1
    assert l.mi_sparse_prefill_noalloc(ctypes.byref(d), FAKE, FAKE, FAKE, None, None, 128, 256, None, None,
                                       None) == 1
    # 256 query heads x 1025 runs of four query blocks > 262144 schedule entries
    big = desc(heads_q=256, heads_kv=1, seq_len=64 * 4 * 1025, head_dim=64)
    for name in ("q_stride", "k_stride", "v_stride", "o_stride"):
        getattr(big, name)[:] = (0, 0, 0)
    assert l.mi_sparse_prefill_noalloc(ctypes.byref(big), FAKE, FAKE, FAKE, None, None, 128, 256, FAKE, None,
                                       None) == 5
    assert b"built-in buffer" in l.mi_last_error()
