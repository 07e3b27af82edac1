"""Helpers for GPU parity tests: moving seeded inputs to the device and
comparing the HIP path's outputs with the oracle's.  No method arithmetic
lives here; the expected values always come from oracle/."""
from __future__ import annotations

import sys
import warnings

import numpy as np
import torch

import workloads as W
from oracle import minference_oracle as O

BF16_ATOL = 2e-2   # attention output, bf16 inputs (max abs)
F32_ATOL = 1e-4    # attention output, fp32 inputs (max abs)
SCORE_RTOL = 1e-3  # estimation scores (relative, elementwise)
NEAR_TIE = 1e-5    # relative score gap under which a selection flip is a near tie

# Every selection that differs from the fp64 oracle's (within NEAR_TIE) is
# recorded here and raised as a SelectionFlip warning; the session summary
# (tests/conftest.py) lists them, so a flip is never silent.
FLIPS: list = []
CHECKED = [0]  # selections compared with the fp64 oracle


class SelectionFlip(UserWarning):
    pass


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_device(x: np.ndarray, dtype: str, dev="cuda"):
    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(x)).to(dev)
    return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(dev)


def f64(x_dev: torch.Tensor) -> np.ndarray:
    return x_dev.detach().float().cpu().numpy().astype(np.float64)


def assert_scores_close(gpu: np.ndarray, ref: np.ndarray, what: str, rtol=SCORE_RTOL):
    gpu = np.asarray(gpu, np.float64)
    err = np.abs(gpu - ref)
    bad = err > rtol * np.abs(ref) + 1e-30
    assert not bad.any(), (f"{what}: {bad.sum()} scores off by more than {rtol} relative; "
                           f"worst at {np.argmax(err / (np.abs(ref) + 1e-30))}")
    return float((err / (np.abs(ref) + 1e-30)).max())


def check_selection(gpu_idx: np.ndarray, gpu_scores: np.ndarray, ref_scores: np.ndarray, k: int,
                    forced, what: str):
    """Gate: the oracle's selection applied to the GPU's own fp32 scores must
    equal the GPU's indices exactly.  Against the fp64 scores, any difference
    must be a near tie at the selection boundary; such flips are reported."""
    gpu_idx = np.asarray(gpu_idx)
    sel = gpu_idx[gpu_idx >= 0]
    own = O.select_topk(np.asarray(gpu_scores, np.float64), k, forced)
    assert np.array_equal(sel, own), f"{what}: GPU selection differs from its own scores' top-k"
    assert np.all(gpu_idx[len(sel):] == -1)
    ref = O.select_topk(ref_scores, k, forced)
    CHECKED[0] += 1
    if np.array_equal(sel, ref):
        return 0
    only_gpu = np.setdiff1d(sel, ref)
    only_ref = np.setdiff1d(ref, sel)
    kth = min(ref_scores[only_ref].min(), ref_scores[only_gpu].max())
    gap = np.abs(np.concatenate([ref_scores[only_gpu], ref_scores[only_ref]]) - kth).max()
    rel = gap / max(abs(kth), 1e-300)
    rec = {"what": what, "members": len(only_gpu), "only_gpu": [int(x) for x in only_gpu[:8]],
           "only_oracle": [int(x) for x in only_ref[:8]], "relative_gap": float(rel)}
    FLIPS.append(rec)
    say(f"  near-tie flip in {what}: {len(only_gpu)} members differ, relative gap {rel:.2e}")
    warnings.warn(SelectionFlip(f"{what}: {len(only_gpu)} members differ from the fp64 selection, "
                                f"relative gap {rel:.2e}"))
    assert rel <= NEAR_TIE, f"{what}: selection differs from the fp64 oracle beyond a near tie ({rel:.2e})"
    return len(only_gpu)


def gpu_index_lists(index, b, h, a):
    bc = int(index.block_count[b, h, a])
    blocks = index.block_idx[b, h, a, :bc].cpu().numpy()
    cc = int(index.col_count[b, h, a])
    cols = index.col_idx[b, h, a, :cc].cpu().numpy()
    return blocks, cols
