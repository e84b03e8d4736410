"""Helpers of the GPU parity tests: device copies of seeded inputs and the
tolerance checks.  Tolerances: compressor and indexer outputs within 1e-3
relative (normwise per row: max|diff| <= 1e-3 * max|oracle row|), bf16
outputs within one bf16 ulp of the rounded oracle value or that normwise
bound, top-k sets bit-exact on identical scores, attention outputs from bf16
inputs within max-abs 2e-2 and mean-abs 2e-3."""
from __future__ import annotations

import os
import sys

import numpy as np
import torch

import synth

REL = 1e-3
ATTN_MAX_ABS = 2e-2
ATTN_MEAN_ABS = 2e-3


def progress(msg):
    """Name the case on the real stderr (and a log) before a GPU step."""
    sys.__stderr__.write(f"[gpu] {msg}\n")
    sys.__stderr__.flush()
    d = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "gpurun_out")
    if os.path.isdir(d):
        with open(os.path.join(d, "gpu_progress.log"), "a") as f:
            f.write(msg + "\n")


def dev_bf16(bits):
    """uint16 bf16 bit patterns (numpy) -> torch.bfloat16 on cuda:0."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to("cuda").view(torch.bfloat16)


def dev(x, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(x))
    if dtype is not None:
        t = t.to(dtype)
    return t.to("cuda")


def host(t):
    if t.dtype == torch.bfloat16:
        return synth.bf16_to_f64(t.view(torch.int16).cpu().numpy().view(np.uint16))
    return t.cpu().numpy().astype(np.float64)


def assert_normwise(got, want, rel=REL, what=""):
    """Per-row (last axis) normwise relative check; -inf positions must match."""
    got = np.asarray(got, np.float64).reshape(-1, np.shape(want)[-1])
    want = np.asarray(want, np.float64).reshape(got.shape)
    ninf_w, ninf_g = np.isneginf(want), np.isneginf(got)
    assert np.array_equal(ninf_w, ninf_g), f"{what}: -inf pattern differs"
    g = np.where(ninf_w, 0.0, got)
    w = np.where(ninf_w, 0.0, want)
    assert np.all(np.isfinite(g)), f"{what}: non-finite output"
    err = np.max(np.abs(g - w), axis=1)
    ref = np.max(np.abs(w), axis=1)
    bad = err > rel * np.maximum(ref, 1e-30)
    assert not bad.any(), f"{what}: rows {np.nonzero(bad)[0][:8]} err {err[bad][:4]} ref {ref[bad][:4]}"


def assert_bf16_matches(got_bf16_f64, want, rel=REL, what=""):
    """bf16 output vs the oracle: within one bf16 ulp or the normwise bound."""
    got = np.asarray(got_bf16_f64).reshape(-1, np.shape(want)[-1])
    want = np.asarray(want, np.float64).reshape(got.shape)
    ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(want), 1e-38))) - 7)
    bound = np.maximum(ulp, rel * np.max(np.abs(want), axis=1, keepdims=True))
    bad = np.abs(got - want) > bound
    assert not bad.any(), f"{what}: {bad.sum()} elements off, worst {np.max(np.abs(got - want) - bound)}"


def assert_attn(got, want, what="", max_abs=ATTN_MAX_ABS, mean_abs=ATTN_MEAN_ABS):
    d = np.abs(np.asarray(got, np.float64) - np.asarray(want, np.float64))
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    assert d.max() <= max_abs, f"{what}: max abs {d.max():.3e}"
    assert d.mean() <= mean_abs, f"{what}: mean abs {d.mean():.3e}"
    return float(d.max()), float(d.mean())


def topk_set_check(got_sel, oracle_scores, oracle_sel, k, band=REL):
    """Sets equal except for swaps among scores within `band` of the k-th score.

    Returns the number of rows whose sets differ (legal swaps)."""
    swaps = 0
    for r in range(got_sel.shape[0]):
        g = set(int(i) for i in got_sel[r] if i >= 0)
        o = set(int(i) for i in oracle_sel[r] if i >= 0)
        assert len(g) == len(o), f"row {r}: {len(g)} vs {len(o)} selected"
        if g == o:
            continue
        s = oracle_scores[r]
        kth = min(s[i] for i in o)
        tol = band * abs(kth)
        for i in g ^ o:
            assert abs(s[i] - kth) <= tol, f"row {r}: entry {i} score {s[i]} outside the swap band of {kth}"
        swaps += 1
    return swaps
