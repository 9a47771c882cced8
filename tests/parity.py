"""Comparison helpers for the GPU parity tests (HIP path vs the CPU oracle).

Protocol:
* routing: near-tie tokens (selection-score gap at the K/K+1 boundary or at the
  kept-group boundary below 1e-6, on the oracle's fp64 scores) are counted and
  excused; every other token must select exactly the oracle's expert set, with
  gates within 1e-5 relative; expert counts must equal the bincount of the
  GPU's own indices and the oracle's counts once the near-tie tokens' GPU
  choices are substituted; a near-tie token's GPU choice must still be a
  top-K within 2e-6;
* outputs: per token, e_t = max|out_gpu - out_ref| / max|out_ref - r x_t|
  (error relative to the MoE contribution, not to the residual), over tokens
  that are not near-tie; max e_t must be within the dtype's bound.
"""
from __future__ import annotations

import numpy as np
import torch

TIE_WINDOW = 1e-6
TOL = {"f32": 1e-4, "bf16": 2e-2, "fp8": 6e-2}


def near_tie_mask(R) -> np.ndarray:
    return (R["gap_k"] < TIE_WINDOW) | (R["gap_g"] < TIE_WINDOW)


def check_routing(idx_gpu: torch.Tensor, gate_gpu: torch.Tensor, counts_gpu: torch.Tensor, R: dict, E: int,
                  G: int, kg: int, gate_rtol: float = 1e-5) -> dict:
    idx = idx_gpu.cpu().numpy().astype(np.int64)
    gate = gate_gpu.cpu().numpy().astype(np.float64)
    counts = counts_gpu.cpu().numpy().astype(np.int64)
    T, K = idx.shape
    near = near_tie_mask(R)
    ok = ~near
    # exact expert sets
    g_sorted = np.sort(idx, axis=1)
    o_sorted = np.sort(R["idx"], axis=1)
    bad = np.nonzero(ok & np.any(g_sorted != o_sorted, axis=1))[0]
    assert bad.size == 0, f"{bad.size} tokens route differently, first {bad[:5]}: gpu {idx[bad[:1]]} oracle {R['idx'][bad[:1]]}"
    # indices in range and distinct per token
    assert idx.min() >= 0 and idx.max() < E
    assert np.all(np.diff(g_sorted, axis=1) > 0)
    # gates, matched by expert id
    go = np.take_along_axis(gate, np.argsort(idx, axis=1), 1)
    ro = np.take_along_axis(R["gate"], np.argsort(R["idx"], axis=1), 1)
    rel = np.abs(go - ro) / np.maximum(np.abs(ro), 1e-30)
    worst = float(rel[ok].max()) if ok.any() else 0.0
    assert worst <= gate_rtol, f"gate rel err {worst}"
    # counts
    assert np.array_equal(counts, np.bincount(idx.ravel(), minlength=E))
    subst = R["idx"].copy()
    subst[near] = idx[near]
    assert np.array_equal(counts, np.bincount(subst.ravel(), minlength=E))
    # near-tie tokens: the GPU choice is still a top-K within the window
    z = R["z"]
    for t in np.nonzero(near)[0]:
        sel = idx[t]
        if G > 1:
            assert len(set((sel // (E // G)).tolist())) <= kg
        assert z[t, sel].sum() >= z[t, R["idx"][t]].sum() - K * 2 * TIE_WINDOW
    return dict(near_tie=int(near.sum()), gate_rel_err=worst, tokens=T)


def layer_error(out_gpu_rows: torch.Tensor, out_ref_rows: np.ndarray, x_rows: np.ndarray, r: bool,
                exclude: np.ndarray | None = None) -> dict:
    g = out_gpu_rows.float().cpu().numpy().astype(np.float64)
    num = np.abs(g - out_ref_rows).max(axis=1)
    den = np.abs(out_ref_rows - (x_rows if r else 0.0)).max(axis=1)
    e = num / np.maximum(den, 1e-30)
    keep = np.ones(len(e), bool) if exclude is None else ~exclude
    assert np.all(np.isfinite(g))
    return dict(max=float(e[keep].max()) if keep.any() else 0.0, median=float(np.median(e[keep])) if keep.any() else 0.0,
                n=int(keep.sum()))
