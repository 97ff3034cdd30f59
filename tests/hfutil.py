"""Shared helpers of the GPU parity tests: device upload, tolerances, comparisons.

Tolerances: for bf16 inputs with fp32 accumulation the output must be within
max-abs 2e-2 and mean-abs 2e-3 of the float64 oracle, and in addition within 1e-2
of max|oracle| (a bar that stays meaningful where outputs are small); for fp32
inputs within max-abs 1e-4. Selected block indices must equal the oracle's
except in rows whose oracle fp32 score gap between the K-th and (K+1)-th block is
below 1e-3 * max|score| (a near tie), where the device set must still be a valid
top-K within that gap. In such a row the output is compared with the oracle's
output for the device's (valid) set, so every row of every sampled block is
compared element by element; the number of such rows is reported.
"""

from __future__ import annotations

import numpy as np
import torch

import oracle

BF16_MAX_ABS = 2e-2
BF16_MEAN_ABS = 2e-3
BF16_REL = 1e-2
F32_MAX_ABS = 1e-4


def dev_bf16(bits: np.ndarray, device="cuda") -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16))
    return t.view(torch.bfloat16).to(device)


def dev_f32(x: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(device)


def host_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def compare_sel(sel_dev: np.ndarray, sel_ref: np.ndarray, s32_ref: np.ndarray, top_k: int):
    """Check the device selection; returns the bool [H][Nqb] mask of rows that differ."""
    assert sel_dev.shape == sel_ref.shape, (sel_dev.shape, sel_ref.shape)
    assert np.all(np.diff(sel_dev, axis=-1) > 0), "selection rows must be strictly ascending"
    differ = (sel_dev != sel_ref).any(-1)
    exempt = oracle.near_tie_rows(s32_ref, top_k)
    bad = differ & ~exempt
    assert not bad.any(), f"{int(bad.sum())} non-exempt rows differ, e.g. {np.argwhere(bad)[:4]}"
    if differ.any():
        hs, is_ = np.nonzero(differ)
        for h, i in zip(hs, is_):
            assert oracle.valid_top_k(s32_ref[h:h + 1, i:i + 1], sel_dev[h:h + 1, i:i + 1])
    return differ


def compare_out(out_dev: np.ndarray, out_ref: np.ndarray, dtype: str, rows_mask=None):
    """Element-wise comparison where out_ref is finite (NaN marks rows not computed)."""
    m = np.isfinite(out_ref)
    if rows_mask is not None:
        m &= rows_mask
    assert m.any()
    d = np.abs(out_dev[m] - out_ref[m])
    stats = dict(max_abs=float(d.max()), mean_abs=float(d.mean()),
                 rel=float(d.max() / max(np.abs(out_ref[m]).max(), 1e-30)), n=int(m.sum()))
    if dtype == "f32":
        assert stats["max_abs"] <= F32_MAX_ABS, stats
    else:
        assert stats["max_abs"] <= BF16_MAX_ABS, stats
        assert stats["mean_abs"] <= BF16_MEAN_ABS, stats
        assert stats["rel"] <= BF16_REL, stats
    return stats


def reference_selection(sel_dev: np.ndarray, sel_ref: np.ndarray, differ: np.ndarray):
    """The selection the oracle's outputs are computed for: the oracle's own, except in
    the near-tie rows where compare_sel accepted a different valid top-K set of the
    device; there the oracle attends over the device's set, so those rows' outputs
    are compared too rather than skipped."""
    return np.where(differ[..., None], sel_dev, sel_ref).astype(np.int32)


def state_close(S_dev, z_dev, S_ref, z_ref, dtype: str):
    """Linear state vs the float64 batch state."""
    fro = np.linalg.norm((S_dev - S_ref).ravel()) / max(np.linalg.norm(S_ref.ravel()), 1e-30)
    zrel = np.abs(z_dev - z_ref).max() / max(np.abs(z_ref).max(), 1e-30)
    lim_s, lim_z = (1e-3, 1e-5) if dtype == "bf16" else (1e-6, 1e-6)
    assert fro <= lim_s and zrel <= lim_z, dict(fro=fro, zrel=zrel)
    return fro, zrel
