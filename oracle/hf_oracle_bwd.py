"""Float64 CPU oracle of the backward pass of the per-chunk hybrid attention.

TEST INFRASTRUCTURE ONLY, like hf_oracle (same rules: only tests/, smoke() and
bench.py's cpu_baseline use it; it shares no code with the HIP path).

The pages train through this path (Hybrid Forcing's decoupled distillation,
[EN] 2.B-C; the state is called learnable in [EN] 2.A.1), but give no formula for
its gradients. This module differentiates the forward definition of hf_oracle
exactly, with the key-block selection held fixed (the selection is a discrete
choice with no gradient):

  forward (per head, query row r of block i, T_i = rows of the selected blocks)
    p_r      = softmax_t(tau q_r . k_t), t in T_i
    out_r    = sum_t p_rt v_t + S phi(q_r) / (z . phi(q_r) + eps)
  loss       L = sum_r dout_r . out_r   (dout is the incoming gradient)

  softmax path:  dv_t += p_rt dout_r;  dp_rt = dout_r . v_t;
                 dl_rt = p_rt (dp_rt - sum_u p_ru dp_ru);
                 dq_r += tau sum_t dl_rt k_t;  dk_t += tau dl_rt q_r
  linear read:   f = phi(q_r), den = z . f + eps, o_lin = S f / den,
                 g = dout_r / den, c = -(dout_r . o_lin) / den;
                 dS += g f^T, dz += c f, dq_r += (S^T g + c z) * phi'(q_r)
  absorb:        S = S0 + sum_n v_n phi(k_n)^T, z = z0 + sum_n phi(k_n), so
                 dv_n = dS phi(k_n), dk_n = phi'(k_n) * (dS^T v_n + dz)

with phi'(x) = 1 for x > 0 and exp(x) otherwise (phi is continuously
differentiable at 0). Pins: tests/test_oracle_bwd_pins.py (central finite
differences of the pinned forward oracle, invariants of softmax).
"""

from __future__ import annotations

import math
from typing import Optional, Tuple

import numpy as np

from .hf_oracle import DEFAULT_EPS, block_ranges, phi


def phi_prime(x: np.ndarray) -> np.ndarray:
    """Derivative of phi = elu + 1: 1 for x > 0, exp(x) otherwise."""
    x = np.asarray(x, np.float64)
    return np.where(x > 0, 1.0, np.exp(np.minimum(x, 0.0)))


def attend_with_sel_backward(q: np.ndarray, k_win: np.ndarray, v_win: np.ndarray,
                             sel: np.ndarray, S: np.ndarray, z: np.ndarray, dout: np.ndarray,
                             block: int, eps: float = DEFAULT_EPS,
                             scale: Optional[float] = None
                             ) -> Tuple[np.ndarray, np.ndarray, np.ndarray, np.ndarray,
                                        np.ndarray]:
    """(dq, dk_win, dv_win, dS, dz) of L = sum(dout * out), out = hf_oracle.attend_with_sel
    with the same arguments; the selection is held fixed. float64."""
    q = np.asarray(q, np.float64)
    k_win = np.asarray(k_win, np.float64)
    v_win = np.asarray(v_win, np.float64)
    dout = np.asarray(dout, np.float64)
    S = np.asarray(S, np.float64)
    z = np.asarray(z, np.float64)
    H, n_q, d = q.shape
    n_kv = k_win.shape[1]
    tau = 1.0 / math.sqrt(d) if scale is None else scale
    qb = block_ranges(n_q, block)
    kb = block_ranges(n_kv, block)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k_win)
    dv = np.zeros_like(v_win)
    dS = np.zeros_like(S)
    dz = np.zeros_like(z)
    for h in range(H):
        for i, (s0, s1) in enumerate(qb):
            rows = np.concatenate([np.arange(*kb[j]) for j in sel[h][i]])  # distinct rows
            qi, doi = q[h, s0:s1], dout[h, s0:s1]
            kt, vt = k_win[h, rows], v_win[h, rows]
            # softmax path
            logits = tau * (qi @ kt.T)
            logits -= logits.max(axis=1, keepdims=True)
            p = np.exp(logits)
            p /= p.sum(axis=1, keepdims=True)
            dv[h, rows] += p.T @ doi
            dp = doi @ vt.T
            dl = p * (dp - (p * dp).sum(axis=1, keepdims=True))
            dq[h, s0:s1] += tau * (dl @ kt)
            dk[h, rows] += tau * (dl.T @ qi)
            # linear read
            f = phi(qi)
            den = f @ z[h] + eps
            o_lin = (f @ S[h].T) / den[:, None]
            g = doi / den[:, None]
            c = -(doi * o_lin).sum(axis=1) / den
            dS[h] += g.T @ f
            dz[h] += c @ f
            dq[h, s0:s1] += (g @ S[h] + c[:, None] * z[h][None, :]) * phi_prime(qi)
    return dq, dk, dv, dS, dz


def absorb_backward(k_ev: np.ndarray, v_ev: np.ndarray, dS: np.ndarray,
                    dz: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """(dk_ev, dv_ev) of L = sum(dS * S) + sum(dz * z) where S and z are the state after
    hf_oracle.absorb(S0, z0, k_ev, v_ev) (S0, z0 do not depend on k_ev, v_ev). float64."""
    k_ev = np.asarray(k_ev, np.float64)
    v_ev = np.asarray(v_ev, np.float64)
    dS = np.asarray(dS, np.float64)
    dz = np.asarray(dz, np.float64)
    dk = np.empty_like(k_ev)
    dv = np.empty_like(v_ev)
    for h in range(k_ev.shape[0]):
        f = phi(k_ev[h])
        dv[h] = f @ dS[h].T
        dk[h] = phi_prime(k_ev[h]) * (v_ev[h] @ dS[h] + dz[h][None, :])
    return dk, dv
