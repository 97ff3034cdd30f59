"""Float64 CPU oracle of Hybrid Forcing's per-chunk hybrid attention.

TEST INFRASTRUCTURE ONLY. This module is the slow, plain reference that the HIP
path is checked against. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it; the library and its Python
binding never do, and it shares no code with them (it reads only NumPy and the
seeded inputs). Everything is computed in float64 on the exact input values
(bf16 or fp32 values widened to float64), one head and one query block at a time,
with no blocking, fusion or reordering beyond what the definitions state.

Sources (the pages):
  [EN]  gist.science English summary of arXiv 2604.10103, "Long-Horizon Streaming
        Video Generation via Hybrid Attention with Decoupled Distillation".
  [ES]  gist.science Spanish summary of the same paper, "Resumen Tecnico: Hybrid
        Forcing".
  [ABS] the authors' abstract on the fugumt.com listing of arXiv 2604.10103v1.

What the pages fix: a compact key-value state that incrementally absorbs the
tokens evicted from the sliding window ([ABS]; [EN] 2.A.1 "Linear Temporal
Attention"; [ES] 2.A.1), read at a cost independent of the video length
([EN] 2.A.1); block-sparse attention inside the sliding window that keeps the
top-K blocks by a block importance score ([EN] 2.A.2 "Block-Sparse Sliding Window
Attention"); the output is the sum of the two paths ([ES] 2.A.2, last bullet).

Readings where the pages are silent (each one is an assumption, not a fact of
the pages):
  * feature map phi = elu + 1 (phi(x) = x + 1 for x > 0, exp(x) otherwise), the
    kernelised linear attention of Katharopoulos et al. (ICML 2020);
  * linear read  o_lin = S phi(q) / (z . phi(q) + eps), eps = 1e-6, where the
    state is S = sum_n v_n phi(k_n)^T (value-major, d_v x d_k) and
    z = sum_n phi(k_n);
  * the two paths are added unweighted, each with its own normalisation;
  * softmax scale tau = 1/sqrt(d), also in the block score;
  * block importance = tau * (mean of the query block's rows) . (mean of the key
    block's rows), means over the block's actual rows;
  * query blocks tile the chunk's rows from row 0 and key blocks tile the
    window's rows from row 0, each with a ragged last block;
  * the window includes the current chunk; no causal or intra-chunk mask;
  * top-K keeps the K largest scores, ties going to the lower key-block index;
    the kept list is returned in ascending order. The selection is an integer
    decision taken on fp32 scores (the device kernels' precision): the score is
    computed in float64 and rounded once to fp32 before ranking;
  * a key row takes part in a query row's softmax iff its block is selected for
    that query row's block (no forced sink, diagonal or current-frame blocks).

Parity pins: see tests/test_oracle_pins.py (closed forms, invariants, brute force
on tiny inputs, library special cases). Nothing in this module is "parity
unpinned" except the readings listed above, which the pages do not fix.
"""

from __future__ import annotations

import math
from typing import Iterable, Optional, Sequence, Tuple

import numpy as np

DEFAULT_EPS = 1e-6


# ------------------------------------------------------------------ feature map


def phi(x: np.ndarray) -> np.ndarray:
    """elu(x) + 1 in float64: x + 1 for x > 0, exp(x) for x <= 0."""
    x = np.asarray(x, dtype=np.float64)
    return np.where(x > 0, x + 1.0, np.exp(np.minimum(x, 0.0)))


# ------------------------------------------------------------- linear KV state
# [ABS]; [EN] 2.A.1 "Linear Temporal Attention" (state incrementally aggregates the
# evicted frames); [ES] 2.A.1 (an evicted frame's information is compressed into
# the linear state).


def state_init(heads: int, dim: int) -> Tuple[np.ndarray, np.ndarray]:
    """Empty state: S = 0 (H x d x d, value-major), z = 0 (H x d)."""
    return np.zeros((heads, dim, dim), np.float64), np.zeros((heads, dim), np.float64)


def absorb(S: np.ndarray, z: np.ndarray, k_ev: np.ndarray, v_ev: np.ndarray) -> None:
    """Fold evicted tokens into the state, in place.

    S[h] += V_ev[h]^T phi(K_ev[h])   (S[h][j][i] += sum_n V[n][j] phi(K[n][i]))
    z[h] += sum_n phi(K_ev[h][n])
    """
    k_ev = np.asarray(k_ev, np.float64)
    v_ev = np.asarray(v_ev, np.float64)
    for h in range(S.shape[0]):
        f = phi(k_ev[h])
        S[h] += v_ev[h].T @ f
        z[h] += f.sum(axis=0)


# ------------------------------------------------------------- block structure


def block_ranges(n_rows: int, block: int) -> list:
    """Contiguous blocks of `block` rows from row 0; the last one may be ragged."""
    return [(s, min(s + block, n_rows)) for s in range(0, n_rows, block)]


def block_means(x: np.ndarray, block: int) -> np.ndarray:
    """Row mean of every block of one head's [N][d] matrix -> [nblocks][d] (float64)."""
    x = np.asarray(x, np.float64)
    return np.stack([x[s:e].mean(axis=0) for s, e in block_ranges(x.shape[0], block)])


# ------------------------------------------------------------- block selection
# [EN] 2.A.2 "Block-Sparse Sliding Window Attention": block importance scores, keep
# the top-K most informative blocks.


def block_scores(q: np.ndarray, k_win: np.ndarray, block: int,
                 scale: Optional[float] = None) -> np.ndarray:
    """Pooled block logits s[h][i][j] = tau * mean(Q block i) . mean(K block j), float64."""
    H, _, d = q.shape
    tau = 1.0 / math.sqrt(d) if scale is None else scale
    out = []
    for h in range(H):
        qm = block_means(q[h], block)
        km = block_means(k_win[h], block)
        out.append(tau * (qm @ km.T))
    return np.stack(out)


def select_from_scores(scores32: np.ndarray, top_k: int) -> np.ndarray:
    """Top-K key blocks per (head, query block) by (score desc, index asc), ascending."""
    H, nqb, nkb = scores32.shape
    if not 1 <= top_k <= nkb:
        raise ValueError("top_k out of range")
    sel = np.zeros((H, nqb, top_k), np.int32)
    for h in range(H):
        for i in range(nqb):
            s = scores32[h, i].astype(np.float64)  # exact widening of the fp32 values
            order = sorted(range(nkb), key=lambda j: (-s[j], j))
            sel[h, i] = np.sort(np.array(order[:top_k], np.int32))
    return sel


def select(q: np.ndarray, k_win: np.ndarray, block: int, top_k: int,
           scale: Optional[float] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Returns (sel [H][Nqb][K] int32 ascending, fp32 scores [H][Nqb][Nkb])."""
    s32 = block_scores(q, k_win, block, scale).astype(np.float32)
    s32[s32 == 0] = 0.0  # -0.0 and +0.0 are the same score
    return select_from_scores(s32, top_k), s32


def near_tie_rows(scores32: np.ndarray, top_k: int, rel: float = 1e-3) -> np.ndarray:
    """Rows whose K-th and (K+1)-th largest scores differ by < rel * max|s| -> bool [H][Nqb]."""
    H, nqb, nkb = scores32.shape
    out = np.zeros((H, nqb), bool)
    if top_k >= nkb:
        return out
    s = np.sort(scores32.astype(np.float64), axis=-1)[..., ::-1]
    gap = s[..., top_k - 1] - s[..., top_k]
    return gap < rel * np.abs(scores32.astype(np.float64)).max(axis=-1)


def valid_top_k(scores32: np.ndarray, sel: np.ndarray, rel: float = 1e-3) -> bool:
    """True iff each row of `sel` is a top-K set of its row up to rel * max|s|."""
    H, nqb, nkb = scores32.shape
    s = scores32.astype(np.float64)
    for h in range(H):
        for i in range(nqb):
            row = sel[h, i]
            if len(set(row.tolist())) != len(row) or row.min() < 0 or row.max() >= nkb:
                return False
            mask = np.zeros(nkb, bool)
            mask[row] = True
            tol = rel * np.abs(s[h, i]).max()
            if (~mask).any() and s[h, i][mask].min() < s[h, i][~mask].max() - tol:
                return False
    return True


# ------------------------------------------------------------------- attention
# Sparse path: [EN] 2.A.2; sum of the paths: [ES] 2.A.2; linear read: [EN] 2.A.1.


def linear_read(q: np.ndarray, S: np.ndarray, z: np.ndarray, eps: float = DEFAULT_EPS) -> np.ndarray:
    """Read of one head's linear state for query rows q [n][d] ([EN] 2.A.1):
    S phi(q_r) / (z . phi(q_r) + eps), float64."""
    fq = phi(np.asarray(q, np.float64))
    return (fq @ S.T) / (fq @ z + eps)[:, None]


def attend_with_sel(q: np.ndarray, k_win: np.ndarray, v_win: np.ndarray, sel: np.ndarray,
                    S: np.ndarray, z: np.ndarray, block: int, eps: float = DEFAULT_EPS,
                    scale: Optional[float] = None,
                    blocks: Optional[Iterable[Tuple[int, int]]] = None,
                    return_parts: bool = False):
    """Hybrid attention output for a given key-block selection, float64.

    For every query row r of query block i of head h:
      T        = rows of the window blocks in sel[h][i]
      o_swa[r] = sum_{t in T} softmax_t(tau q_r . k_t) v_t
      o_lin[r] = S[h] phi(q_r) / (z[h] . phi(q_r) + eps)
      out[r]   = o_swa[r] + o_lin[r]
    `blocks` limits the work to the listed (h, i) pairs; other rows are NaN.
    """
    q = np.asarray(q, np.float64)
    k_win = np.asarray(k_win, np.float64)
    v_win = np.asarray(v_win, np.float64)
    H, n_q, d = q.shape
    n_kv = k_win.shape[1]
    tau = 1.0 / math.sqrt(d) if scale is None else scale
    qb = block_ranges(n_q, block)
    kb = block_ranges(n_kv, block)
    if blocks is None:
        blocks = [(h, i) for h in range(H) for i in range(len(qb))]
    o_swa = np.full(q.shape, np.nan)
    o_lin = np.full(q.shape, np.nan)
    for h, i in blocks:
        s0, s1 = qb[i]
        rows = np.concatenate([np.arange(*kb[j]) for j in sel[h][i]])
        qi = q[h, s0:s1]
        logits = tau * (qi @ k_win[h, rows].T)
        logits -= logits.max(axis=1, keepdims=True)
        p = np.exp(logits)
        p /= p.sum(axis=1, keepdims=True)
        o_swa[h, s0:s1] = p @ v_win[h, rows]
        o_lin[h, s0:s1] = linear_read(qi, S[h], z[h], eps)
    out = o_swa + o_lin
    if return_parts:
        return out, o_swa, o_lin
    return out


def attend(q, k_win, v_win, S, z, block: int, top_k: int, eps: float = DEFAULT_EPS,
           scale: Optional[float] = None, blocks=None):
    """Select, then attend. Returns (out, sel, fp32 scores)."""
    sel, s32 = select(q, k_win, block, top_k, scale)
    out = attend_with_sel(q, k_win, v_win, sel, S, z, block, eps, scale, blocks)
    return out, sel, s32


# ----------------------------------------------------- relative temporal RoPE
# [EN] 2.C "Stability Enhancements" (Relative RoPE Constraint) and [ES] 2.C: the
# temporal rotary position indices are kept below a fixed bound in training and in
# inference, positions being relative offsets. The pages give neither the rotated
# features, the frequencies nor the bound; the readings taken here:
#   * the standard rotary form: the first rot_dims features of a query or key vector
#     rotate in adjacent pairs (2i, 2i+1), pair i by the angle p * base^(-2i/rot_dims)
#     for position p; the other features (spatial position, applied upstream) stay;
#   * the position of a window token is its frame's offset from the window's first
#     frame, capped: p = min(row // tokens_per_frame, cap); the queries are the
#     window's last rows (the current chunk);
#   * the rotation applies to the softmax path (block scores and sparse attention);
#     the linear state absorbs and reads position-free (unrotated) features.


def rope_positions(n_rows: int, tokens_per_frame: int, cap: int, row0: int = 0) -> np.ndarray:
    """Temporal positions of window rows row0 .. row0 + n_rows - 1: min(frame, cap),
    frames counted from the window's first row."""
    rows = np.arange(row0, row0 + n_rows, dtype=np.int64)
    return np.minimum(rows // tokens_per_frame, cap)


def rope_rotate(x: np.ndarray, pos: np.ndarray, rot_dims: int, theta_base: float) -> np.ndarray:
    """Rotate the first rot_dims features of every row of x [H][n][d] in pairs
    (2i, 2i+1) by pos[n] * theta_base^(-2i/rot_dims), float64."""
    x = np.array(x, dtype=np.float64, copy=True)
    if rot_dims == 0:
        return x
    i = np.arange(rot_dims // 2, dtype=np.float64)
    ang = np.asarray(pos, np.float64)[:, None] * theta_base ** (-2.0 * i / rot_dims)[None, :]
    c, s = np.cos(ang), np.sin(ang)
    a = x[..., 0:rot_dims:2].copy()
    b = x[..., 1:rot_dims:2].copy()
    x[..., 0:rot_dims:2] = a * c - b * s
    x[..., 1:rot_dims:2] = a * s + b * c
    return x


def attend_rope(q, k_win, v_win, S, z, block: int, top_k: int, tokens_per_frame: int, cap: int,
                rot_dims: int, theta_base: float, eps: float = DEFAULT_EPS,
                scale: Optional[float] = None, blocks=None):
    """Hybrid attention with the relative temporal rotation on the softmax path.
    The window [H][n_kv][d] starts on a frame boundary; q holds its last n_q rows.
    Returns (out, sel, fp32 scores)."""
    n_q, n_kv = q.shape[1], k_win.shape[1]
    qr = rope_rotate(q, rope_positions(n_q, tokens_per_frame, cap, n_kv - n_q), rot_dims,
                     theta_base)
    kr = rope_rotate(k_win, rope_positions(n_kv, tokens_per_frame, cap), rot_dims, theta_base)
    sel, s32 = select(qr, kr, block, top_k, scale)
    _, o_swa, _ = attend_with_sel(qr, kr, v_win, sel, S, z, block, eps, scale, blocks,
                                  return_parts=True)
    o_lin = np.full(o_swa.shape, np.nan)
    rows = np.isfinite(o_swa[..., 0])
    q = np.asarray(q, np.float64)
    for h in range(q.shape[0]):
        o_lin[h, rows[h]] = linear_read(q[h, rows[h]], S[h], z[h], eps)
    return o_swa + o_lin, sel, s32


# --------------------------------------------------- head-aware ragged windows
# Related work on the pages ("Resumen Tecnico: Pyramid Forcing", 3 "Optimizacion de
# Calculo de Cache KV Heterogenea"): heads keep KV caches of different lengths,
# stored as flattened sequences with boundary indices, and attention runs over them
# without padding. Here each head runs the hybrid attention above over its own
# window; nothing else changes.


def attend_ragged(q, k_flat, v_flat, offsets, S, z, block: int, top_ks,
                  eps: float = DEFAULT_EPS, scale: Optional[float] = None, blocks=None):
    """Head h attends the window rows k_flat[offsets[h]:offsets[h+1]] (and v_flat's)
    with its own top_ks[h]. Returns (out [H][n_q][d], list of per-head selections
    [Nqb][K_h], list of per-head fp32 scores [Nqb][Nkb_h])."""
    q = np.asarray(q, np.float64)
    H = q.shape[0]
    out = np.full(q.shape, np.nan)
    sels, scores = [], []
    for h in range(H):
        o0, o1 = int(offsets[h]), int(offsets[h + 1])
        hb = None if blocks is None else [(0, i) for hh, i in blocks if hh == h]
        if hb == []:
            sel, s32 = select(q[h:h + 1], np.asarray(k_flat, np.float64)[None, o0:o1], block,
                              top_ks[h], scale)
        else:
            o, sel, s32 = attend(q[h:h + 1], np.asarray(k_flat, np.float64)[None, o0:o1],
                                 np.asarray(v_flat, np.float64)[None, o0:o1], S[h:h + 1],
                                 z[h:h + 1], block, top_ks[h], eps, scale, hb)
            out[h] = o[0]
        sels.append(sel[0])
        scores.append(s32[0])
    return out, sels, scores


# --------------------------------------------------------------- stream order
# [EN] 1 "Problem Statement" and [ES] 1: the window slides and the oldest frames
# leave the cache; [ABS]: evicted tokens are absorbed into the state.


def stream_step_frames(t: int, chunk: int, window: int) -> Tuple[Tuple[int, int], Tuple[int, int]]:
    """Frames handled at chunk step t: (newly evicted [lo, hi), window [lo, hi)).

    Chunk t holds frames [c t, c t + c). The window before attending chunk t is
    the last W frames up to and including the chunk; frames that fell out of it
    since step t-1 are absorbed first.
    """
    hi = chunk * t + chunk
    win_lo = max(0, hi - window)
    ev_lo = max(0, chunk * (t - 1) + chunk - window) if t > 0 else 0
    return (ev_lo, win_lo), (win_lo, hi)


def as_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    """Input values as float64: bf16 bit patterns (uint16) or fp32 arrays."""
    if dtype == "bf16":
        b = np.ascontiguousarray(x, dtype=np.uint16)
        return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return np.asarray(x, np.float32).astype(np.float64)
