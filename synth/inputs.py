"""Seeded synthetic Q/K/V for the hybrid-attention workloads.

Every array is drawn from NumPy's PCG64 generator seeded with
``SeedSequence([seed, stream, frame])``, so any frame of any stream can be
regenerated on its own. Values are drawn in fp32; bf16 workloads are then rounded
to bfloat16 with round-to-nearest-even and handed out as raw 16-bit patterns
(``uint16``), which both the oracle (widened to float64) and the device path
(viewed as bfloat16) read bit for bit.

The shapes stand in for one attention layer of a Wan2.1-1.3B-like video
transformer at 832x480 (the model and resolution named in the authors' abstract
on the fugumt.com listing of arXiv 2604.10103v1). The head count, head size and
tokens per latent frame are assumptions: 12 heads, d = 128, and
1560 = (480/8/2) * (832/8/2) tokens per latent frame (8x VAE, 2x2 patches).
No dataset or trained weight is used or needed.
"""

from __future__ import annotations

import math
from dataclasses import dataclass
from typing import Optional

import numpy as np

# Stream identifiers mixed into the seed sequence.
STREAM_Q = 1
STREAM_K = 2
STREAM_V = 3
STREAM_DRIFT = 4
STREAM_PLANT = 5


# --------------------------------------------------------------------------- bf16


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bfloat16 (round-to-nearest-even); return the bit patterns."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    bias = ((u >> 16) & 1) + 0x7FFF
    out = ((u + bias) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():  # keep NaN a (quiet) NaN instead of rounding it into infinity
        out[nan] = ((u[nan] >> 16) | 0x40).astype(np.uint16)
    return out


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to the fp32 values they encode (exact)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """fp32 -> nearest bfloat16 value, returned as fp32."""
    return bf16_bits_to_f32(bf16_bits(x))


# ---------------------------------------------------------------------- workloads


@dataclass(frozen=True)
class Workload:
    name: str
    heads: int
    head_dim: int
    frame_tokens: int
    chunk_frames: int
    window_frames: int
    block: int
    dtype: str  # "bf16" or "f32": element type of Q, K, V and the output
    top_k: Optional[int] = None  # fixed number of key blocks per query block ...
    top_k_frac: Optional[float] = None  # ... or a fraction of the window's key blocks
    eps: float = 1e-6
    input_scale_by_sqrt_d: bool = True  # draw N(0,1)/sqrt(d) instead of N(0,1)
    n_frames: int = 12
    drift_std: float = 0.0  # per-frame random-walk step of K's mean (long stream)
    layers: int = 1

    @property
    def chunk_tokens(self) -> int:
        return self.chunk_frames * self.frame_tokens

    @property
    def window_tokens(self) -> int:
        return self.window_frames * self.frame_tokens

    @property
    def input_std(self) -> float:
        return 1.0 / math.sqrt(self.head_dim) if self.input_scale_by_sqrt_d else 1.0


WORKLOADS = {
    # 1 head, d = 64, 64 tokens/frame, 6 frames in 2-frame chunks, window 2 frames,
    # blocks of 16 tokens, 2 key blocks per query block, fp32 N(0,1).
    "tiny_f32": Workload(
        "tiny_f32", heads=1, head_dim=64, frame_tokens=64, chunk_frames=2,
        window_frames=2, block=16, dtype="f32", top_k=2,
        input_scale_by_sqrt_d=False, n_frames=6),
    # One Wan-1.3B-like layer: 12 heads, d = 128, 1560 tokens/frame, 3-frame chunk,
    # 9-frame window, 64-token blocks, top-K = 25% of window blocks, bf16.
    "wan_layer_bf16": Workload(
        "wan_layer_bf16", heads=12, head_dim=128, frame_tokens=1560, chunk_frames=3,
        window_frames=9, block=64, dtype="bf16", top_k_frac=0.25, n_frames=12),
    # 60 chunk steps (180 latent frames) on the same per-layer shapes, with a slow
    # random-walk drift of K's mean per frame.
    "long_stream_bf16": Workload(
        "long_stream_bf16", heads=12, head_dim=128, frame_tokens=1560, chunk_frames=3,
        window_frames=9, block=64, dtype="bf16", top_k_frac=0.25, n_frames=180,
        drift_std=0.05),
    # Planted block structure on the same shapes; the fraction is swept by the caller.
    "planted_bf16": Workload(
        "planted_bf16", heads=12, head_dim=128, frame_tokens=1560, chunk_frames=3,
        window_frames=9, block=64, dtype="bf16", top_k_frac=0.25, n_frames=12),
    # The Wan-1.3B-like layer with per-head window lengths (RAGGED_WINDOW_FRAMES), the
    # windows stored flattened one after the other with boundary indices.
    "ragged_heads_bf16": Workload(
        "ragged_heads_bf16", heads=12, head_dim=128, frame_tokens=1560, chunk_frames=3,
        window_frames=9, block=64, dtype="bf16", top_k_frac=0.25, n_frames=12),
    # 30 independent layers of the Wan-1.3B-like shapes per 3-frame chunk.
    "full_depth_bf16": Workload(
        "full_depth_bf16", heads=12, head_dim=128, frame_tokens=1560, chunk_frames=3,
        window_frames=9, block=64, dtype="bf16", top_k_frac=0.25, n_frames=12,
        layers=30),
}

# Head-aware ragged windows: window length of each head in latent frames (the
# current 3-frame chunk included), a pyramid of three head classes of four heads each
# standing in for per-head cache policies that keep more or less history.
RAGGED_WINDOW_FRAMES = (9, 9, 9, 9, 6, 6, 6, 6, 4, 4, 4, 4)

PLANTED_FRACTIONS = (0.125, 0.25, 0.5, 1.0)
PLANTED_LOGIT_BIAS = 2.0


def top_k_count(frac: float, n_blocks: int) -> int:
    """Workload parameter: ceil(frac * n_blocks), clamped to [1, n_blocks]."""
    return int(min(max(math.ceil(frac * n_blocks - 1e-9), 1), n_blocks))


def _rng(seed: int, stream: int, frame: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, stream, frame])))


def frame_block(seed: int, stream: int, frame: int, heads: int, tokens: int, dim: int,
                std: float) -> np.ndarray:
    """One latent frame of one stream: fp32 [heads][tokens][dim] ~ N(0, std^2)."""
    x = _rng(seed, stream, frame).standard_normal((heads, tokens, dim), dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


def _frames(seed, stream, lo, hi, wl: Workload) -> np.ndarray:
    parts = [frame_block(seed, stream, f, wl.heads, wl.frame_tokens, wl.head_dim, wl.input_std)
             for f in range(lo, hi)]
    if not parts:
        return np.zeros((wl.heads, 0, wl.head_dim), np.float32)
    return np.concatenate(parts, axis=1)


# ------------------------------------------------------------------ tiny fp32 case


def tiny_f32_frames(seed: int):
    """The tiny fp32 case: Q, K, V fp32 [1][6*64][64] ~ N(0,1), all 6 frames."""
    wl = WORKLOADS["tiny_f32"]
    q = _frames(seed, STREAM_Q, 0, wl.n_frames, wl)
    k = _frames(seed, STREAM_K, 0, wl.n_frames, wl)
    v = _frames(seed, STREAM_V, 0, wl.n_frames, wl)
    return q, k, v


# ------------------------------------------------------------ one Wan-like layer


def wan_layer_inputs(seed: int, wl: Workload = WORKLOADS["wan_layer_bf16"], *,
                     as_f32: bool = False):
    """One layer at stream step 3 of a 3-frame-chunk / 9-frame-window stream.

    K and V cover latent frames 0..11; frames 0..2 have been evicted (absorbed
    into the linear state) and frames 3..11 form the window. Q is the current
    chunk (frames 9..11). Returns bf16 bit patterns (or the fp32 values before
    rounding when ``as_f32``) and the token offsets of the evicted span and the
    window inside the K/V buffers.
    """
    c, w = wl.chunk_frames, wl.window_frames
    t = 3
    hi = c * t + c
    win_lo = max(0, hi - w)
    q = _frames(seed, STREAM_Q, hi - c, hi, wl)
    k = _frames(seed, STREAM_K, 0, hi, wl)
    v = _frames(seed, STREAM_V, 0, hi, wl)
    out = dict(ev_lo=0, ev_hi=win_lo * wl.frame_tokens, win_lo=win_lo * wl.frame_tokens,
               win_hi=hi * wl.frame_tokens)
    if as_f32:
        out.update(q=q, k=k, v=v)
    else:
        out.update(q=bf16_bits(q), k=bf16_bits(k), v=bf16_bits(v))
    return out


# ------------------------------------------------------------ ragged head windows


def ragged_layer_inputs(seed: int, window_frames=RAGGED_WINDOW_FRAMES,
                        wl: Workload = WORKLOADS["ragged_heads_bf16"]):
    """The Wan-like layer at stream step 3 where head h keeps the last window_frames[h]
    frames of frames 0..11 (the chunk, frames 9..11, included): K and V of all heads'
    windows flattened one after the other ([sum_h n_h][d] bf16 bits, head h's rows at
    offsets[h] .. offsets[h + 1]), Q of the chunk ([H][3T][d]) and the evicted frames
    0..2 of every head (for the state; [H][3T][d])."""
    base = wan_layer_inputs(seed, wl)
    T, hi = wl.frame_tokens, base["win_hi"]
    offsets = np.zeros(wl.heads + 1, np.int64)
    for h, f in enumerate(window_frames):
        offsets[h + 1] = offsets[h] + f * T
    parts_k = [base["k"][h, hi - f * T:hi] for h, f in enumerate(window_frames)]
    parts_v = [base["v"][h, hi - f * T:hi] for h, f in enumerate(window_frames)]
    return dict(q=base["q"], k_flat=np.concatenate(parts_k), v_flat=np.concatenate(parts_v),
                offsets=offsets, k_ev=base["k"][:, :base["ev_hi"]],
                v_ev=base["v"][:, :base["ev_hi"]])


# --------------------------------------------------------------- planted structure


def planted_inputs(seed: int, frac: float, wl: Workload = WORKLOADS["planted_bf16"]):
    """Wan-like layer with a planted set of key blocks per query block.

    For each head, every query block i gets a random set P_i of K window blocks
    (K = top_k_count(frac, Nkb)). With orthonormal e_0..e_{Nqb-1} in R^d, every
    Q row of block i gets + a*e_i and every K row of window block j gets
    + b*sum_{i : j in P_i} e_i, with a*b/sqrt(d) = PLANTED_LOGIT_BIAS, so the
    pooled block logit of (i, j) rises by that bias exactly when j is in P_i.
    The structure is added in fp32 before the bf16 rounding.
    """
    base = wan_layer_inputs(seed, wl, as_f32=True)
    q, k, v = base["q"], base["k"], base["v"]
    H, d, B = wl.heads, wl.head_dim, wl.block
    n_q = q.shape[1]
    win_lo, win_hi = base["win_lo"], base["win_hi"]
    n_kv = win_hi - win_lo
    nqb = -(-n_q // B)
    nkb = -(-n_kv // B)
    if nqb > d:
        raise ValueError("planted structure needs one orthonormal direction per query block")
    kk = top_k_count(frac, nkb)
    amp = math.sqrt(PLANTED_LOGIT_BIAS * math.sqrt(d))  # a = b, a*b/sqrt(d) = bias
    rng = _rng(seed, STREAM_PLANT, int(round(frac * 1000)))
    sets = np.zeros((H, nqb, kk), np.int32)
    for h in range(H):
        g = rng.standard_normal((d, nqb))
        e, _ = np.linalg.qr(g)  # d x nqb, orthonormal columns
        e = e.T.astype(np.float64)  # nqb x d
        kadd = np.zeros((nkb, d), np.float64)
        for i in range(nqb):
            p = np.sort(rng.choice(nkb, size=kk, replace=False)).astype(np.int32)
            sets[h, i] = p
            q[h, i * B:min((i + 1) * B, n_q)] += np.float32(amp) * e[i].astype(np.float32)
            kadd[p] += e[i]
        kadd = (amp * kadd).astype(np.float32)
        for j in range(nkb):
            lo = win_lo + j * B
            hi = min(win_lo + (j + 1) * B, win_hi)
            k[h, lo:hi] += kadd[j]
    return dict(q=bf16_bits(q), k=bf16_bits(k), v=bf16_bits(v), ev_lo=base["ev_lo"],
                ev_hi=base["ev_hi"], win_lo=win_lo, win_hi=win_hi, top_k=kk, planted=sets)


# ----------------------------------------------------------------- long stream


class LongStream:
    """Per-frame generator of the long stream: 180 latent frames, drifting K mean.

    K_f = N(0,1)/sqrt(d) + m_f with m_0 = 0 and m_f = m_{f-1} + N(0, drift_std^2)
    per (head, dim), added in fp32 before the bf16 rounding; Q and V do not drift.
    """

    def __init__(self, seed: int, wl: Workload = WORKLOADS["long_stream_bf16"]):
        self.seed = seed
        self.wl = wl
        steps = _rng(seed, STREAM_DRIFT, 0).standard_normal(
            (wl.n_frames, wl.heads, wl.head_dim), dtype=np.float32) * np.float32(wl.drift_std)
        steps[0] = 0.0
        self.drift = np.cumsum(steps, axis=0, dtype=np.float32)  # [frames][H][d]

    def frame(self, stream: str, f: int) -> np.ndarray:
        """bf16 bit patterns [H][T][d] of frame f of stream 'q', 'k' or 'v'."""
        wl = self.wl
        sid = {"q": STREAM_Q, "k": STREAM_K, "v": STREAM_V}[stream]
        x = frame_block(self.seed, sid, f, wl.heads, wl.frame_tokens, wl.head_dim, wl.input_std)
        if stream == "k":
            x += self.drift[f][:, None, :]
        return bf16_bits(x)

    def frames(self, stream: str, lo: int, hi: int) -> np.ndarray:
        wl = self.wl
        if hi <= lo:
            return np.zeros((wl.heads, 0, wl.head_dim), np.uint16)
        return np.concatenate([self.frame(stream, f) for f in range(lo, hi)], axis=1)
