"""PyTorch-facing handle over libhf: one hybrid-attention layer's streaming state.

The linear state (S, z) and the workspace are torch tensors on the GPU; every call
passes raw pointers and the current HIP stream to the C ABI and returns without
synchronising. Nothing here computes any part of the attention.
"""

from __future__ import annotations

from typing import Optional, Tuple

import torch

from . import binding as B

_DTYPES = {torch.bfloat16: B.HF_BF16, torch.float32: B.HF_F32}


def _check(status: int, what: str) -> None:
    if status != B.HF_OK:
        raise B.HfError(status, what)


def _rows(t: torch.Tensor, name: str, d: int) -> Tuple[int, int]:
    """(n, head stride in elements) of a [H][n][d] tensor with contiguous rows."""
    if t.dim() != 3 or t.shape[2] != d:
        raise ValueError(f"{name} must be [H][n][{d}], got {tuple(t.shape)}")
    if t.shape[1] > 1 and t.stride(1) != d or t.stride(2) != 1:
        raise ValueError(f"{name} must have contiguous rows of {d} elements")
    hs = t.stride(0) if t.shape[0] > 1 else max(t.shape[1] * d, 1)
    return t.shape[1], hs


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


class HybridAttentionState:
    """Per-layer state of the per-chunk hybrid attention (see include/hf.h)."""

    def __init__(self, num_heads: int, head_dim: int, block_size: int, dtype: torch.dtype,
                 max_n_q: int, max_n_kv: int, max_n_ev: int, max_top_k: int,
                 eps: float = 1e-6, softmax_scale: float = 0.0,
                 device: Optional[torch.device] = None, S: Optional[torch.Tensor] = None,
                 z: Optional[torch.Tensor] = None, next_ev_index: int = 0):
        if dtype not in _DTYPES:
            raise ValueError(f"unsupported dtype {dtype}")
        self.device = torch.device(device) if device is not None else torch.device("cuda", torch.cuda.current_device())
        self.dtype = dtype
        self.cfg = B.hf_config(num_heads, head_dim, block_size, _DTYPES[dtype], eps,
                               softmax_scale, max_n_q, max_n_kv, max_n_ev, max_top_k)
        ws = B.hf_workspace_bytes(self.cfg)
        if ws == 0:
            raise B.HfError(B.HF_ERR_UNSUPPORTED, "hf_workspace_bytes")
        adopt = S is not None
        if adopt != (z is not None):
            raise ValueError("pass both S and z to adopt a saved state, or neither")
        if adopt:
            if S.shape != (num_heads, head_dim, head_dim) or z.shape != (num_heads, head_dim):
                raise ValueError("S must be [H][d][d] and z [H][d]")
            self.S = S.to(device=self.device, dtype=torch.float32).contiguous().clone()
            self.z = z.to(device=self.device, dtype=torch.float32).contiguous().clone()
        else:
            self.S = torch.empty((num_heads, head_dim, head_dim), dtype=torch.float32,
                                 device=self.device)
            self.z = torch.empty((num_heads, head_dim), dtype=torch.float32, device=self.device)
        self.workspace = torch.empty(ws, dtype=torch.uint8, device=self.device)
        st, h = B.hf_state_init(self.cfg, self.S.data_ptr(), self.z.data_ptr(),
                                self.workspace.data_ptr(), ws, 0 if adopt else 1,
                                next_ev_index, _stream(self.device))
        _check(st, "hf_state_init")
        self._h = h

    # ------------------------------------------------------------------ calls

    @property
    def handle(self) -> int:
        if self._h is None:
            raise RuntimeError("state is closed")
        return self._h

    @property
    def next_ev_index(self) -> int:
        return B.hf_next_ev_index(self.handle)

    def _check_input(self, t: torch.Tensor, name: str) -> Tuple[int, int]:
        if t.dtype != self.dtype or t.device != self.device:
            raise ValueError(f"{name} must be {self.dtype} on {self.device}")
        if t.shape[0] != self.cfg.num_heads:
            raise ValueError(f"{name} must have {self.cfg.num_heads} heads")
        return _rows(t, name, self.cfg.head_dim)

    def set_rope(self, rot_dims: int, theta_base: float = 10000.0, tokens_per_frame: int = 1560,
                 cap: int = 8) -> None:
        """Relative temporal rotation of the softmax path (hf_set_rope); rot_dims = 0 turns
        it off. Allocates the rotation workspace (angle table and rotated keys)."""
        if rot_dims == 0:
            _check(B.hf_set_rope(self.handle, None, 0, 0, _stream(self.device)), "hf_set_rope")
            self.rope_workspace = None
            return
        rope = B.hf_rope(rot_dims, theta_base, tokens_per_frame, cap)
        nbytes = B.hf_rope_workspace_bytes(self.cfg, rope)
        if nbytes == 0:
            raise B.HfError(B.HF_ERR_INVALID_ARG, "hf_rope_workspace_bytes")
        ws = torch.empty(nbytes, dtype=torch.uint8, device=self.device)
        _check(B.hf_set_rope(self.handle, rope, ws.data_ptr(), nbytes, _stream(self.device)),
               "hf_set_rope")
        self.rope_workspace = ws

    def absorb_evicted(self, k_ev: torch.Tensor, v_ev: torch.Tensor,
                       ev_index: Optional[int] = None) -> None:
        """S += V^T phi(K), z += sum phi(K) over the evicted tokens (enqueued)."""
        n, hs = self._evicted_args(k_ev, v_ev)
        idx = self.next_ev_index if ev_index is None else ev_index
        _check(B.hf_absorb_evicted(self.handle, k_ev.data_ptr(), v_ev.data_ptr(), n, hs, idx,
                                   _stream(self.device)), "hf_absorb_evicted")

    def _evicted_args(self, k_ev: torch.Tensor, v_ev: torch.Tensor):
        n, hs = self._check_input(k_ev, "k_ev")
        n2, hs2 = self._check_input(v_ev, "v_ev")
        if n2 != n or hs2 != hs:
            raise ValueError("k_ev and v_ev must have the same length and head stride")
        return n, hs

    def _attend_args(self, q, k_win, v_win, top_k, out, sel_out):
        n_q, q_hs = self._check_input(q, "q")
        n_kv, kv_hs = self._check_input(k_win, "k_win")
        n_kv2, kv_hs2 = self._check_input(v_win, "v_win")
        if n_kv2 != n_kv or kv_hs2 != kv_hs:
            raise ValueError("k_win and v_win must have the same length and head stride")
        if out is None:
            out = torch.empty((self.cfg.num_heads, n_q, self.cfg.head_dim), dtype=self.dtype,
                              device=self.device)
        n_o, o_hs = self._check_input(out, "out")
        if n_o != n_q:
            raise ValueError("out must have as many rows as q")
        sel_ptr = self._sel_ptr(sel_out, n_q, top_k)
        return out, (q.data_ptr(), n_q, q_hs, k_win.data_ptr(), v_win.data_ptr(), n_kv, kv_hs,
                     int(top_k), out.data_ptr(), o_hs, sel_ptr)

    def _sel_ptr(self, sel_out: Optional[torch.Tensor], n_q: int, top_k: int) -> int:
        if sel_out is None:
            return 0
        nqb = -(-n_q // self.cfg.block_size)
        if (sel_out.dtype != torch.int32 or sel_out.device != self.device
                or tuple(sel_out.shape) != (self.cfg.num_heads, nqb, top_k)
                or not sel_out.is_contiguous()):
            raise ValueError(f"sel_out must be contiguous int32 [H][{nqb}][{top_k}]")
        return sel_out.data_ptr()

    def attend_chunk(self, q: torch.Tensor, k_win: torch.Tensor, v_win: torch.Tensor,
                     top_k: int, out: Optional[torch.Tensor] = None,
                     sel_out: Optional[torch.Tensor] = None,
                     win_index: Optional[int] = None) -> torch.Tensor:
        """Hybrid attention of the chunk q over the window (and the state); enqueued.
        With win_index (absolute index of the window's first token in the stream), the
        key pooling uses the state's cache of 8-token key sums (same results)."""
        out, args = self._attend_args(q, k_win, v_win, top_k, out, sel_out)
        if win_index is None:
            _check(B.hf_attend_chunk(self.handle, *args, _stream(self.device)), "hf_attend_chunk")
        else:
            a = list(args)
            a.insert(7, int(win_index))  # after kv_head_stride
            _check(B.hf_attend_chunk_cached(self.handle, *a, _stream(self.device)),
                   "hf_attend_chunk_cached")
        return out

    def absorb_and_attend(self, k_ev: torch.Tensor, v_ev: torch.Tensor, q: torch.Tensor,
                          k_win: torch.Tensor, v_win: torch.Tensor, top_k: int,
                          out: Optional[torch.Tensor] = None,
                          sel_out: Optional[torch.Tensor] = None,
                          ev_index: Optional[int] = None,
                          side_stream: Optional[torch.cuda.Stream] = None,
                          win_index: Optional[int] = None) -> torch.Tensor:
        """absorb_evicted then attend_chunk in one call (same results); with a side
        stream the absorb overlaps the block scoring and selection. With win_index
        (one stream only) the key pooling uses the state's cache of 8-token key sums."""
        n_ev, ev_hs = self._evicted_args(k_ev, v_ev)
        out, args = self._attend_args(q, k_win, v_win, top_k, out, sel_out)
        idx = self.next_ev_index if ev_index is None else ev_index
        if win_index is None:
            side = side_stream.cuda_stream if side_stream is not None else 0
            _check(B.hf_absorb_and_attend(self.handle, k_ev.data_ptr(), v_ev.data_ptr(), n_ev,
                                          ev_hs, idx, *args, _stream(self.device), side),
                   "hf_absorb_and_attend")
        else:
            if side_stream is not None:
                raise ValueError("the cached form runs on one stream")
            a = list(args)
            a.insert(7, int(win_index))  # after kv_head_stride
            _check(B.hf_absorb_and_attend_cached(self.handle, k_ev.data_ptr(), v_ev.data_ptr(),
                                                 n_ev, ev_hs, idx, *a, _stream(self.device)),
                   "hf_absorb_and_attend_cached")
        return out

    def absorb_and_attend_ahead(self, q: torch.Tensor, k_win: torch.Tensor, v_win: torch.Tensor,
                                top_k: int, k_next: Optional[torch.Tensor] = None,
                                v_next: Optional[torch.Tensor] = None,
                                out: Optional[torch.Tensor] = None,
                                sel_out: Optional[torch.Tensor] = None,
                                next_index: Optional[int] = None,
                                win_index: Optional[int] = None) -> torch.Tensor:
        """Attend the chunk with the state as of the previous call's pending absorb
        (reduced first), and form the partial states of the next chunk's evicted tokens
        (k_next, v_next) inside the attention launch as the new pending absorb
        (hf_absorb_and_attend_ahead). absorb_flush() completes a pending absorb."""
        out, args = self._attend_args(q, k_win, v_win, top_k, out, sel_out)
        if k_next is None:
            n_next, nx_hs, kp, vp = 0, 0, 0, 0
        else:
            n_next, nx_hs = self._evicted_args(k_next, v_next)
            kp, vp = k_next.data_ptr(), v_next.data_ptr()
        idx = self.next_ev_index if next_index is None else next_index
        a = list(args)
        a.insert(7, -1 if win_index is None else int(win_index))  # after kv_head_stride
        _check(B.hf_absorb_and_attend_ahead(self.handle, *a, kp, vp, n_next, nx_hs, idx,
                                            _stream(self.device)),
               "hf_absorb_and_attend_ahead")
        return out

    def absorb_flush(self) -> None:
        """Reduce the pending absorb of absorb_and_attend_ahead into S and z."""
        _check(B.hf_absorb_flush(self.handle, _stream(self.device)), "hf_absorb_flush")

    @property
    def pending_ev(self) -> int:
        """Tokens whose partial states wait for the next call to reduce them."""
        return B.hf_pending_ev(self.handle)

    def attend_ragged(self, q: torch.Tensor, k_flat: torch.Tensor, v_flat: torch.Tensor,
                      kv_offsets, top_k, out: Optional[torch.Tensor] = None,
                      sel_out: Optional[torch.Tensor] = None) -> torch.Tensor:
        """Head-aware ragged windows (hf_attend_ragged): head h attends rows
        kv_offsets[h] .. kv_offsets[h + 1] of k_flat / v_flat ([rows][d]) with its own
        top_k[h]; sel_out, if given, is int32 [H][ceil(n_q / B)][max(top_k)]."""
        n_q, q_hs = self._check_input(q, "q")
        d = self.cfg.head_dim
        for name, t in (("k_flat", k_flat), ("v_flat", v_flat)):
            if t.dtype != self.dtype or t.device != self.device or t.dim() != 2 or \
                    t.shape[1] != d or not t.is_contiguous():
                raise ValueError(f"{name} must be contiguous [rows][{d}] {self.dtype}")
        if out is None:
            out = torch.empty((self.cfg.num_heads, n_q, d), dtype=self.dtype, device=self.device)
        _, o_hs = self._check_input(out, "out")
        sel_ptr = 0
        if sel_out is not None:
            nqb = -(-n_q // self.cfg.block_size)
            if sel_out.dtype != torch.int32 or tuple(sel_out.shape) != \
                    (self.cfg.num_heads, nqb, max(top_k)) or not sel_out.is_contiguous():
                raise ValueError("sel_out must be contiguous int32 [H][ceil(n_q/B)][max(top_k)]")
            sel_ptr = sel_out.data_ptr()
        _check(B.hf_attend_ragged(self.handle, q.data_ptr(), n_q, q_hs, k_flat.data_ptr(),
                                  v_flat.data_ptr(), list(kv_offsets), list(top_k), out.data_ptr(),
                                  o_hs, sel_ptr, _stream(self.device)), "hf_attend_ragged")
        return out

    def key_cache_reset(self) -> None:
        """Forget the cached 8-token key sums (host-side; enqueues nothing)."""
        _check(B.hf_key_cache_reset(self.handle), "hf_key_cache_reset")

    # ------------------------------------------------------- managed window

    def window_attach(self, window_tokens: int, ring_tokens: Optional[int] = None) -> None:
        """Let the state keep the sliding window of window_tokens tokens in a K/V ring of
        ring_tokens rows per head (default 2 * window_tokens), allocated here."""
        ring = 2 * window_tokens if ring_tokens is None else int(ring_tokens)
        shape = (self.cfg.num_heads, max(ring, 1), self.cfg.head_dim)
        k_ring = torch.empty(shape, dtype=self.dtype, device=self.device)
        v_ring = torch.empty(shape, dtype=self.dtype, device=self.device)
        _check(B.hf_window_attach(self.handle, k_ring.data_ptr(), v_ring.data_ptr(), ring,
                                  int(window_tokens)), "hf_window_attach")
        self.k_ring, self.v_ring = k_ring, v_ring

    def begin_chunk(self, n: int) -> Tuple[torch.Tensor, torch.Tensor]:
        """Start a chunk of n tokens; returns the ring views [H][n][d] that its K and V
        must be written to (on the current stream) before window_attend."""
        st, kp, vp, hs = B.hf_window_begin_chunk(self.handle, int(n), _stream(self.device))
        _check(st, "hf_window_begin_chunk")
        row_bytes = self.cfg.head_dim * self.k_ring.element_size()
        row = (kp - self.k_ring.data_ptr()) // row_bytes
        if (vp - self.v_ring.data_ptr()) // row_bytes != row or hs != self.k_ring.stride(0):
            raise RuntimeError("hf_window_begin_chunk returned an unexpected slot")
        return self.k_ring[:, row:row + n], self.v_ring[:, row:row + n]

    def window_attend(self, q: torch.Tensor, top_k: int, out: Optional[torch.Tensor] = None,
                      sel_out: Optional[torch.Tensor] = None) -> torch.Tensor:
        """Hybrid attention of the current chunk's queries against the managed window
        and the state (absorbing what left the window first); enqueued."""
        n_q, q_hs = self._check_input(q, "q")
        if out is None:
            out = torch.empty((self.cfg.num_heads, n_q, self.cfg.head_dim), dtype=self.dtype,
                              device=self.device)
        n_o, o_hs = self._check_input(out, "out")
        if n_o != n_q:
            raise ValueError("out must have as many rows as q")
        sel_ptr = self._sel_ptr(sel_out, n_q, top_k)
        _check(B.hf_window_attend(self.handle, q.data_ptr(), n_q, q_hs, int(top_k),
                                  out.data_ptr(), o_hs, sel_ptr, _stream(self.device)),
               "hf_window_attend")
        return out

    def window_range(self) -> Tuple[int, int]:
        """(absolute index of the first token, token count) of the managed window."""
        st, first, count = B.hf_window_range(self.handle)
        _check(st, "hf_window_range")
        return first, count

    # ------------------------------------------------------------ backward

    def attend_backward(self, q: torch.Tensor, k_win: torch.Tensor, v_win: torch.Tensor,
                        sel: torch.Tensor, dout: torch.Tensor):
        """Gradients of an attend_chunk call with its selection `sel` held fixed; the
        state must be as at that call. Returns fp32 (dq, dk_win, dv_win, dS, dz)."""
        _, args = self._attend_args(q, k_win, v_win, sel.shape[2], q, None)
        n_q, q_hs, n_kv, kv_hs = args[1], args[2], args[5], args[6]
        n_d, d_hs = self._check_input(dout, "dout")
        if n_d != n_q:
            raise ValueError("dout must have as many rows as q")
        nqb = -(-n_q // self.cfg.block_size)
        if (sel.dtype != torch.int32 or sel.device != self.device or not sel.is_contiguous()
                or tuple(sel.shape[:2]) != (self.cfg.num_heads, nqb)):
            raise ValueError(f"sel must be contiguous int32 [H][{nqb}][top_k]")
        H, d = self.cfg.num_heads, self.cfg.head_dim
        f32 = dict(dtype=torch.float32, device=self.device)
        dq = torch.empty((H, n_q, d), **f32)
        dk, dv = torch.empty((H, n_kv, d), **f32), torch.empty((H, n_kv, d), **f32)
        dS, dz = torch.empty((H, d, d), **f32), torch.empty((H, d), **f32)
        if getattr(self, "_bwd_ws", None) is None:
            self._bwd_ws = torch.empty(B.hf_backward_workspace_bytes(self.cfg), dtype=torch.uint8,
                                       device=self.device)
        _check(B.hf_attend_backward(self.handle, q.data_ptr(), n_q, q_hs, k_win.data_ptr(),
                                    v_win.data_ptr(), n_kv, kv_hs, sel.data_ptr(),
                                    int(sel.shape[2]), dout.data_ptr(), d_hs, dq.data_ptr(),
                                    n_q * d, dk.data_ptr(), dv.data_ptr(), n_kv * d, dS.data_ptr(),
                                    dz.data_ptr(), self._bwd_ws.data_ptr(), self._bwd_ws.numel(),
                                    _stream(self.device)), "hf_attend_backward")
        return dq, dk, dv, dS, dz

    def absorb_backward(self, k_ev: torch.Tensor, v_ev: torch.Tensor, dS: torch.Tensor,
                        dz: torch.Tensor):
        """fp32 (dk_ev, dv_ev) through an absorb of k_ev, v_ev, from the state's dS, dz."""
        n, hs = self._evicted_args(k_ev, v_ev)
        H, d = self.cfg.num_heads, self.cfg.head_dim
        for t, shape in ((dS, (H, d, d)), (dz, (H, d))):
            if t.dtype != torch.float32 or tuple(t.shape) != shape or not t.is_contiguous():
                raise ValueError(f"dS, dz must be contiguous fp32 {shape}")
        f32 = dict(dtype=torch.float32, device=self.device)
        dk, dv = torch.empty((H, n, d), **f32), torch.empty((H, n, d), **f32)
        _check(B.hf_absorb_backward(self.handle, k_ev.data_ptr(), v_ev.data_ptr(), n, hs,
                                    dS.data_ptr(), dz.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                                    max(n, 1) * d, _stream(self.device)), "hf_absorb_backward")
        return dk, dv

    def block_scores(self, q: torch.Tensor, k_win: torch.Tensor) -> torch.Tensor:
        """fp32 pooled block scores [H][ceil(n_q/B)][ceil(n_kv/B)] (enqueued)."""
        n_q, q_hs = self._check_input(q, "q")
        n_kv, kv_hs = self._check_input(k_win, "k_win")
        bs = self.cfg.block_size
        scores = torch.empty((self.cfg.num_heads, -(-n_q // bs), -(-n_kv // bs)),
                             dtype=torch.float32, device=self.device)
        _check(B.hf_block_scores(self.handle, q.data_ptr(), n_q, q_hs, k_win.data_ptr(), n_kv,
                                 kv_hs, scores.data_ptr(), _stream(self.device)),
               "hf_block_scores")
        return scores

    def profile_start(self, max_launches: int) -> None:
        """Record HIP events around each kernel this state launches (profiling aid)."""
        _check(B.hf_profile_start(self.handle, max_launches), "hf_profile_start")

    def profile_stop(self):
        """{kernel: (total ms, launches)} since profile_start; waits for the events."""
        st, res = B.hf_profile_stop(self.handle)
        _check(st, "hf_profile_stop")
        return res

    def close(self) -> None:
        if getattr(self, "_h", None) is not None:
            B.hf_state_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def window_frames(step: int, chunk_frames: int, window_frames: int):
    """Caller-side window bookkeeping of a chunked stream.

    Chunk `step` holds frames [c*step, c*step + c). Before attending it, the frames
    that left the last-W-frames window since the previous step are evicted (and
    must be absorbed); the window is the last W frames up to and including the
    chunk. Returns ((evict_lo, evict_hi), (win_lo, win_hi)) in frames.
    """
    end = chunk_frames * (step + 1)
    lo = end - window_frames if end > window_frames else 0
    prev_end = chunk_frames * step
    prev_lo = prev_end - window_frames if prev_end > window_frames else 0
    return (prev_lo if step > 0 else 0, lo), (lo, end)
