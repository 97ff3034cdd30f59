"""ctypes binding of libhf.so (the C ABI declared in include/hf.h).

Argument marshalling only: every step of the hybrid attention runs in the HIP
kernels of libhf. PyTorch provides device memory and the stream. If the library
has not been built, importing this module raises; there is no fallback.
"""

from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, Structure, c_float, c_int, c_int32, c_int64, c_size_t, c_void_p

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libhf.so")

HF_OK = 0
HF_ERR_INVALID_ARG = 1
HF_ERR_UNSUPPORTED = 2
HF_ERR_STATE = 3
HF_ERR_HIP = 4
HF_BF16 = 0
HF_F32 = 1


class hf_config(Structure):
    _fields_ = [
        ("num_heads", c_int32),
        ("head_dim", c_int32),
        ("block_size", c_int32),
        ("dtype", c_int32),
        ("eps", c_float),
        ("softmax_scale", c_float),
        ("max_n_q", c_int64),
        ("max_n_kv", c_int64),
        ("max_n_ev", c_int64),
        ("max_top_k", c_int32),
    ]


class hf_rope(ctypes.Structure):
    _fields_ = [
        ("rot_dims", c_int32),
        ("theta_base", c_float),
        ("tokens_per_frame", c_int64),
        ("cap", c_int32),
    ]


class HfError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {hf_status_string(status)}")


def _load():
    if not os.path.exists(_LIB_PATH):
        raise ImportError(
            f"{_LIB_PATH} is missing: build the HIP library first "
            "(python hybrid_linear_block_amd/build.py, or __graft_entry__.build())")
    lib = ctypes.CDLL(_LIB_PATH)
    P = c_void_p
    sig = {
        "hf_workspace_bytes": (c_size_t, [POINTER(hf_config)]),
        "hf_state_init": (c_int, [POINTER(hf_config), P, P, P, c_size_t, c_int, c_int64, P,
                                  POINTER(c_void_p)]),
        "hf_absorb_evicted": (c_int, [P, P, P, c_int64, c_int64, c_int64, P]),
        "hf_attend_chunk": (c_int, [P, P, c_int64, c_int64, P, P, c_int64, c_int64, c_int32, P,
                                    c_int64, P, P]),
        "hf_absorb_and_attend": (c_int, [P, P, P, c_int64, c_int64, c_int64, P, c_int64, c_int64,
                                         P, P, c_int64, c_int64, c_int32, P, c_int64, P, P, P]),
        "hf_attend_chunk_cached": (c_int, [P, P, c_int64, c_int64, P, P, c_int64, c_int64,
                                           c_int64, c_int32, P, c_int64, P, P]),
        "hf_absorb_and_attend_cached": (c_int, [P, P, P, c_int64, c_int64, c_int64, P, c_int64,
                                                c_int64, P, P, c_int64, c_int64, c_int64, c_int32,
                                                P, c_int64, P, P]),
        "hf_absorb_and_attend_ahead": (c_int, [P, P, c_int64, c_int64, P, P, c_int64, c_int64,
                                               c_int64, c_int32, P, c_int64, P, P, P, c_int64,
                                               c_int64, c_int64, P]),
        "hf_absorb_flush": (c_int, [P, P]),
        "hf_pending_ev": (c_int64, [P]),
        "hf_key_cache_reset": (c_int, [P]),
        "hf_window_attach": (c_int, [P, P, P, c_int64, c_int64]),
        "hf_window_begin_chunk": (c_int, [P, c_int64, P, POINTER(c_void_p), POINTER(c_void_p),
                                          POINTER(c_int64)]),
        "hf_window_attend": (c_int, [P, P, c_int64, c_int64, c_int32, P, c_int64, P, P]),
        "hf_window_range": (c_int, [P, POINTER(c_int64), POINTER(c_int64)]),
        "hf_block_scores": (c_int, [P, P, c_int64, c_int64, P, c_int64, c_int64, P, P]),
        "hf_backward_workspace_bytes": (c_size_t, [POINTER(hf_config)]),
        "hf_attend_backward": (c_int, [P, P, c_int64, c_int64, P, P, c_int64, c_int64, P, c_int32,
                                       P, c_int64, P, c_int64, P, P, c_int64, P, P, P, c_size_t,
                                       P]),
        "hf_absorb_backward": (c_int, [P, P, P, c_int64, c_int64, P, P, P, P, c_int64, P]),
        "hf_attend_ragged": (c_int, [P, P, c_int64, c_int64, P, P, POINTER(c_int64),
                                     POINTER(c_int32), P, c_int64, P, P]),
        "hf_rope_workspace_bytes": (c_size_t, [POINTER(hf_config), POINTER(hf_rope)]),
        "hf_set_rope": (c_int, [P, POINTER(hf_rope), P, c_size_t, P]),
        "hf_attend_chunk_noalloc": (c_int, [POINTER(hf_config), P, P, P, c_int64, c_int64, P, P,
                                            c_int64, c_int64, c_int32, P, c_int64, P, P]),
        "hf_profile_start": (c_int, [P, c_int32]),
        "hf_profile_stop": (c_int, [P, POINTER(ctypes.c_double), POINTER(c_int32)]),
        "hf_next_ev_index": (c_int64, [P]),
        "hf_state_destroy": (None, [P]),
        "hf_status_string": (ctypes.c_char_p, [c_int]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib = _load()

EXPORTED = ("hf_workspace_bytes", "hf_state_init", "hf_absorb_evicted", "hf_attend_chunk",
            "hf_absorb_and_attend", "hf_attend_chunk_cached", "hf_absorb_and_attend_cached",
            "hf_absorb_and_attend_ahead", "hf_absorb_flush", "hf_pending_ev",
            "hf_key_cache_reset", "hf_window_attach", "hf_window_begin_chunk",
            "hf_window_attend", "hf_window_range", "hf_block_scores",
            "hf_backward_workspace_bytes", "hf_attend_backward", "hf_absorb_backward",
            "hf_attend_ragged", "hf_rope_workspace_bytes", "hf_set_rope",
            "hf_attend_chunk_noalloc",
            "hf_profile_start",
            "hf_profile_stop", "hf_next_ev_index", "hf_state_destroy", "hf_status_string")
HF_KERNEL_NAMES = ("absorb", "block_pool", "score_select", "sparse_swa", "bwd_index", "bwd_dq",
                   "bwd_dkv", "bwd_state", "absorb_bwd")


def library_path() -> str:
    return _LIB_PATH


# ---------------------------------------------------------------- raw C calls
# Same names and argument order as include/hf.h; pointers and streams are ints.


def hf_status_string(status: int) -> str:
    return _lib.hf_status_string(int(status)).decode()


def hf_workspace_bytes(cfg: hf_config) -> int:
    return int(_lib.hf_workspace_bytes(ctypes.byref(cfg)))


def hf_state_init(cfg: hf_config, S: int, z: int, workspace: int, ws_bytes: int, zero_fill: int,
                  next_ev_index: int, stream: int):
    """Returns (status, handle or None)."""
    h = c_void_p()
    st = _lib.hf_state_init(ctypes.byref(cfg), S, z, workspace, ws_bytes, int(zero_fill),
                            int(next_ev_index), stream, ctypes.byref(h))
    return st, (h.value if st == HF_OK else None)


def hf_absorb_evicted(state: int, k_ev: int, v_ev: int, n_ev: int, ev_head_stride: int,
                      ev_index: int, stream: int) -> int:
    return _lib.hf_absorb_evicted(state, k_ev, v_ev, n_ev, ev_head_stride, ev_index, stream)


def hf_attend_chunk(state: int, q: int, n_q: int, q_head_stride: int, k_win: int, v_win: int,
                    n_kv: int, kv_head_stride: int, top_k: int, out: int, out_head_stride: int,
                    sel_out: int, stream: int) -> int:
    return _lib.hf_attend_chunk(state, q, n_q, q_head_stride, k_win, v_win, n_kv,
                                kv_head_stride, top_k, out, out_head_stride, sel_out, stream)


def hf_absorb_and_attend(state: int, k_ev: int, v_ev: int, n_ev: int, ev_head_stride: int,
                         ev_index: int, q: int, n_q: int, q_head_stride: int, k_win: int,
                         v_win: int, n_kv: int, kv_head_stride: int, top_k: int, out: int,
                         out_head_stride: int, sel_out: int, stream: int, side_stream: int) -> int:
    return _lib.hf_absorb_and_attend(state, k_ev, v_ev, n_ev, ev_head_stride, ev_index, q, n_q,
                                     q_head_stride, k_win, v_win, n_kv, kv_head_stride, top_k,
                                     out, out_head_stride, sel_out, stream, side_stream)


def hf_attend_chunk_cached(state: int, q: int, n_q: int, q_head_stride: int, k_win: int,
                           v_win: int, n_kv: int, kv_head_stride: int, win_index: int, top_k: int,
                           out: int, out_head_stride: int, sel_out: int, stream: int) -> int:
    return _lib.hf_attend_chunk_cached(state, q, n_q, q_head_stride, k_win, v_win, n_kv,
                                       kv_head_stride, win_index, top_k, out, out_head_stride,
                                       sel_out, stream)


def hf_absorb_and_attend_cached(state: int, k_ev: int, v_ev: int, n_ev: int, ev_head_stride: int,
                                ev_index: int, q: int, n_q: int, q_head_stride: int, k_win: int,
                                v_win: int, n_kv: int, kv_head_stride: int, win_index: int,
                                top_k: int, out: int, out_head_stride: int, sel_out: int,
                                stream: int) -> int:
    return _lib.hf_absorb_and_attend_cached(state, k_ev, v_ev, n_ev, ev_head_stride, ev_index, q,
                                            n_q, q_head_stride, k_win, v_win, n_kv,
                                            kv_head_stride, win_index, top_k, out,
                                            out_head_stride, sel_out, stream)


def hf_absorb_and_attend_ahead(state: int, q: int, n_q: int, q_head_stride: int, k_win: int,
                               v_win: int, n_kv: int, kv_head_stride: int, win_index: int,
                               top_k: int, out: int, out_head_stride: int, sel_out: int,
                               k_next: int, v_next: int, n_next: int, next_head_stride: int,
                               next_index: int, stream: int) -> int:
    return _lib.hf_absorb_and_attend_ahead(state, q, n_q, q_head_stride, k_win, v_win, n_kv,
                                           kv_head_stride, win_index, top_k, out,
                                           out_head_stride, sel_out, k_next, v_next, n_next,
                                           next_head_stride, next_index, stream)


def hf_absorb_flush(state: int, stream: int) -> int:
    return _lib.hf_absorb_flush(state, stream)


def hf_pending_ev(state: int) -> int:
    return _lib.hf_pending_ev(state)


def hf_key_cache_reset(state: int) -> int:
    return _lib.hf_key_cache_reset(state)


def hf_window_attach(state: int, k_ring: int, v_ring: int, ring_tokens: int,
                     window_tokens: int) -> int:
    return _lib.hf_window_attach(state, k_ring, v_ring, ring_tokens, window_tokens)


def hf_window_begin_chunk(state: int, n: int, stream: int):
    """Returns (status, k_slot, v_slot, head_stride)."""
    k, v, hs = c_void_p(), c_void_p(), c_int64()
    st = _lib.hf_window_begin_chunk(state, n, stream, ctypes.byref(k), ctypes.byref(v),
                                    ctypes.byref(hs))
    return st, k.value, v.value, hs.value


def hf_window_attend(state: int, q: int, n_q: int, q_head_stride: int, top_k: int, out: int,
                     out_head_stride: int, sel_out: int, stream: int) -> int:
    return _lib.hf_window_attend(state, q, n_q, q_head_stride, top_k, out, out_head_stride,
                                 sel_out, stream)


def hf_window_range(state: int):
    """Returns (status, first token, token count)."""
    first, count = c_int64(), c_int64()
    st = _lib.hf_window_range(state, ctypes.byref(first), ctypes.byref(count))
    return st, first.value, count.value


def hf_block_scores(state: int, q: int, n_q: int, q_head_stride: int, k_win: int, n_kv: int,
                    kv_head_stride: int, scores_out: int, stream: int) -> int:
    return _lib.hf_block_scores(state, q, n_q, q_head_stride, k_win, n_kv, kv_head_stride,
                                scores_out, stream)


def hf_backward_workspace_bytes(cfg: hf_config) -> int:
    return int(_lib.hf_backward_workspace_bytes(ctypes.byref(cfg)))


def hf_attend_backward(state: int, q: int, n_q: int, q_head_stride: int, k_win: int, v_win: int,
                       n_kv: int, kv_head_stride: int, sel: int, top_k: int, dout: int,
                       dout_head_stride: int, dq: int, dq_head_stride: int, dk_win: int,
                       dv_win: int, dkv_head_stride: int, dS: int, dz: int, bwd_ws: int,
                       bwd_ws_bytes: int, stream: int) -> int:
    return _lib.hf_attend_backward(state, q, n_q, q_head_stride, k_win, v_win, n_kv,
                                   kv_head_stride, sel, top_k, dout, dout_head_stride, dq,
                                   dq_head_stride, dk_win, dv_win, dkv_head_stride, dS, dz,
                                   bwd_ws, bwd_ws_bytes, stream)


def hf_absorb_backward(state: int, k_ev: int, v_ev: int, n_ev: int, ev_head_stride: int, dS: int,
                       dz: int, dk_ev: int, dv_ev: int, dev_head_stride: int, stream: int) -> int:
    return _lib.hf_absorb_backward(state, k_ev, v_ev, n_ev, ev_head_stride, dS, dz, dk_ev, dv_ev,
                                   dev_head_stride, stream)


def hf_attend_ragged(state: int, q: int, n_q: int, q_head_stride: int, k_flat: int, v_flat: int,
                     kv_offsets, top_k, out: int, out_head_stride: int, sel_out: int,
                     stream: int) -> int:
    """kv_offsets (num_heads + 1) and top_k (num_heads): sequences of ints (host)."""
    off = (c_int64 * len(kv_offsets))(*[int(x) for x in kv_offsets])
    tk = (c_int32 * len(top_k))(*[int(x) for x in top_k])
    return _lib.hf_attend_ragged(state, q, n_q, q_head_stride, k_flat, v_flat, off, tk, out,
                                 out_head_stride, sel_out, stream)


def hf_rope_workspace_bytes(cfg: hf_config, rope: hf_rope) -> int:
    return int(_lib.hf_rope_workspace_bytes(ctypes.byref(cfg), ctypes.byref(rope)))


def hf_set_rope(state: int, rope, workspace: int, ws_bytes: int, stream: int) -> int:
    return _lib.hf_set_rope(state, ctypes.byref(rope) if rope is not None else None, workspace,
                            ws_bytes, stream)


def hf_attend_chunk_noalloc(cfg: hf_config, S: int, z: int, q: int, n_q: int, q_head_stride: int,
                            k_win: int, v_win: int, n_kv: int, kv_head_stride: int, top_k: int,
                            out: int, out_head_stride: int, sel_out: int, stream: int) -> int:
    return _lib.hf_attend_chunk_noalloc(ctypes.byref(cfg), S, z, q, n_q, q_head_stride, k_win,
                                        v_win, n_kv, kv_head_stride, top_k, out, out_head_stride,
                                        sel_out, stream)


def hf_profile_start(state: int, max_launches: int) -> int:
    return _lib.hf_profile_start(state, int(max_launches))


def hf_profile_stop(state: int):
    """Returns (status, {kernel name: (total ms, launches)})."""
    ms = (ctypes.c_double * len(HF_KERNEL_NAMES))()
    n = (c_int32 * len(HF_KERNEL_NAMES))()
    st = _lib.hf_profile_stop(state, ms, n)
    return st, {k: (ms[i], n[i]) for i, k in enumerate(HF_KERNEL_NAMES)}


def hf_next_ev_index(state) -> int:
    return int(_lib.hf_next_ev_index(state))


def hf_state_destroy(state) -> None:
    _lib.hf_state_destroy(state)
