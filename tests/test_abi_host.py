"""Host-side checks of the C ABI (include/hf.h / libhf.so); no GPU needed.

Validation happens before any HIP call, so every error path is exercised here on
the CPU. Calls with valid arguments need a device; without one they must fail
with HF_ERR_HIP rather than crash.
"""

import ctypes
import os
import re
import shutil
import subprocess

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hf.h")

hla = pytest.importorskip("hybrid_linear_block_amd",
                          reason="libhf.so not built (run __graft_entry__.build())")
B = hla.binding

NO_GPU = not torch.cuda.is_available()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(hf_[a-z_]+)\s*\(", text)))


def test_every_declared_function_is_exported():
    names = declared_functions()
    assert "hf_attend_chunk" in names and "hf_absorb_evicted" in names
    lib = ctypes.CDLL(hla.library_path())
    for n in names:
        assert hasattr(lib, n), f"{n} declared in hf.h but not exported"
    assert set(B.EXPORTED) == set(names)


def test_config_struct_layout_matches_c():
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    src = r"""
#include <stdio.h>
#include <stddef.h>
#include "hf.h"
int main(void) {
  printf("%zu %zu %zu %zu %zu %zu %zu %zu %zu %zu %zu\n", sizeof(hf_config),
         offsetof(hf_config, num_heads), offsetof(hf_config, head_dim),
         offsetof(hf_config, block_size), offsetof(hf_config, dtype), offsetof(hf_config, eps),
         offsetof(hf_config, softmax_scale), offsetof(hf_config, max_n_q),
         offsetof(hf_config, max_n_kv), offsetof(hf_config, max_n_ev),
         offsetof(hf_config, max_top_k));
  return 0;
}
"""
    tmp = os.path.join(ROOT, "tests", "_abi_layout_probe")
    with open(tmp + ".c", "w") as f:
        f.write(src)
    try:
        subprocess.check_call(["gcc", "-std=c99", "-Wall", "-Werror", "-I",
                               os.path.join(ROOT, "include"), tmp + ".c", "-o", tmp])
        got = [int(x) for x in subprocess.check_output([tmp]).split()]
    finally:
        for p in (tmp, tmp + ".c"):
            if os.path.exists(p):
                os.remove(p)
    C = B.hf_config
    want = [ctypes.sizeof(C)] + [getattr(C, f).offset for f, _ in C._fields_]
    assert got == want


def test_status_strings():
    for code in range(5):
        s = hla.hf_status_string(code)
        assert s.startswith("HF_")
    assert "unknown" in hla.hf_status_string(99)


def cfg(**kw):
    base = dict(num_heads=12, head_dim=128, block_size=64, dtype=B.HF_BF16, eps=1e-6,
                softmax_scale=0.0, max_n_q=4680, max_n_kv=14040, max_n_ev=4680, max_top_k=55)
    base.update(kw)
    return B.hf_config(*[base[f] for f, _ in B.hf_config._fields_])


def test_workspace_bytes():
    ok = hla.hf_workspace_bytes(cfg())
    assert ok > 0 and ok % 256 == 0
    assert hla.hf_workspace_bytes(cfg(max_n_kv=2 * 14040)) > ok
    assert hla.hf_workspace_bytes(cfg(dtype=B.HF_F32, block_size=16, head_dim=64)) > 0
    for bad in (dict(head_dim=96), dict(block_size=32), dict(dtype=7), dict(num_heads=0),
                dict(max_top_k=0), dict(max_n_q=0), dict(max_top_k=300), dict(eps=-1.0),
                dict(eps=0.0), dict(eps=float("inf")), dict(eps=float("nan")), dict(max_n_kv=64 * 2049),
                dict(dtype=B.HF_BF16, block_size=16)):
        assert hla.hf_workspace_bytes(cfg(**bad)) == 0, bad
    # Launch sizes are 32-bit: heads x (query + key blocks) is capped at 2^26.
    nb = lambda n: -(-n // 64)  # noqa: E731
    heads_ok = (1 << 26) // (nb(4680) + nb(14040))
    assert hla.hf_workspace_bytes(cfg(num_heads=heads_ok)) > 0
    assert hla.hf_workspace_bytes(cfg(num_heads=heads_ok + 1)) == 0


def test_backward_workspace_bytes():
    """Per-row statistics (4 fp32 per query row and head), the inverse selection
    index (a count and a list of query blocks per key block and head) and, for bf16
    states, the partial dS and dz of every 256-query-row chunk, 256-byte aligned
    pieces."""
    c = cfg()
    H, B_, d = c.num_heads, c.block_size, c.head_dim
    nqb, nkb = -(-c.max_n_q // B_), -(-c.max_n_kv // B_)
    up = lambda x: -(-x // 256) * 256  # noqa: E731
    expect = up(H * c.max_n_q * 16) + up(H * nkb * 4) + up(H * nkb * nqb * 4)
    parts = up(H * -(-c.max_n_q // 256) * (d * d + d) * 4)
    assert hla.hf_backward_workspace_bytes(c) == expect + parts
    f32 = cfg(dtype=B.HF_F32, block_size=16, head_dim=64)
    nqb, nkb = -(-f32.max_n_q // 16), -(-f32.max_n_kv // 16)
    assert hla.hf_backward_workspace_bytes(f32) == (up(H * f32.max_n_q * 16) + up(H * nkb * 4) +
                                                     up(H * nkb * nqb * 4))
    assert hla.hf_backward_workspace_bytes(cfg(head_dim=96)) == 0


def test_state_init_validation():
    c = cfg()
    ws = hla.hf_workspace_bytes(c)
    A = 1 << 20  # a fake, 16-byte aligned device address (never dereferenced on error)
    st, h = hla.hf_state_init(cfg(head_dim=96), A, A, A, ws, 1, 0, 0)
    assert st == B.HF_ERR_UNSUPPORTED and h is None
    st, _ = hla.hf_state_init(cfg(num_heads=0), A, A, A, ws, 1, 0, 0)
    assert st == B.HF_ERR_INVALID_ARG
    for S, z, w in ((0, A, A), (A, 0, A), (A, A, 0), (A + 4, A, A), (A, A + 8, A), (A, A, A + 2)):
        st, _ = hla.hf_state_init(c, S, z, w, ws, 1, 0, 0)
        assert st == B.HF_ERR_INVALID_ARG
    st, _ = hla.hf_state_init(c, A, A, A, ws - 1, 1, 0, 0)
    assert st == B.HF_ERR_INVALID_ARG
    st, _ = hla.hf_state_init(c, A, A, A, ws, 1, -5, 0)
    assert st == B.HF_ERR_INVALID_ARG
    h = ctypes.c_void_p()
    assert B._lib.hf_state_init(ctypes.byref(c), A, A, A, ws, 1, 0, None, None) == \
        B.HF_ERR_INVALID_ARG
    del h
    if NO_GPU:  # valid arguments reach the runtime, which has no device here
        st, h = hla.hf_state_init(c, A, A, A, ws, 1, 0, 0)
        assert st == B.HF_ERR_HIP and h is None


def test_calls_on_null_state_are_rejected():
    A = 1 << 20
    assert hla.hf_absorb_evicted(None, A, A, 10, 1280, 0, 0) == B.HF_ERR_INVALID_ARG
    assert hla.hf_attend_chunk(None, A, 10, 1280, A, A, 10, 1280, 1, A, 1280, 0, 0) == \
        B.HF_ERR_INVALID_ARG
    assert hla.hf_block_scores(None, A, 10, 1280, A, 10, 1280, A, 0) == B.HF_ERR_INVALID_ARG
    assert hla.hf_absorb_and_attend(None, A, A, 10, 1280, 0, A, 10, 1280, A, A, 10, 1280, 1, A,
                                    1280, 0, 0, 0) == B.HF_ERR_INVALID_ARG
    assert hla.hf_attend_chunk_cached(None, A, 10, 1280, A, A, 16, 2048, 0, 1, A, 1280, 0, 0) == \
        B.HF_ERR_INVALID_ARG
    assert hla.hf_absorb_and_attend_cached(None, A, A, 10, 1280, 0, A, 10, 1280, A, A, 16, 2048,
                                           0, 1, A, 1280, 0, 0) == B.HF_ERR_INVALID_ARG
    assert hla.hf_absorb_and_attend_ahead(None, A, 10, 1280, A, A, 16, 2048, -1, 1, A, 1280, 0,
                                          A, A, 10, 1280, 0, 0) == B.HF_ERR_INVALID_ARG
    assert hla.hf_absorb_flush(None, 0) == B.HF_ERR_INVALID_ARG
    assert hla.hf_pending_ev(None) == -1
    assert hla.hf_key_cache_reset(None) == B.HF_ERR_INVALID_ARG
    assert hla.hf_window_attach(None, A, A, 20, 10) == B.HF_ERR_INVALID_ARG
    assert hla.hf_window_begin_chunk(None, 1, 0)[0] == B.HF_ERR_INVALID_ARG
    assert hla.hf_window_attend(None, A, 10, 1280, 1, A, 1280, 0, 0) == B.HF_ERR_INVALID_ARG
    assert hla.hf_window_range(None)[0] == B.HF_ERR_INVALID_ARG
    assert hla.hf_attend_backward(None, A, 10, 1280, A, A, 10, 1280, A, 1, A, 1280, A, 1280, A, A,
                                  1280, A, A, A, 1 << 20, 0) == B.HF_ERR_INVALID_ARG
    assert hla.hf_absorb_backward(None, A, A, 10, 1280, A, A, A, A, 1280, 0) == \
        B.HF_ERR_INVALID_ARG
    assert hla.hf_profile_start(None, 4) == B.HF_ERR_INVALID_ARG
    assert hla.hf_next_ev_index(None) == -1
    hla.hf_state_destroy(None)  # allowed


def test_window_bookkeeping_matches_the_oracle():
    import oracle
    for c, W in ((2, 2), (3, 9), (1, 4), (4, 3)):
        for t in range(40):
            assert hla.window_frames(t, c, W) == oracle.stream_step_frames(t, c, W)


def test_noalloc_validation():
    """hf_attend_chunk_noalloc rejects bad arguments and calls too large for its static
    scratch before any HIP call; valid calls reach the runtime (no device here)."""
    A = 1 << 20
    c = cfg()
    H, d = c.num_heads, c.head_dim
    ok = dict(S=A, z=A, q=A, n_q=4680, qs=4680 * d, k=A, v=A, n_kv=14040, kvs=14040 * d,
              top_k=55, out=A, outs=4680 * d, sel=0)

    def call(cf=c, **kw):
        a = dict(ok, **kw)
        return hla.hf_attend_chunk_noalloc(cf, a["S"], a["z"], a["q"], a["n_q"], a["qs"], a["k"],
                                           a["v"], a["n_kv"], a["kvs"], a["top_k"], a["out"],
                                           a["outs"], a["sel"], 0)

    for bad in (dict(S=0), dict(z=A + 4), dict(q=0), dict(out=A + 2), dict(top_k=0),
                dict(top_k=221), dict(n_kv=0), dict(n_q=-1), dict(qs=10), dict(sel=A + 1)):
        assert call(**bad) == B.HF_ERR_INVALID_ARG, bad
    assert call(cf=cfg(head_dim=96)) == B.HF_ERR_UNSUPPORTED
    assert call(cf=cfg(eps=0.0)) == B.HF_ERR_INVALID_ARG
    # beyond the scratch: 4x the Wan-like window and chunk (about 11 MB of scratch)
    assert call(n_q=4 * 4680, qs=4 * 4680 * d, n_kv=4 * 14040, kvs=4 * 14040 * d,
                top_k=4 * 55, outs=4 * 4680 * d) == B.HF_ERR_INVALID_ARG
    assert call(n_q=0) == B.HF_OK  # nothing to do, nothing enqueued
    if NO_GPU:
        assert call() == B.HF_ERR_HIP
