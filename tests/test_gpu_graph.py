"""hf_attend_chunk captured into a HIP graph (torch.cuda.CUDAGraph) on one MI355X.

A denoising loop re-runs the chunk's attention over fixed buffers whose contents
change between runs; graph replays of the captured call must give, every time, the
outputs and selections of an eager call on the same contents, bit for bit. Replays
are interleaved with eager work and synchronisations.
"""

import numpy as np
import pytest
import torch

import synth
from hfutil import dev_bf16, dev_f32
from synth.inputs import frame_block

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import hybrid_linear_block_amd as hla  # the HIP library must load: no fallback path
else:
    hla = None


def _draw(seed, stream, H, n, d, std, dt):
    x = frame_block(seed, stream, 0, H, n, d, std)
    return dev_bf16(synth.bf16_bits(x)) if dt == "bf16" else dev_f32(x)


def _bits(t):
    return t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32)


@pytest.mark.parametrize("dt,d,B", [("bf16", 128, 64), ("f32", 64, 16)])
def test_graph_replays_match_eager(dt, d, B):
    H, n_q, n_kv, n_ev, K = 2, 200, 600, 300, 3
    std = 1.0 / np.sqrt(d)
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    mk = dict(max_n_q=n_q, max_n_kv=n_kv, max_n_ev=n_ev, max_top_k=K)
    g_st = hla.HybridAttentionState(H, d, B, tdt, **mk)
    e_st = hla.HybridAttentionState(H, d, B, tdt, **mk)
    kev, vev = _draw(81, 1, H, n_ev, d, std, dt), _draw(81, 2, H, n_ev, d, std, dt)
    for st in (g_st, e_st):  # a non-empty linear state, so the epilogue's read counts
        st.absorb_evicted(kev, vev)
    q = _draw(81, 3, H, n_q, d, std, dt)
    kw = _draw(81, 4, H, n_kv, d, std, dt)
    vw = _draw(81, 5, H, n_kv, d, std, dt)
    out = torch.empty((H, n_q, d), dtype=tdt, device="cuda")
    nqb = -(-n_q // B)
    sel = torch.empty((H, nqb, K), dtype=torch.int32, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # eager warm-up off the capture
        g_st.attend_chunk(q, kw, vw, K, out=out, sel_out=sel)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        g_st.attend_chunk(q, kw, vw, K, out=out, sel_out=sel)
    torch.cuda.synchronize()
    for r in range(4):
        q.copy_(_draw(82 + r, 3, H, n_q, d, std, dt))
        kw.copy_(_draw(82 + r, 4, H, n_kv, d, std, dt))
        vw.copy_(_draw(82 + r, 5, H, n_kv, d, std, dt))
        graph.replay()
        e_sel = torch.empty_like(sel)
        e_out = e_st.attend_chunk(q, kw, vw, K, sel_out=e_sel)
        torch.cuda.synchronize()
        print(f"replay {r}", flush=True)
        assert torch.equal(sel, e_sel)
        assert torch.equal(_bits(out), _bits(e_out))
        assert bool(torch.isfinite(out.float()).all())


@pytest.mark.parametrize("dt,d,B", [("bf16", 128, 64), ("f32", 64, 16)])
def test_graph_absorb_and_attend_replays_match_eager(dt, d, B):
    """The one-stream absorb + attention (three launches, the absorb's partial states
    next to the pooling and its reduce next to the selection) captured once: every
    replay absorbs the captured tokens again and attends the buffers' current contents;
    an eager state fed the same calls must hold the same state and give the same
    outputs and selections after every replay, bit for bit."""
    H, n_q, n_kv, n_ev, K = 2, 200, 600, 150, 3
    std = 1.0 / np.sqrt(d)
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    mk = dict(max_n_q=n_q, max_n_kv=n_kv, max_n_ev=n_ev, max_top_k=K)
    g_st = hla.HybridAttentionState(H, d, B, tdt, **mk)
    e_st = hla.HybridAttentionState(H, d, B, tdt, **mk)
    kev, vev = _draw(91, 1, H, n_ev, d, std, dt), _draw(91, 2, H, n_ev, d, std, dt)
    q = _draw(91, 3, H, n_q, d, std, dt)
    kw = _draw(91, 4, H, n_kv, d, std, dt)
    vw = _draw(91, 5, H, n_kv, d, std, dt)
    out = torch.empty((H, n_q, d), dtype=tdt, device="cuda")
    nqb = -(-n_q // B)
    sel = torch.empty((H, nqb, K), dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):  # recording enqueues nothing: the state is still empty
        g_st.absorb_and_attend(kev, vev, q, kw, vw, K, out=out, sel_out=sel, ev_index=0)
    torch.cuda.synchronize()
    for r in range(4):
        kev.copy_(_draw(92 + r, 1, H, n_ev, d, std, dt))
        vev.copy_(_draw(92 + r, 2, H, n_ev, d, std, dt))
        q.copy_(_draw(92 + r, 3, H, n_q, d, std, dt))
        kw.copy_(_draw(92 + r, 4, H, n_kv, d, std, dt))
        vw.copy_(_draw(92 + r, 5, H, n_kv, d, std, dt))
        graph.replay()
        e_sel = torch.empty_like(sel)
        e_out = e_st.absorb_and_attend(kev, vev, q, kw, vw, K, sel_out=e_sel, ev_index=r * n_ev)
        torch.cuda.synchronize()
        print(f"replay {r}", flush=True)
        assert torch.equal(g_st.S, e_st.S) and torch.equal(g_st.z, e_st.z)
        assert torch.equal(sel, e_sel)
        assert torch.equal(_bits(out), _bits(e_out))
        assert bool(torch.isfinite(out.float()).all())


@pytest.mark.parametrize("dt,d,B", [("bf16", 128, 64), ("f32", 64, 16)])
def test_graph_ahead_replays_match_eager(dt, d, B):
    """The absorb-ahead call captured in its steady state (a pending absorb to reduce in
    the selection launch, the next one formed with the attention): every replay reduces
    what the previous replay formed, attends the buffers' current contents and forms the
    absorb of the current evicted tokens. An eager state fed the same calls must hold the
    same state and give the same outputs and selections after every replay, bit for bit,
    and the same state after a final flush."""
    H, n_q, n_kv, n_ev, K = 2, 200, 600, 150, 3
    std = 1.0 / np.sqrt(d)
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    mk = dict(max_n_q=n_q, max_n_kv=n_kv, max_n_ev=n_ev, max_top_k=K)
    g_st = hla.HybridAttentionState(H, d, B, tdt, **mk)
    e_st = hla.HybridAttentionState(H, d, B, tdt, **mk)
    kev, vev = _draw(93, 1, H, n_ev, d, std, dt), _draw(93, 2, H, n_ev, d, std, dt)
    q = _draw(93, 3, H, n_q, d, std, dt)
    kw = _draw(93, 4, H, n_kv, d, std, dt)
    vw = _draw(93, 5, H, n_kv, d, std, dt)
    out = torch.empty((H, n_q, d), dtype=tdt, device="cuda")
    nqb = -(-n_q // B)
    sel = torch.empty((H, nqb, K), dtype=torch.int32, device="cuda")
    for st in (g_st, e_st):  # eager first call: leaves the first absorb pending
        st.absorb_and_attend_ahead(q, kw, vw, K, k_next=kev, v_next=vev)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        g_st.absorb_and_attend_ahead(q, kw, vw, K, k_next=kev, v_next=vev, out=out, sel_out=sel)
    torch.cuda.synchronize()
    for r in range(4):
        kev.copy_(_draw(94 + r, 1, H, n_ev, d, std, dt))
        vev.copy_(_draw(94 + r, 2, H, n_ev, d, std, dt))
        q.copy_(_draw(94 + r, 3, H, n_q, d, std, dt))
        kw.copy_(_draw(94 + r, 4, H, n_kv, d, std, dt))
        vw.copy_(_draw(94 + r, 5, H, n_kv, d, std, dt))
        graph.replay()
        e_sel = torch.empty_like(sel)
        e_out = e_st.absorb_and_attend_ahead(q, kw, vw, K, k_next=kev, v_next=vev, sel_out=e_sel)
        torch.cuda.synchronize()
        print(f"replay {r}", flush=True)
        assert torch.equal(g_st.S, e_st.S) and torch.equal(g_st.z, e_st.z)
        assert torch.equal(sel, e_sel)
        assert torch.equal(_bits(out), _bits(e_out))
        assert bool(torch.isfinite(out.float()).all())
    g_st.absorb_flush()
    e_st.absorb_flush()
    torch.cuda.synchronize()
    assert torch.equal(g_st.S, e_st.S) and torch.equal(g_st.z, e_st.z)
