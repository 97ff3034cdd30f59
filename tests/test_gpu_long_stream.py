"""Long stream on the GPU: 60 chunk steps (180 latent frames) of the Wan-like layer.

Each step absorbs the frames that left the 9-frame window (from step 3 on) and
attends the new 3-frame chunk. At every step the device state (S, z) is compared
with the float64 state of all tokens evicted so far, the selection with the
oracle's, and sampled output blocks with the oracle's outputs. K drifts slowly
(random-walk mean per frame) so the state stays non-trivial. A second state runs the
same stream through the absorb-ahead call (each step forms the next step's absorb in
its attention launch): its outputs, selections, S and z equal the first state's bit
for bit at every step.
"""

import time

import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import hybrid_linear_block_amd as hla  # the HIP library must load: no fallback path
from hfutil import (compare_out, compare_sel, dev_bf16, host_f64,  # noqa: E402
                    reference_selection, state_close)


@pytest.mark.timeout(900)
def test_long_stream_60_steps():
    wl = synth.WORKLOADS["long_stream_bf16"]
    H, d, B, T = wl.heads, wl.head_dim, wl.block, wl.frame_tokens
    c, W, F = wl.chunk_frames, wl.window_frames, wl.n_frames
    t0 = time.time()
    ls = synth.LongStream(31337)
    kbits = ls.frames("k", 0, F)
    vbits = ls.frames("v", 0, F)
    kd, vd = dev_bf16(kbits), dev_bf16(vbits)
    print(f"generated {F} frames in {time.time() - t0:.1f}s", flush=True)
    st = hla.HybridAttentionState(H, d, B, torch.bfloat16, max_n_q=c * T, max_n_kv=W * T,
                                  max_n_ev=c * T, max_top_k=synth.top_k_count(wl.top_k_frac, 220))
    ah = hla.HybridAttentionState(H, d, B, torch.bfloat16, max_n_q=c * T, max_n_kv=W * T,
                                  max_n_ev=c * T, max_top_k=synth.top_k_count(wl.top_k_frac, 220))
    S, z = oracle.state_init(H, d)
    rng = np.random.default_rng(5)
    n_steps = F // c
    for t in range(n_steps):
        (e0, e1), (w0, w1) = hla.window_frames(t, c, W)
        assert ((e0, e1), (w0, w1)) == oracle.stream_step_frames(t, c, W)
        if e1 > e0:
            st.absorb_evicted(kd[:, e0 * T:e1 * T], vd[:, e0 * T:e1 * T], ev_index=e0 * T)
            oracle.absorb(S, z, oracle.as_f64(kbits[:, e0 * T:e1 * T], "bf16"),
                          oracle.as_f64(vbits[:, e0 * T:e1 * T], "bf16"))
        qbits = ls.frames("q", w1 - c, w1)
        n_kv = (w1 - w0) * T
        nkb = -(-n_kv // B)
        K = synth.top_k_count(wl.top_k_frac, nkb)
        sel = torch.empty((H, c * T // B + 1, K), dtype=torch.int32, device="cuda")
        qd = dev_bf16(qbits)
        out = st.attend_chunk(qd, kd[:, w0 * T:w1 * T], vd[:, w0 * T:w1 * T], K, sel_out=sel)
        (n0, n1), _ = hla.window_frames(t + 1, c, W)  # the next step's evicted frames
        sel_ah = torch.empty_like(sel)
        out_ah = ah.absorb_and_attend_ahead(qd, kd[:, w0 * T:w1 * T], vd[:, w0 * T:w1 * T], K,
                                            k_next=kd[:, n0 * T:n1 * T], v_next=vd[:, n0 * T:n1 * T],
                                            sel_out=sel_ah)
        torch.cuda.synchronize()
        assert torch.equal(sel_ah, sel) and torch.equal(out_ah.view(torch.int16), out.view(torch.int16))
        assert torch.equal(ah.S, st.S) and torch.equal(ah.z, st.z)
        assert ah.pending_ev == (n1 - n0) * T
        fro, zrel = state_close(host_f64(st.S), host_f64(st.z), S, z, "bf16")
        q64 = oracle.as_f64(qbits, "bf16")
        k64 = oracle.as_f64(kbits[:, w0 * T:w1 * T], "bf16")
        v64 = oracle.as_f64(vbits[:, w0 * T:w1 * T], "bf16")
        sel_ref, s32 = oracle.select(q64, k64, B, K)
        sel_dev = sel.cpu().numpy()
        differ = compare_sel(sel_dev, sel_ref, s32, K)
        blocks = sorted({(int(rng.integers(H)), int(rng.integers(74))) for _ in range(3)} |
                        {(t % H, 73)} | {(int(h), int(i)) for h, i in zip(*np.nonzero(differ))})
        ref = oracle.attend_with_sel(q64, k64, v64, reference_selection(sel_dev, sel_ref, differ),
                                     S, z, B, blocks=blocks)
        stats = compare_out(host_f64(out), ref, "bf16")
        if t % 10 == 0 or t == n_steps - 1:
            print(f"step {t}: window {w0}-{w1} K={K} S fro={fro:.2e} z rel={zrel:.2e} "
                  f"out {stats} ties={int(differ.sum())} ({time.time() - t0:.0f}s)", flush=True)
    assert st.next_ev_index == (F - W) * T
    # The running float64 state equals one batch absorb of every evicted token.
    Sb, zb = oracle.state_init(H, d)
    for h0 in range(0, H, 4):  # a few heads at a time to bound host memory
        hs = slice(h0, h0 + 4)
        Sh, zh = oracle.state_init(4, d)
        oracle.absorb(Sh, zh, oracle.as_f64(kbits[hs, :(F - W) * T], "bf16"),
                      oracle.as_f64(vbits[hs, :(F - W) * T], "bf16"))
        Sb[hs], zb[hs] = Sh, zh
    assert np.abs(Sb - S).max() <= 1e-9 * np.abs(Sb).max()
    assert np.abs(zb - z).max() <= 1e-12 * np.abs(zb).max()
    state_close(host_f64(st.S), host_f64(st.z), Sb, zb, "bf16")
