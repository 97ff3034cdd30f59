"""Head-aware ragged windows (hf_attend_ragged) on one MI355X against the oracle.

Head h attends its own window, stored flattened after the previous head's, with its
own top-K ("Resumen Tecnico: Pyramid Forcing", 3: variable-length per-head KV caches as
flattened sequences with boundary indices, attention without padding). Checked: the
Wan-like layer with a pyramid of window lengths (9, 6 and 4 frames) against
oracle.attend_ragged (each head's selection with the near-tie rule, the state, sampled
outputs); small cases with ragged tails and a window shorter than one block, compared
in full; equal windows bit for bit equal to hf_attend_chunk over the dense layout; the
argument checks.
"""

import numpy as np
import pytest
import torch

import oracle
import synth
from synth.inputs import frame_block

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import hybrid_linear_block_amd as hla  # the HIP library must load: no fallback path
else:
    hla = None
from hfutil import (compare_out, compare_sel, dev_bf16, dev_f32, host_f64,  # noqa: E402
                    reference_selection, state_close)

TORCH_DT = {"bf16": torch.bfloat16, "f32": torch.float32}


def _check(q64, kf64, vf64, off, S, z, B, top_ks, out, sel, dtype, blocks=None):
    """Per head: selection (near-tie rule), then outputs over the accepted sets."""
    H = q64.shape[0]
    _, sels_ref, s32s = oracle.attend_ragged(q64, kf64, vf64, off, S, z, B, top_ks,
                                             blocks=[(0, 0)] if blocks is not None else None)
    sel = sel.cpu().numpy()
    ref = np.full(q64.shape, np.nan)
    n_diff = 0
    for h in range(H):
        K = top_ks[h]
        dev = sel[h:h + 1, :, :K]
        differ = compare_sel(dev, sels_ref[h][None], s32s[h][None], K)
        n_diff += int(differ.sum())
        use = reference_selection(dev, sels_ref[h][None], differ)
        o0, o1 = int(off[h]), int(off[h + 1])
        hb = None if blocks is None else [(0, i) for hh, i in blocks if hh == h] + \
            [(0, int(i)) for i in np.nonzero(differ[0])[0]]
        if hb == []:
            continue
        ref[h] = oracle.attend_with_sel(q64[h:h + 1], kf64[None, o0:o1], vf64[None, o0:o1], use,
                                        S[h:h + 1], z[h:h + 1], B, blocks=hb)[0]
    return compare_out(host_f64(out), ref, dtype), n_diff


def test_wan_layer_ragged_pyramid():
    wl = synth.WORKLOADS["ragged_heads_bf16"]
    H, d, B, T = wl.heads, wl.head_dim, wl.block, wl.frame_tokens
    inp = synth.ragged_layer_inputs(77)
    off = inp["offsets"]
    lens = np.diff(off)
    top_ks = [synth.top_k_count(wl.top_k_frac, -(-int(n) // B)) for n in lens]
    qd, kfd, vfd = dev_bf16(inp["q"]), dev_bf16(inp["k_flat"]), dev_bf16(inp["v_flat"])
    ked, ved = dev_bf16(inp["k_ev"]), dev_bf16(inp["v_ev"])
    n_q = qd.shape[1]
    st = hla.HybridAttentionState(H, d, B, torch.bfloat16, max_n_q=n_q, max_n_kv=int(lens.max()),
                                  max_n_ev=ked.shape[1], max_top_k=max(top_ks))
    st.absorb_evicted(ked, ved)
    nqb = -(-n_q // B)
    sel = torch.full((H, nqb, max(top_ks)), -1, dtype=torch.int32, device="cuda")
    out = st.attend_ragged(qd, kfd, vfd, off, top_ks, sel_out=sel)
    torch.cuda.synchronize()
    S, z = oracle.state_init(H, d)
    oracle.absorb(S, z, oracle.as_f64(inp["k_ev"], "bf16"), oracle.as_f64(inp["v_ev"], "bf16"))
    state_close(host_f64(st.S), host_f64(st.z), S, z, "bf16")
    rng = np.random.default_rng(3)
    blocks = {(h, nqb - 1) for h in range(H)}
    while len(blocks) < H + 24:
        blocks.add((int(rng.integers(H)), int(rng.integers(nqb))))
    stats, n_diff = _check(oracle.as_f64(inp["q"], "bf16"), oracle.as_f64(inp["k_flat"], "bf16"),
                           oracle.as_f64(inp["v_flat"], "bf16"), off, S, z, B, top_ks, out, sel,
                           "bf16", blocks=sorted(blocks))
    print("ragged pyramid", top_ks, stats, "near-tie rows:", n_diff, flush=True)


@pytest.mark.parametrize("dt,d,B,lens,top_ks", [
    ("bf16", 128, 64, [600, 200, 37, 333], [3, 2, 1, 5]),  # ragged tails; one window < 1 block
    ("bf16", 64, 64, [130, 1000, 64], [2, 7, 1]),
    ("f32", 64, 16, [150, 33, 80], [4, 2, 5]),
])
def test_ragged_small_full_compare(dt, d, B, lens, top_ks):
    H, n_q = len(lens), 150
    off = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    std = 1.0 / np.sqrt(d)
    draws = {}
    for name, stream, n in (("q", 1, None), ("k", 2, int(off[-1])), ("v", 3, int(off[-1])),
                            ("ke", 4, None), ("ve", 5, None)):
        shape_h, shape_n = (1, n) if n is not None else (H, n_q if name == "q" else 40)
        x = frame_block(9 + H, stream, 0, shape_h, shape_n, d, std)
        x = x[0] if n is not None else x
        if dt == "bf16":
            bits = synth.bf16_bits(x)
            draws[name] = (dev_bf16(bits), oracle.as_f64(bits, "bf16"))
        else:
            draws[name] = (dev_f32(x), x.astype(np.float64))
    st = hla.HybridAttentionState(H, d, B, TORCH_DT[dt], max_n_q=n_q, max_n_kv=max(lens),
                                  max_n_ev=40, max_top_k=max(top_ks))
    st.absorb_evicted(draws["ke"][0], draws["ve"][0])
    sel = torch.full((H, -(-n_q // B), max(top_ks)), -1, dtype=torch.int32, device="cuda")
    out = st.attend_ragged(draws["q"][0], draws["k"][0], draws["v"][0], off, top_ks, sel_out=sel)
    torch.cuda.synchronize()
    S, z = oracle.state_init(H, d)
    oracle.absorb(S, z, draws["ke"][1], draws["ve"][1])
    stats, n_diff = _check(draws["q"][1], draws["k"][1], draws["v"][1], off, S, z, B, top_ks, out,
                           sel, dt)
    print(dt, lens, stats, "near-tie rows:", n_diff, flush=True)


@pytest.mark.parametrize("dt,d,B", [("bf16", 128, 64), ("f32", 64, 16)])
def test_ragged_equal_windows_match_attend_chunk_bitwise(dt, d, B):
    H, n_q, n_kv, K = 4, 300, 1000, 5
    g = torch.Generator(device="cuda").manual_seed(11)
    tdt = TORCH_DT[dt]
    mk = lambda *s: (torch.randn(s, generator=g, device="cuda") / d ** 0.5).to(tdt)  # noqa
    q, k, v = mk(H, n_q, d), mk(H, n_kv, d), mk(H, n_kv, d)
    args = dict(max_n_q=n_q, max_n_kv=n_kv, max_n_ev=8, max_top_k=K)
    a = hla.HybridAttentionState(H, d, B, tdt, **args)
    b = hla.HybridAttentionState(H, d, B, tdt, **args)
    nqb = -(-n_q // B)
    sa = torch.empty((H, nqb, K), dtype=torch.int32, device="cuda")
    sb = torch.empty((H, nqb, K), dtype=torch.int32, device="cuda")
    oa = a.attend_chunk(q, k, v, K, sel_out=sa)
    ob = b.attend_ragged(q, k.reshape(-1, d), v.reshape(-1, d), [h * n_kv for h in range(H + 1)],
                         [K] * H, sel_out=sb)
    torch.cuda.synchronize()
    bits = lambda t: t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32)  # noqa
    assert torch.equal(sa, sb)
    assert torch.equal(bits(oa), bits(ob))


def test_ragged_argument_checks():
    H, d, B = 3, 128, 64
    st = hla.HybridAttentionState(H, d, B, torch.bfloat16, max_n_q=64, max_n_kv=256, max_n_ev=8,
                                  max_top_k=4)
    q = torch.zeros((H, 64, d), dtype=torch.bfloat16, device="cuda")
    kf = torch.zeros((600, d), dtype=torch.bfloat16, device="cuda")
    ok_off, ok_k = [0, 100, 300, 500], [2, 4, 4]
    st.attend_ragged(q, kf, kf, ok_off, ok_k)
    for off, tk in (([0, 100, 300, 600], ok_k),   # a window above max_n_kv (300 rows)
                    ([0, 100, 100, 300], ok_k),   # an empty window
                    (ok_off, [2, 5, 4]),          # top_k above max_top_k
                    (ok_off, [3, 4, 4]),          # top_k above the head's 2 key blocks
                    (ok_off, [0, 4, 4])):
        with pytest.raises(hla.HfError) as ei:
            st.attend_ragged(q, kf, kf, off, tk)
        assert ei.value.status == hla.HF_ERR_INVALID_ARG, (off, tk)
    torch.cuda.synchronize()
