"""hf_attend_chunk_noalloc (the allocation-free entry point, scratch in a static device
array) against hf_attend_chunk of a state with the same S and z, through the C ABI:
outputs and selections equal bit for bit, on two calls in a row where the second is
smaller (the scratch keeps the first call's contents)."""

import ctypes

import numpy as np
import pytest
import torch

import synth
from synth.inputs import frame_block

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import hybrid_linear_block_amd as hla  # the HIP library must load: no fallback path
else:
    hla = None


def _draw(seed, stream, H, n, d, dt):
    x = frame_block(seed, stream, 0, H, n, d, 1.0 / np.sqrt(d))
    if dt == torch.bfloat16:
        bits = synth.bf16_bits(x)
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(x).cuda()


def _bits(t):
    return t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32)


@pytest.mark.parametrize("dt,d,B", [(torch.bfloat16, 128, 64), (torch.bfloat16, 64, 64),
                                    (torch.float32, 64, 16)])
def test_noalloc_matches_attend_chunk(dt, d, B):
    H, n_ev = 4, 700
    sizes = [(1560 * 3, 1560 * 9, 55), (333, 1000, 3)]  # the second call is smaller
    if B == 16:
        sizes = [(600, 2000, 30), (100, 150, 4)]
    kev, vev = _draw(5, 1, H, n_ev, d, dt), _draw(5, 2, H, n_ev, d, dt)
    n_q0, n_kv0, k0 = sizes[0]
    st = hla.HybridAttentionState(H, d, B, dt, max_n_q=n_q0, max_n_kv=n_kv0, max_n_ev=n_ev,
                                  max_top_k=k0)
    st.absorb_evicted(kev, vev)
    for call, (n_q, n_kv, K) in enumerate(sizes):
        print(f"call {call}: {dt} d={d} B={B} n_q={n_q} n_kv={n_kv} K={K}", flush=True)
        q = _draw(10 + call, 3, H, n_q, d, dt)
        k = _draw(10 + call, 4, H, n_kv, d, dt)
        v = _draw(10 + call, 5, H, n_kv, d, dt)
        nqb = -(-n_q // B)
        sel_ref = torch.empty((H, nqb, K), dtype=torch.int32, device="cuda")
        out_ref = st.attend_chunk(q, k, v, K, sel_out=sel_ref)
        out = torch.empty_like(q)
        sel = torch.full((H, nqb, K), -1, dtype=torch.int32, device="cuda")
        stream = torch.cuda.current_stream().cuda_stream
        r = hla.hf_attend_chunk_noalloc(st.cfg, st.S.data_ptr(), st.z.data_ptr(), q.data_ptr(),
                                        n_q, n_q * d, k.data_ptr(), v.data_ptr(), n_kv, n_kv * d,
                                        K, out.data_ptr(), n_q * d, sel.data_ptr(), stream)
        assert r == hla.HF_OK, hla.hf_status_string(r)
        out2 = torch.empty_like(q)  # and with the selection kept in the scratch
        r = hla.hf_attend_chunk_noalloc(st.cfg, st.S.data_ptr(), st.z.data_ptr(), q.data_ptr(),
                                        n_q, n_q * d, k.data_ptr(), v.data_ptr(), n_kv, n_kv * d,
                                        K, out2.data_ptr(), n_q * d, 0, stream)
        assert r == hla.HF_OK, hla.hf_status_string(r)
        torch.cuda.synchronize()
        assert torch.equal(sel, sel_ref)
        assert torch.equal(_bits(out), _bits(out_ref))
        assert torch.equal(_bits(out2), _bits(out_ref))
    st.close()
