"""The allocation-free decode attention (dsa_sparse_attn_decode_static)
against the workspace entry point (dsa_sparse_attn_decode) through the C
ABI: two calls in a row, the second one smaller, each checked element by
element (the two share their kernels and split plan, so the bits agree; the
attention bars are checked too)."""
import numpy as np
import pytest
import torch

import dsa_synth
import sparse_attention_long_dsa_amd as dsa
from tests.helpers import assert_attention, say

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)
    dsa.lib()


def _case(wl):
    dc = dsa_synth.device_case(wl)
    cache = dsa.Cache(dc.kv, dc.k_idx, dc.block_table, dc.seq_lens, v=dc.v, d_v=wl.d_v)
    st = dsa.DecodeStep(cache, wl.n_q, wl.H, wl.H_idx, wl.topk, max(wl.seq_lens), wl.d_v)
    st(dc.q, dc.q_idx, dc.w, wl.sm_scale)  # indices from the regular path
    out_ref, lse_ref = st.out.clone(), st.lse.clone()
    out, lse = dsa.sparse_attn_decode_static(cache, dc.q, st.idx, wl.sm_scale)
    torch.cuda.synchronize()
    assert torch.equal(out, out_ref) and torch.equal(lse, lse_ref), "bits differ"
    assert_attention(out, lse, out_ref.float().cpu().numpy(), lse_ref.cpu().numpy(), wl.name)
    return dc, st


def test_static_scratch_matches_workspace_path_twice():
    big = dsa_synth.latent("static_big", "decode", [3000, 20000, 40000, 70000], seed=61,
                           topk=2048)
    small = dsa_synth.latent("static_small", "decode", [900, 5000], seed=62, topk=512)
    tiny = dsa_synth.small_mqa("static_tiny", "decode", [1024, 77], seed=63, topk=64)
    for wl in (big, small, tiny):
        say(f"[static scratch] {wl.name}: lens {wl.seq_lens}")
        _case(wl)
    say("   ok: bitwise equal to the workspace entry point on consecutive calls")
