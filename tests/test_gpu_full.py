"""The five reference workloads at full size, in the launch configuration the
benchmark times.  Sampled rows are checked element by element against the
oracle (scores and Top-K bit-exact, attention within the bar); every row is
checked for the properties that hold at any size."""
import numpy as np
import pytest
import torch

import dsa_synth
import oracle
from tests.helpers import (assert_attention, assert_idx_rows_valid, assert_topk_consistent,
                           gpu_decode, gpu_prefill, oracle_decode_sampled, say)

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)
    yield
    torch.cuda.empty_cache()


def sample_seqs(wl, k):
    L = np.asarray(wl.seq_lens)
    picks = [0, wl.n_seq - 1, int(L.argmax()), int(L.argmin())]
    rng = np.random.default_rng(wl.seed)
    picks += rng.integers(0, wl.n_seq, size=k).tolist()
    out = []
    for p in picks:
        if p not in out:
            out.append(p)
    return out[:k]


@pytest.mark.parametrize("n,k", [(1, 1), (2, 3), (4, 3), (5, 2)])
def test_full_decode(n, k):
    wl = dsa_synth.workload(n)
    say(f"[full decode] {wl.name}: B={wl.n_q} sum(L)={sum(wl.seq_lens)}")
    dc = dsa_synth.device_case(wl)
    step = gpu_decode(dc)
    assert_idx_rows_valid(step.idx, wl.seq_lens, wl.topk)
    assert_topk_consistent(step.scores, step.idx, wl.seq_lens, wl.topk)
    seqs = sample_seqs(wl, k)
    say(f"   oracle on sequences {seqs}")
    ref = oracle_decode_sampled(wl, seqs)
    for b, (sc, idx, out, lse) in ref.items():
        L = wl.seq_lens[b]
        g_sc = step.scores[b, :L].cpu().numpy()
        np.testing.assert_array_equal(g_sc, sc[:L], err_msg=f"scores of sequence {b}")
        np.testing.assert_array_equal(step.idx[b].cpu().numpy(), idx, err_msg=f"idx {b}")
        mx, mn = assert_attention(step.out[b], step.lse[b], out, lse, f"{wl.name} seq {b}")
        say(f"   seq {b} (L={L}): exact scores and Top-K, attention max|err| {mx:.2e}")
    del dc, step


def test_full_prefill():
    wl = dsa_synth.workload(3)
    T = wl.seq_lens[0]
    say(f"[full prefill] {wl.name}: T={T}")
    dc = dsa_synth.device_case(wl)
    step = gpu_prefill(dc)
    n_valid = np.arange(1, T + 1)
    assert_idx_rows_valid(step.idx, n_valid, wl.topk)
    rows_chk = np.random.default_rng(3).choice(T, 256, replace=False)
    assert_topk_consistent(step.scores[rows_chk], step.idx[rows_chk], n_valid[rows_chk], wl.topk)
    rows = np.array([0, 1, 100, 2046, 2047, 2048, 2049, 4095, 6000, 8190, 8191], dtype=np.int32)
    hc = dsa_synth.host_case(wl)
    sc = oracle.index_score(hc.k_idx, hc.block_table, wl.block_size, hc.q_idx[rows], hc.w[rows],
                            np.zeros(len(rows), np.int32), rows, ld=T)
    idx = oracle.topk(sc, rows + 1, wl.topk)
    out, lse = oracle.sparse_attn(hc.kv, None, hc.block_table, wl.block_size, hc.q[rows],
                                  np.zeros(len(rows), np.int32), idx, wl.sm_scale, d_v=wl.d_v)
    g_sc = step.scores[rows.tolist()].cpu().numpy()
    for r, t in enumerate(rows):
        assert np.array_equal(g_sc[r, :t + 1], sc[r, :t + 1]), f"scores row {t}"
    np.testing.assert_array_equal(step.idx[rows.tolist()].cpu().numpy(), idx)
    mx, mn = assert_attention(step.out[rows.tolist()], step.lse[rows.tolist()], out, lse,
                              wl.name)
    say(f"   rows {rows.tolist()}: exact scores and Top-K, attention max|err| {mx:.2e}")
    del dc, step
