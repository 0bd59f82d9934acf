"""The five reference workloads at full size, in the launch configuration the
benchmark times, against the oracle.

Decode (workloads 1, 2, 4, 5): every sequence of the batch is compared with
the oracle -- scores and Top-K indices bit for bit, attention within the bars
-- and the step is run twice to check that its results are bitwise
reproducible.  Prefill (workload 3, 8192 tokens): rows 0..511 and every 16th
row after them (and the last row) are compared with the oracle the same way;
every row is checked for the properties that hold at any size.  Each test
prints its worst attention error and the share of the bars it uses."""
import numpy as np
import pytest
import torch

import dsa_synth
import oracle
import sparse_attention_long_dsa_amd as dsa
from tests.helpers import (assert_attention, assert_idx_rows_valid, assert_topk_consistent,
                           attention_margin, gpu_decode, gpu_prefill, oracle_decode_rows, say)

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)
    yield
    torch.cuda.empty_cache()


@pytest.mark.parametrize("n", [1, 2, 4, 5])
def test_full_decode(n):
    wl = dsa_synth.workload(n)
    say(f"[full decode] {wl.name}: B={wl.n_q} sum(L)={sum(wl.seq_lens)}")
    dc = dsa_synth.device_case(wl)
    step = gpu_decode(dc)
    first = (step.idx.clone(), step.out.clone(), step.lse.clone())
    step(dc.q, dc.q_idx, dc.w, wl.sm_scale)  # the same step again: bitwise equal
    torch.cuda.synchronize()
    assert torch.equal(first[0], step.idx), "Top-K differs between two runs"
    assert torch.equal(first[1], step.out) and torch.equal(first[2], step.lse), \
        "attention differs between two runs"
    assert_idx_rows_valid(step.idx, wl.seq_lens, wl.topk)
    g_idx = step.idx.cpu().numpy()
    g_out = step.out.float().cpu().numpy()
    g_lse = step.lse.cpu().numpy()
    worst_mx = worst_mn = 0.0
    for b in range(wl.n_seq):
        L = wl.seq_lens[b]
        sc, idx, out, lse = oracle_decode_rows(wl, [b])[b]
        g_sc = step.scores[b, :L].cpu().numpy()
        np.testing.assert_array_equal(g_sc, sc[:L], err_msg=f"scores of sequence {b}")
        np.testing.assert_array_equal(g_idx[b], idx, err_msg=f"Top-K of sequence {b}")
        mx, mn = assert_attention(g_out[b], g_lse[b], out, lse, f"{wl.name} seq {b}")
        worst_mx, worst_mn = max(worst_mx, mx), max(worst_mn, mn)
    fm, fn = attention_margin(worst_mx, worst_mn)
    say(f"   all {wl.n_seq} sequences: scores and Top-K exact, run twice bitwise equal; "
        f"worst attention max|err| {worst_mx:.2e} ({100 * fm:.0f}% of 1e-2), "
        f"worst mean|err| {worst_mn:.2e} ({100 * fn:.0f}% of 1e-3)")
    del dc, step


def test_full_prefill():
    wl = dsa_synth.workload(3)
    T = wl.seq_lens[0]
    say(f"[full prefill] {wl.name}: T={T}")
    dc = dsa_synth.device_case(wl)
    step = gpu_prefill(dc)
    n_valid = np.arange(1, T + 1)
    assert_idx_rows_valid(step.idx, n_valid, wl.topk)
    rows = np.array(sorted(set(range(512)) | set(range(512, T, 16)) | {T - 1}), dtype=np.int32)
    say(f"   oracle on {len(rows)} rows (0..511, every 16th after, the last)")
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
    g_out = step.out[rows.tolist()].float().cpu().numpy()
    mx, mn = assert_attention(g_out, step.lse[rows.tolist()], out, lse, wl.name)
    per_row = np.abs(g_out - out).reshape(len(rows), -1).max(axis=1)
    w = int(np.argmax(per_row))
    fm, fn = attention_margin(mx, mn)
    say(f"   scores and Top-K exact on every compared row; attention max|err| {mx:.2e} "
        f"({100 * fm:.0f}% of 1e-2, worst at row {rows[w]}), mean|err| {mn:.2e} "
        f"({100 * fn:.0f}% of 1e-3)")
    # rows not compared with the oracle: the selection is consistent with the
    # GPU scores (kept >= dropped, lowest positions among ties)
    rest = np.setdiff1d(np.arange(T), rows)
    pick = np.random.default_rng(3).choice(rest, 256, replace=False)
    assert_topk_consistent(step.scores[pick], step.idx[pick], n_valid[pick], wl.topk)
    # the fused selection (no score matrix) gives the same kept positions on
    # every one of the 8192 rows
    cache = dsa.Cache(dc.kv, dc.k_idx, dc.block_table, dc.seq_lens, v=dc.v, d_v=wl.d_v)
    fused = dsa.index_topk_prefill(cache, dc.q_idx, dc.w, step.q_seq, step.q_pos, wl.topk)
    torch.cuda.synchronize()
    assert torch.equal(fused, step.idx), "fused prefill selection differs on some row"
    say("   fused index + Top-K equal on all rows")
    del dc, step
