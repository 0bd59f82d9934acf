"""GPU parity: the HIP path through the C ABI against the oracle, element by
element on seeded inputs, at sizes the oracle finishes in seconds (several
tiles, ragged tails, both Top-K paths, both shape families), plus edge cases.
"""
import dataclasses

import numpy as np
import pytest
import torch

import dsa_synth
import oracle
import sparse_attention_long_dsa_amd as dsa
from tests.helpers import (assert_attention, assert_idx_rows_valid, assert_topk_consistent,
                           gpu_decode, gpu_prefill, say)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)
    dsa.lib()


def check_decode(wl, sample_rows=None, rel=False):
    say(f"[decode] {wl.name} lens={wl.seq_lens[:6]}... K={wl.topk} bs={wl.block_size}")
    dc = dsa_synth.device_case(wl)
    step = gpu_decode(dc)
    hc = dsa_synth.host_case(wl)
    sc, idx, out, lse = oracle.decode_step(hc)
    g_sc = step.scores.cpu().numpy()
    for b, L in enumerate(wl.seq_lens):
        np.testing.assert_array_equal(g_sc[b, :L], sc[b, :L], err_msg=f"scores row {b}")
    np.testing.assert_array_equal(step.idx.cpu().numpy(), idx)
    mx, mn = assert_attention(step.out, step.lse, out, lse, wl.name, rel=rel)
    # the separate index-score and Top-K calls give the same bits as the fused call
    sep = dsa.DecodeStep(step.cache, wl.n_q, wl.H, wl.H_idx, wl.topk, max(wl.seq_lens), wl.d_v,
                         fused=False)
    sep.select(dc.q_idx, dc.w)
    torch.cuda.synchronize()
    assert torch.equal(sep.idx, step.idx), "separate calls differ from the fused call"
    for b, L in enumerate(wl.seq_lens):
        assert torch.equal(sep.scores[b, :L], step.scores[b, :L])
    # attention alone, fed the oracle's indices
    o2, l2 = dsa.sparse_attn_decode(step.cache, dc.q, torch.from_numpy(idx).cuda(), wl.sm_scale)
    assert_attention(o2, l2, out, lse, wl.name + " (oracle idx)", rel=rel)
    say(f"   ok: max|err| {mx:.2e} mean|err| {mn:.2e}")
    return dc, step


def test_tiny_decode_chain_and_determinism():
    wl = dsa_synth.workload(1)
    dc, step = check_decode(wl)
    first = (step.idx.clone(), step.out.clone(), step.lse.clone())
    step(dc.q, dc.q_idx, dc.w, wl.sm_scale)
    torch.cuda.synchronize()
    assert torch.equal(first[0], step.idx)
    assert torch.equal(first[1], step.out) and torch.equal(first[2], step.lse)


def test_small_family_ragged_decode():
    wl = dsa_synth.small_mqa("small_ragged", "decode", [1, 17, 64, 65, 1000, 2500], seed=21,
                             topk=64, block_size=16)
    check_decode(wl)


def test_small_family_many_splits():
    # Top-K 2048 over one or two sequences splits each query's kept rows
    # over up to 64 workgroups: the split merge takes its general path
    # (more splits than its register-resident fast path holds)
    wl = dsa_synth.small_mqa("small_many_splits", "decode", [2100, 5000], seed=27, topk=2048,
                             block_size=16)
    check_decode(wl)


def test_latent_decode_empty_and_tiny_sequences():
    # one latent decode batch through the fused chain: a sequence with no
    # cached position (nothing to select: idx all -1, out 0, lse -inf), one
    # and two positions, a 16-position group and one past it, rows around K
    wl = dsa_synth.latent("latent_tiny", "decode", [0, 1, 2, 16, 17, 2047, 2048, 2049], seed=91,
                          topk=2048)
    _, step = check_decode(wl)
    assert torch.all(step.idx[0] == -1)
    assert torch.all(step.out[0] == 0) and torch.all(torch.isneginf(step.lse[0]))
    assert torch.all(step.idx[1, 1:] == -1) and step.idx[1, 0].item() == 0


def test_latent_decode_short_rows():
    # rows <= 16384 take the one-workgroup-per-row Top-K path
    wl = dsa_synth.latent("latent_short", "decode", [700, 2048, 2049, 5000, 9001], seed=22,
                          topk=2048)
    check_decode(wl)


def test_latent_decode_long_rows():
    # rows > 16384 take the multi-workgroup Top-K path
    wl = dsa_synth.latent("latent_long", "decode", [1500, 17000, 40000], seed=23, topk=2048)
    check_decode(wl)


def test_latent_decode_odd_K_and_block():
    wl = dsa_synth.latent("latent_oddK", "decode", [37, 300, 20001], seed=24, topk=37,
                          block_size=16)
    check_decode(wl)


def test_latent_decode_peaked_softmax():
    # sm_scale 1: logits spread with std ~24, so a later tile's maximum passes
    # the first tile's by far more than the fp16 weight range and the
    # attention blocks run their tiles again from the true maximum
    wl = dataclasses.replace(
        dsa_synth.latent("latent_peaked", "decode", [900, 5000, 20000], seed=26, topk=2048),
        sm_scale=1.0)
    check_decode(wl, rel=True)


def test_latent_decode_wide_batch():
    # more than 1024 sequences: the index score takes its per-(sequence,
    # chunk) kernel instead of the token-balanced one
    lens = [int(x) for x in np.random.default_rng(28).integers(1, 300, size=1100)]
    wl = dsa_synth.latent("latent_wide", "decode", lens, seed=28, topk=64, block_size=16)
    check_decode(wl)


def test_block_table_invariance():
    a = dsa_synth.latent("inv", "decode", [3000, 20000], seed=25, topk=512)
    b = dsa_synth.latent("inv", "decode", [3000, 20000], seed=25, topk=512, table_seed=99)
    assert not np.array_equal(dsa_synth.block_table(a), dsa_synth.block_table(b))
    sa = gpu_decode(dsa_synth.device_case(a))
    sb = gpu_decode(dsa_synth.device_case(b))
    assert torch.equal(sa.idx, sb.idx)
    assert torch.equal(sa.out, sb.out)


def check_prefill(wl, pos0=0, T=None, rel=False):
    T = wl.seq_lens[0] - pos0 if T is None else T
    say(f"[prefill] {wl.name} pos0={pos0} T={T} K={wl.topk}")
    dc = dsa_synth.device_case(wl)
    step = gpu_prefill(dc, pos0=pos0, T=T)
    hc = dsa_synth.host_case(wl)
    rows = np.arange(pos0, pos0 + T)
    sc = oracle.index_score(hc.k_idx, hc.block_table, wl.block_size, hc.q_idx[rows], hc.w[rows],
                            np.zeros(T, np.int32), rows.astype(np.int32), ld=pos0 + T)
    idx = oracle.topk(sc, rows + 1, wl.topk)
    out, lse = oracle.sparse_attn(hc.kv, hc.v, hc.block_table, wl.block_size, hc.q[rows],
                                  np.zeros(T, np.int32), idx, wl.sm_scale, d_v=wl.d_v)
    g_sc = step.scores.cpu().numpy()
    for t in range(T):
        n = pos0 + t + 1
        assert np.array_equal(g_sc[t, :n], sc[t, :n]), f"scores row {t}"
    np.testing.assert_array_equal(step.idx.cpu().numpy(), idx)
    mx, mn = assert_attention(step.out, step.lse, out, lse, wl.name, rel=rel)
    if _fused_applies(wl, pos0 + T):
        check_fused_prefill(dc, torch.arange(pos0, pos0 + T, dtype=torch.int32, device="cuda"),
                            torch.zeros(T, dtype=torch.int32, device="cuda"), idx)
    say(f"   ok: max|err| {mx:.2e} mean|err| {mn:.2e}")


def _fused_applies(wl, max_pos_plus_one):
    """dsa_index_topk_prefill covers the (64, 128) indexer, rows <= 8192."""
    return wl.H_idx == 64 and wl.d_idx == 128 and max_pos_plus_one <= 8192


def check_fused_prefill(dc, q_pos, q_seq, idx_ref, rows=None):
    """The fused prefill selection (no score matrix) on the same queries: the
    kept positions equal the oracle's, exactly."""
    wl = dc.wl
    T = q_pos.shape[0]
    cache = dsa.Cache(dc.kv, dc.k_idx, dc.block_table, dc.seq_lens, v=dc.v, d_v=wl.d_v)
    if rows is None:
        q_idx, w = dc.q_idx[q_pos.long()].contiguous(), dc.w[q_pos.long()].contiguous()
    else:
        q_idx, w = rows
    got = dsa.index_topk_prefill(cache, q_idx, w, q_seq, q_pos, wl.topk)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(got.cpu().numpy(), idx_ref, err_msg="fused prefill selection")
    say(f"   fused index + Top-K: {T} rows exact")


def test_latent_prefill():
    check_prefill(dsa_synth.latent("prefill_latent", "prefill", [700], seed=31, topk=256))


def test_latent_prefill_chunk():
    check_prefill(dsa_synth.latent("prefill_chunk", "prefill", [700], seed=32, topk=200),
                  pos0=300, T=400)


def test_latent_prefill_block_size_16():
    check_prefill(dsa_synth.latent("prefill_bs16", "prefill", [500], seed=37, topk=100,
                                   block_size=16), pos0=37, T=463)


def test_latent_prefill_chunk_past_8192_keys():
    # the prefill indexer covers at most 8192 keys per workgroup: positions
    # 9000..9039 see two key chunks (the second one partial)
    check_prefill(dsa_synth.latent("prefill_long", "prefill", [9040], seed=35, topk=2048),
                  pos0=9000, T=40)


def test_latent_prefill_single_query():
    check_prefill(dsa_synth.latent("prefill_one", "prefill", [300], seed=36, topk=256),
                  pos0=299, T=1)


def test_latent_prefill_peaked_softmax():
    wl = dsa_synth.latent("prefill_peaked", "prefill", [600], seed=34, topk=256)
    check_prefill(dataclasses.replace(wl, sm_scale=1.0), rel=True)


def test_small_family_prefill():
    check_prefill(dsa_synth.small_mqa("prefill_small", "prefill", [333], seed=33, topk=64,
                                      block_size=16))


# ----------------------------------------------------------------------------- Top-K alone

def _topk_case(scores, n_valid, K):
    d_sc = torch.from_numpy(scores).cuda()
    d_nv = torch.from_numpy(np.asarray(n_valid, np.int32)).cuda()
    got = dsa.topk(d_sc, K, n_valid=d_nv)
    torch.cuda.synchronize()
    want = oracle.topk(scores, np.asarray(n_valid, np.int32), K)
    np.testing.assert_array_equal(got.cpu().numpy(), want)
    assert_idx_rows_valid(got, n_valid, K)


@pytest.mark.parametrize("ld", [3000, 50000, 50001])
def test_topk_ties_and_special_rows(ld):
    rng = np.random.default_rng(ld)
    rows = [
        np.full(ld, 7.0),                                  # all equal
        rng.integers(0, 2, ld).astype(np.float64),         # two values
        np.arange(ld, dtype=np.float64),                   # increasing
        np.arange(ld, dtype=np.float64)[::-1].copy(),      # decreasing
        rng.integers(-50, 50, ld).astype(np.float64),      # negative and positive ties
        np.where(rng.random(ld) < 0.5, 0.0, -0.0),         # signed zeros compare equal
        rng.normal(size=ld) * 1e30,                        # wide exponents
        rng.normal(size=ld).astype(np.float32).astype(np.float64) * 1e-30,
    ]
    scores = np.stack(rows).astype(np.float32)
    n_valid = [ld, ld - 1, ld, 2100, ld // 2, ld, 2049, ld]
    for K in (1, 2048, 777):
        _topk_case(scores, n_valid, K)


def test_topk_long_rows_where_pruning_falls_back():
    """Long rows whose pruned candidate list misleads: a list longer than the
    in-LDS capacity (two values, heavy ties) and a list shorter than K (high
    scores placed exactly on the sampled positions - groups of four from
    floor(4 g n / 8192) - so the sample overrates the bound).  Both must still
    be exact."""
    n = 50000
    rng = np.random.default_rng(7)
    planted = np.zeros(n)
    starts = (np.arange(175, dtype=np.int64) * 4 * n) // 8192
    planted[(starts[:, None] + np.arange(4)).ravel()] = 1.0
    rows = [rng.integers(0, 2, n).astype(np.float64), planted,
            planted + rng.integers(0, 3, n) * 1e-3]
    scores = np.stack(rows).astype(np.float32)
    _topk_case(scores, [n, n, n], 2048)


def test_topk_short_rows_with_fewer_candidates_than_K():
    scores = np.random.default_rng(5).integers(0, 9, (6, 4096)).astype(np.float32)
    _topk_case(scores, [0, 1, 63, 64, 65, 4096], 64)


def test_topk_causal_rows():
    T = 3000
    scores = np.random.default_rng(6).integers(0, 30, (T, T)).astype(np.float32)
    got = dsa.topk(torch.from_numpy(scores).cuda(), 128, causal_base=0)
    want = oracle.topk(scores, np.arange(1, T + 1, dtype=np.int32), 128)
    np.testing.assert_array_equal(got.cpu().numpy(), want)


# ----------------------------------------------------------------------------- cache write

def _bf16_rows(rng, n, d):
    x = torch.from_numpy(rng.normal(size=(n, d)).astype(np.float32)).to(torch.bfloat16)
    return x.view(torch.int16).numpy().view(np.uint16)


def _cache_write_case(wl, seed):
    say(f"[cache write] {wl.name}")
    rng = np.random.default_rng(seed)
    dc = dsa_synth.device_case(wl)
    hc = dsa_synth.host_case(wl)
    cap = wl.max_blocks * wl.block_size
    own = [nb * wl.block_size for nb in wl.blocks_per_seq]  # slots of each sequence's own blocks
    # distinct slots of both sequences, plus tokens the call must skip
    picks = [(0, int(p)) for p in rng.choice(own[0], 40, replace=False)] + \
            [(1, int(p)) for p in rng.choice(own[1], 40, replace=False)]
    picks += [(2, 0), (-1, 3), (0, -5), (1, cap)]
    seq = np.array([b for b, _ in picks], np.int32)
    pos = np.array([p for _, p in picks], np.int32)
    n = len(picks)
    kv_new = _bf16_rows(rng, n, wl.d_qk)
    kidx_new = _bf16_rows(rng, n, wl.d_idx)
    v_new = _bf16_rows(rng, n, wl.d_v) if wl.separate_v else None
    cache = dsa.Cache(dc.kv, dc.k_idx, dc.block_table, dc.seq_lens, v=dc.v, d_v=wl.d_v)
    dsa.cache_write(cache, torch.from_numpy(seq).cuda(), torch.from_numpy(pos).cuda(),
                    torch.from_numpy(kv_new.view(np.int16)).view(torch.bfloat16).cuda(),
                    torch.from_numpy(kidx_new.view(np.int16)).view(torch.bfloat16).cuda(),
                    None if v_new is None else
                    torch.from_numpy(v_new.view(np.int16)).view(torch.bfloat16).cuda())
    torch.cuda.synchronize()
    oracle.cache_write(hc.kv, hc.block_table, wl.block_size, seq, pos, kv_new)
    oracle.cache_write(hc.k_idx, hc.block_table, wl.block_size, seq, pos, kidx_new)
    if v_new is not None:
        oracle.cache_write(hc.v, hc.block_table, wl.block_size, seq, pos, v_new)

    def host_bits(t):
        return t.reshape(-1, t.shape[-1]).view(torch.int16).cpu().numpy().view(np.uint16)

    np.testing.assert_array_equal(host_bits(dc.kv), hc.kv)
    np.testing.assert_array_equal(host_bits(dc.k_idx), hc.k_idx)
    if v_new is not None:
        np.testing.assert_array_equal(host_bits(dc.v), hc.v)
    say("   ok: pools bit-identical to the oracle's")


def test_cache_write_latent_pools():
    _cache_write_case(dsa_synth.latent("cw_latent", "decode", [300, 700], seed=41, topk=256), 41)


def test_cache_write_separate_v_pool():
    _cache_write_case(dsa_synth.small_mqa("cw_small", "decode", [100, 250], seed=42, topk=64,
                                          block_size=16), 42)


def test_cache_written_rows_are_what_decode_reads():
    # a cache filled token by token through dsa_cache_write (shuffled order)
    # from the logical rows gives the decode step the oracle computes on the
    # generator's pool
    wl = dsa_synth.latent("cw_roundtrip", "decode", [900, 2100], seed=43, topk=512)
    say(f"[cache write -> decode] {wl.name}")
    hc = dsa_synth.host_case(wl)
    dc = dsa_synth.device_case(wl)
    bs = wl.block_size
    seq, pos = [], []
    for b, L in enumerate(wl.seq_lens):
        seq += [b] * L
        pos += list(range(L))
    seq, pos = np.array(seq, np.int32), np.array(pos, np.int32)
    perm = np.random.default_rng(43).permutation(len(seq))
    seq, pos = seq[perm], pos[perm]
    rows = hc.block_table[seq, pos // bs] * bs + pos % bs
    dc.kv.fill_(float("nan"))
    dc.k_idx.fill_(float("nan"))
    cache = dsa.Cache(dc.kv, dc.k_idx, dc.block_table, dc.seq_lens, d_v=wl.d_v)

    def dev(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()

    dsa.cache_write(cache, torch.from_numpy(seq).cuda(), torch.from_numpy(pos).cuda(),
                    dev(hc.kv[rows]), dev(hc.k_idx[rows]))
    step = dsa.DecodeStep(cache, wl.n_q, wl.H, wl.H_idx, wl.topk, max(wl.seq_lens), wl.d_v)
    step(dc.q, dc.q_idx, dc.w, wl.sm_scale)
    torch.cuda.synchronize()
    sc, idx, out, lse = oracle.decode_step(hc)
    np.testing.assert_array_equal(step.idx.cpu().numpy(), idx)
    mx, mn = assert_attention(step.out, step.lse, out, lse, wl.name)
    say(f"   ok: max|err| {mx:.2e} mean|err| {mn:.2e}")


# ----------------------------------------------------------------------------- index holes

def test_attention_skips_negative_indices():
    # entries < 0 inside the first min(K, n) slots are skipped; a row with no
    # kept entry gives out = 0, lse = -inf
    wl = dsa_synth.latent("holes", "decode", [700, 3000, 5000], seed=27, topk=512)
    say(f"[holes] {wl.name}")
    dc = dsa_synth.device_case(wl)
    hc = dsa_synth.host_case(wl)
    _, idx, _, _ = oracle.decode_step(hc)
    rng = np.random.default_rng(27)
    holes = idx.copy()
    holes[rng.random(holes.shape) < 0.3] = -1      # random holes
    holes[1, :40] = -1                             # a first tile with nothing kept
    holes[2, :] = -1                               # nothing kept at all
    out, lse = oracle.sparse_attn(hc.kv, hc.v, hc.block_table, wl.block_size, hc.q, hc.q_seq,
                                  holes, wl.sm_scale, d_v=wl.d_v)
    assert np.all(out[2] == 0) and np.all(np.isneginf(lse[2]))
    cache = dsa.Cache(dc.kv, dc.k_idx, dc.block_table, dc.seq_lens, d_v=wl.d_v)
    o, l = dsa.sparse_attn_decode(cache, dc.q, torch.from_numpy(holes).cuda(), wl.sm_scale)
    torch.cuda.synchronize()
    mx, mn = assert_attention(o, None, out, None, wl.name)
    lg = l.cpu().numpy()
    assert np.all(np.isneginf(lg[2]))
    np.testing.assert_allclose(lg[:2], lse[:2], atol=1e-2)
    say(f"   ok: max|err| {mx:.2e} mean|err| {mn:.2e}")


# ----------------------------------------------------------------------------- per-query calls

def _dev_bf16(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()


def _check_queries(wl, q_seq, q_pos, sm_scale=None, rel=False):
    """One prefill-path call (index score, Top-K, attention) over arbitrary
    queries (q_seq[i], q_pos[i]) of a multi-sequence cache, against the oracle."""
    sm_scale = wl.sm_scale if sm_scale is None else sm_scale
    q_seq = np.asarray(q_seq, np.int32)
    q_pos = np.asarray(q_pos, np.int32)
    T = len(q_seq)
    say(f"[queries] {wl.name}: {T} queries over sequences {sorted(set(q_seq.tolist()))}, "
        f"scale {sm_scale}")
    dc = dsa_synth.device_case(wl)
    hc = dsa_synth.host_case(wl)
    q, q_idx, w = dsa_synth.host_query_rows(wl, 0, T)
    cache = dsa.Cache(dc.kv, dc.k_idx, dc.block_table, dc.seq_lens, v=dc.v, d_v=wl.d_v)
    step = dsa.PrefillStep(cache, T, wl.H, wl.topk, wl.d_v, q_seq=torch.from_numpy(q_seq).cuda(),
                           q_pos=torch.from_numpy(q_pos).cuda())
    step(_dev_bf16(q), _dev_bf16(q_idx), torch.from_numpy(w).cuda(), sm_scale)
    torch.cuda.synchronize()
    ld = step.scores.shape[1]
    sc = oracle.index_score(hc.k_idx, hc.block_table, wl.block_size, q_idx, w, q_seq, q_pos, ld=ld)
    idx = oracle.topk(sc, q_pos + 1, wl.topk)
    out, lse = oracle.sparse_attn(hc.kv, hc.v, hc.block_table, wl.block_size, q, q_seq, idx,
                                  sm_scale, d_v=wl.d_v)
    g_sc = step.scores.cpu().numpy()
    for i in range(T):
        assert np.array_equal(g_sc[i, :q_pos[i] + 1], sc[i, :q_pos[i] + 1]), f"scores row {i}"
    np.testing.assert_array_equal(step.idx.cpu().numpy(), idx)
    mx, mn = assert_attention(step.out, step.lse, out, lse, wl.name, rel=rel)
    if _fused_applies(wl, int(q_pos.max()) + 1):
        check_fused_prefill(dc, torch.from_numpy(q_pos).cuda(), torch.from_numpy(q_seq).cuda(),
                            idx, rows=(_dev_bf16(q_idx), torch.from_numpy(w).cuda()))
    say(f"   ok: max|err| {mx:.2e} mean|err| {mn:.2e}")
    return dc, step, (sc, idx, out, lse)


def test_prefill_call_with_chunks_of_two_sequences():
    # positions 300..690 of sequence 0, then 0..499 of sequence 1: the query
    # block 384..399 holds both sequences (the index kernel's per-sequence pass)
    wl = dsa_synth.latent("two_seq_prefill", "decode", [700, 500], seed=51, topk=256)
    q_seq = [0] * 391 + [1] * 500
    q_pos = list(range(300, 691)) + list(range(500))
    _check_queries(wl, q_seq, q_pos)


def test_small_family_prefill_call_with_two_sequences():
    wl = dsa_synth.small_mqa("two_seq_small", "decode", [333, 200], seed=52, topk=64,
                             block_size=16)
    q_seq = [0] * 100 + [1] * 150 + [0] * 30
    q_pos = list(range(233, 333)) + list(range(50, 200)) + list(range(30))
    _check_queries(wl, q_seq, q_pos)


def test_several_decode_queries_per_sequence():
    # the decode index kernel with per-query arrays: the last three positions
    # of every sequence (e.g. several draft tokens), attention by the
    # per-query (prefill) path
    wl = dsa_synth.latent("multi_query_decode", "decode", [3000, 17000, 40000], seed=53,
                          topk=2048)
    say(f"[decode, 3 queries per sequence] {wl.name}")
    dc = dsa_synth.device_case(wl)
    hc = dsa_synth.host_case(wl)
    q_seq = np.repeat(np.arange(3, dtype=np.int32), 3)
    q_pos = np.array([L - 3 + j for L in wl.seq_lens for j in range(3)], np.int32)
    T = len(q_seq)
    q, q_idx, w = dsa_synth.host_query_rows(wl, 0, T)
    cache = dsa.Cache(dc.kv, dc.k_idx, dc.block_table, dc.seq_lens, d_v=wl.d_v)
    ld = (max(wl.seq_lens) + 63) // 64 * 64
    d_seq, d_pos = torch.from_numpy(q_seq).cuda(), torch.from_numpy(q_pos).cuda()
    scores = dsa.index_score(cache, _dev_bf16(q_idx), torch.from_numpy(w).cuda(), dsa.DSA_DECODE,
                             q_seq=d_seq, q_pos=d_pos, ld=ld)
    g_idx = dsa.topk(scores, wl.topk, n_valid=d_pos + 1)
    o, l = dsa.sparse_attn_prefill(cache, _dev_bf16(q), d_seq, d_pos, g_idx, wl.sm_scale)
    torch.cuda.synchronize()
    sc = oracle.index_score(hc.k_idx, hc.block_table, wl.block_size, q_idx, w, q_seq, q_pos, ld=ld)
    idx = oracle.topk(sc, q_pos + 1, wl.topk)
    out, lse = oracle.sparse_attn(hc.kv, None, hc.block_table, wl.block_size, q, q_seq, idx,
                                  wl.sm_scale, d_v=wl.d_v)
    g_sc = scores.cpu().numpy()
    for i in range(T):
        assert np.array_equal(g_sc[i, :q_pos[i] + 1], sc[i, :q_pos[i] + 1]), f"scores row {i}"
    np.testing.assert_array_equal(g_idx.cpu().numpy(), idx)
    mx, mn = assert_attention(o, l, out, lse, wl.name)
    say(f"   ok: max|err| {mx:.2e} mean|err| {mn:.2e}")


@pytest.mark.parametrize("scale", [0.0, -1.0 / 24.0])
def test_latent_zero_and_negative_softmax_scale(scale):
    # the softmax scale may be any finite value: 0 gives equal weights, a
    # negative one favours the lowest logits (decode and prefill kernels)
    wl = dsa_synth.latent("scale_decode", "decode", [900, 5000, 20000], seed=54, topk=2048)
    wl = dataclasses.replace(wl, sm_scale=scale)
    check_decode(wl)
    wp = dsa_synth.latent("scale_prefill", "decode", [600], seed=55, topk=256)
    _check_queries(wp, [0] * 300, list(range(300, 600)), sm_scale=scale)


def test_debug_build_flags_bad_device_data():
    """The DSA_DEBUG_BOUNDS build checks the device data the host never reads.
    The pool holds one block more than the cache description declares, so
    the planted bad values address real memory in every build."""
    wl = dsa_synth.latent("debug_bounds", "decode", [3000, 20000], seed=56, topk=512)
    say(f"[debug build] {wl.name}")
    D = dsa.debug_lib()
    dc = dsa_synth.device_case(wl)
    nb = wl.pool_blocks
    kv = torch.cat([dc.kv, torch.zeros_like(dc.kv[:1])]).contiguous()
    kidx = torch.cat([dc.k_idx, torch.zeros_like(dc.k_idx[:1])]).contiguous()
    cache = dsa.Cache(kv, kidx, dc.block_table, dc.seq_lens, d_v=wl.d_v)
    cache.c.num_blocks = nb  # the extra block lies outside the description
    st = dsa.DecodeStep(cache, wl.n_q, wl.H, wl.H_idx, wl.topk, max(wl.seq_lens), wl.d_v)
    # clean data: no error, and the same bits as the release build
    st(dc.q, dc.q_idx, dc.w, wl.sm_scale, library=D)
    assert dsa.check_device_errors(library=D) == 0
    dbg = (st.idx.clone(), st.out.clone())
    st(dc.q, dc.q_idx, dc.w, wl.sm_scale)
    torch.cuda.synchronize()
    assert torch.equal(dbg[0], st.idx) and torch.equal(dbg[1], st.out)
    assert dsa.check_device_errors() == 3  # release build: nothing checked
    # a block-table entry outside [0, num_blocks)
    bt = dc.block_table.clone()
    bt[1, 5] = nb
    cache_bad = dsa.Cache(kv, kidx, bt, dc.seq_lens, d_v=wl.d_v)
    cache_bad.c.num_blocks = nb
    st.cache = cache_bad
    st(dc.q, dc.q_idx, dc.w, wl.sm_scale, library=D)
    assert dsa.check_device_errors(library=D) == 7
    assert dsa.check_device_errors(library=D) == 0  # the record was cleared
    # a kept index past its row's candidate count
    idx = dbg[0].clone()
    idx[0, 3] = wl.seq_lens[0]
    dsa.sparse_attn_decode(cache, dc.q, idx, wl.sm_scale, library=D)
    assert dsa.check_device_errors(library=D) == 7
    # a sequence length beyond the block table
    lens = dc.seq_lens.clone()
    lens[0] = wl.max_blocks * wl.block_size + 1
    cache_len = dsa.Cache(kv, kidx, dc.block_table, lens, d_v=wl.d_v)
    cache_len.c.num_blocks = nb
    dsa.index_score(cache_len, dc.q_idx, dc.w, dsa.DSA_DECODE, out=st.scores, library=D)
    assert dsa.check_device_errors(library=D) == 7
    say("   ok: clean data passes, bad block / index / length are flagged")


# ----------------------------------------------------------------------------- fused Top-K

def _logical_rows(wl, bt, b, L):
    return bt[b, np.arange(L) // wl.block_size] * wl.block_size + np.arange(L) % wl.block_size


def _fused_case(wl, hc, what):
    """Upload the host case's indexer keys / queries, run the fused and the
    separate selection, compare both with the oracle bit for bit."""
    say(f"[fused Top-K] {what}")
    dc = dsa_synth.device_case(wl)
    dc.k_idx.copy_(torch.from_numpy(hc.k_idx.view(np.int16)).view(torch.bfloat16)
                   .reshape(dc.k_idx.shape))
    dc.q_idx.copy_(torch.from_numpy(hc.q_idx.view(np.int16)).view(torch.bfloat16))
    dc.w.copy_(torch.from_numpy(hc.w))
    cache = dsa.Cache(dc.kv, dc.k_idx, dc.block_table, dc.seq_lens, d_v=wl.d_v)
    ld = max(wl.seq_lens)
    fused = dsa.DecodeStep(cache, wl.n_q, wl.H, wl.H_idx, wl.topk, ld, wl.d_v)
    sep = dsa.DecodeStep(cache, wl.n_q, wl.H, wl.H_idx, wl.topk, ld, wl.d_v, fused=False)
    fused.select(dc.q_idx, dc.w)
    sep.select(dc.q_idx, dc.w)
    torch.cuda.synchronize()
    sc = oracle.index_score(hc.k_idx, hc.block_table, wl.block_size, hc.q_idx, hc.w, hc.q_seq,
                            hc.q_pos, ld=ld)
    idx = oracle.topk(sc, hc.q_pos + 1, wl.topk)
    np.testing.assert_array_equal(fused.idx.cpu().numpy(), idx, err_msg=what)
    np.testing.assert_array_equal(sep.idx.cpu().numpy(), idx, err_msg=what + " (separate)")
    return fused


def test_fused_topk_score_patterns():
    """Score patterns chosen against the group-maxima bound: every score equal
    (ties everywhere: the first K positions), scores constant within each
    16-position group (group-level ties), the high scores packed into a few
    groups, and a row whose top scores sit in the last, partial group."""
    lens = [16385, 20000, 33000, 131072, 70001]
    wl = dsa_synth.latent("fused_patterns", "decode", lens, seed=71, topk=2048, H_idx=64)
    hc = dsa_synth.host_case(wl, with_kv=False)
    bt = hc.block_table
    one = 0x3F80  # bf16 1.0
    # sequence 0: q = 0 -> every score 0
    hc.q_idx[0] = 0
    # sequence 1: key of position p is ((p // 16) % 3 - 1) in every column, q = 1
    r = _logical_rows(wl, bt, 1, lens[1])
    vals = np.array([0xBF80, 0x0000, 0x3F80], np.uint16)  # -1, 0, 1
    hc.k_idx[r] = vals[(np.arange(lens[1]) // 16) % 3][:, None]
    hc.q_idx[1] = one
    # sequence 2: keys 0 except 3 groups of 16 with key 1 (plus random noise
    # elsewhere below them): q = 1
    r = _logical_rows(wl, bt, 2, lens[2])
    hc.k_idx[r] = 0
    for g in (5, 1000, 2062):
        hc.k_idx[r[16 * g:16 * g + 16]] = one
    hc.q_idx[2] = one
    # sequence 4: the largest keys in the last (partial) group
    r = _logical_rows(wl, bt, 4, lens[4])
    hc.k_idx[r[-1:]] = 0x4040  # 3.0
    hc.q_idx[4] = one
    _fused_case(wl, hc, "patterns")


@pytest.mark.parametrize("K,n_a,n_b", [(1000, 900, 400), (2048, 2000, 1000), (2048, 2000, 1500),
                                       (2048, 2000, 2500)])
def test_fused_topk_ties_in_the_candidate_list(K, n_a, n_b):
    """Ties at the K-th score inside the candidate list.  In a 65000-position
    row, n_a positions share the highest score and n_b the second highest
    (every 13th position, so each is the maximum of its 16-position group),
    all others score far lower: the bound is the second score, the list holds
    exactly the n_a + n_b positions (1300, 3000, 3500: searched by one wave;
    4500: by the whole workgroup), and the kept ones are the n_a and the
    lowest K - n_a of the n_b."""
    L = 65000
    wl = dsa_synth.latent("fused_ties", "decode", [L, 30000], seed=75, topk=K, H_idx=64)
    hc = dsa_synth.host_case(wl, with_kv=False)
    r = _logical_rows(wl, hc.block_table, 0, L)
    hc.q_idx[0] = 0x3F80  # q = 1: a score is relu(sum of the key row) * sum(w), w >= 1
    hc.k_idx[r[13 * np.arange(n_a)]] = 0x4040           # 3.0: sum 384
    hc.k_idx[r[30000 + 13 * np.arange(n_b)]] = 0x4000   # 2.0: sum 256 (random rows: |sum| < 150)
    f = _fused_case(wl, hc, f"ties at the K-th score: K={K}, {n_a} + {n_b} listed")
    kept = f.idx[0].cpu().numpy()
    np.testing.assert_array_equal(
        kept, np.concatenate([13 * np.arange(n_a), 30000 + 13 * np.arange(K - n_a)]))


def test_fused_topk_negative_and_zero_scores():
    """Scores at or below zero, where the expansion forms keys instead of
    comparing raw bits: one row with every head weight negated (scores
    -w . relu(q . k): zeros of both signs and negative values), one with
    weights of alternating sign (both signs), one as generated."""
    lens = [20000, 70000, 131072]
    wl = dsa_synth.latent("fused_negative", "decode", lens, seed=76, topk=2048, H_idx=64)
    hc = dsa_synth.host_case(wl, with_kv=False)
    hc.w[0] = -hc.w[0]
    hc.w[1, 1::2] = -hc.w[1, 1::2]
    _fused_case(wl, hc, "scores <= 0 and of both signs")


def test_fused_topk_small_K():
    # K = 37: rows have at least 4 K groups, the bound comes from the group
    # maxima alone; the longest row uses every group slot of the kernel
    wl = dsa_synth.latent("fused_smallK", "decode", [17000, 100000, 262144], seed=72, topk=37)
    hc = dsa_synth.host_case(wl, with_kv=False)
    _fused_case(wl, hc, "K=37, rows up to 262144")


def test_index_topk_long_rows_with_query_positions():
    """Row capacity past 262144: the fused call takes the long-row selection;
    queries given by per-query positions (two per sequence, the second a few
    positions before the end)."""
    wl = dsa_synth.latent("long_rows_q", "decode", [20000, 300000, 1100000], seed=74, topk=2048)
    say(f"[index + Top-K, long rows, per-query positions] {wl.seq_lens}")
    dc = dsa_synth.device_case(wl)
    hc = dsa_synth.host_case(wl, with_kv=False)
    q_seq = np.repeat(np.arange(wl.n_seq, dtype=np.int32), 2)
    q_pos = np.array([L - 1 - 5 * j for L in wl.seq_lens for j in range(2)], np.int32)
    T = len(q_seq)
    _, q_idx, w = dsa_synth.host_query_rows(wl, 0, T)
    cache = dsa.Cache(dc.kv, dc.k_idx, dc.block_table, dc.seq_lens, d_v=wl.d_v)
    ld = (max(wl.seq_lens) + 63) // 64 * 64
    scores = torch.empty((T, ld), dtype=torch.float32, device="cuda")
    idx = torch.empty((T, wl.topk), dtype=torch.int32, device="cuda")
    ws = dsa.index_topk_workspace(T, ld, wl.topk)
    dsa.index_topk_decode(cache, _dev_bf16(q_idx), torch.from_numpy(w).cuda(), wl.topk, scores,
                          idx, ws, q_seq=torch.from_numpy(q_seq).cuda(),
                          q_pos=torch.from_numpy(q_pos).cuda())
    torch.cuda.synchronize()
    sc = oracle.index_score(hc.k_idx, hc.block_table, wl.block_size, q_idx, w, q_seq, q_pos, ld=ld)
    want = oracle.topk(sc, q_pos + 1, wl.topk)
    np.testing.assert_array_equal(idx.cpu().numpy(), want)
    say("   ok: Top-K exact")


def test_fused_topk_with_query_positions():
    # the fused selection with per-query positions (counts = q_pos + 1)
    wl = dsa_synth.latent("fused_q", "decode", [30000, 90000], seed=75, topk=2048)
    say(f"[fused index + Top-K, per-query positions] {wl.seq_lens}")
    dc = dsa_synth.device_case(wl)
    hc = dsa_synth.host_case(wl, with_kv=False)
    q_seq = np.array([0, 0, 1, 1, 1], np.int32)
    q_pos = np.array([29999, 17000, 89999, 45000, 16500], np.int32)
    T = len(q_seq)
    _, q_idx, w = dsa_synth.host_query_rows(wl, 0, T)
    cache = dsa.Cache(dc.kv, dc.k_idx, dc.block_table, dc.seq_lens, d_v=wl.d_v)
    ld = 90048
    scores = torch.empty((T, ld), dtype=torch.float32, device="cuda")
    idx = torch.empty((T, wl.topk), dtype=torch.int32, device="cuda")
    ws = dsa.index_topk_workspace(T, ld, wl.topk)
    dsa.index_topk_decode(cache, _dev_bf16(q_idx), torch.from_numpy(w).cuda(), wl.topk, scores,
                          idx, ws, q_seq=torch.from_numpy(q_seq).cuda(),
                          q_pos=torch.from_numpy(q_pos).cuda())
    torch.cuda.synchronize()
    sc = oracle.index_score(hc.k_idx, hc.block_table, wl.block_size, q_idx, w, q_seq, q_pos, ld=ld)
    want = oracle.topk(sc, q_pos + 1, wl.topk)
    np.testing.assert_array_equal(idx.cpu().numpy(), want)
    say("   ok: Top-K exact")


def test_incremental_decode_eight_steps():
    """Eight consecutive decode steps: each appends one token per sequence
    with dsa_cache_write, then runs the fused index score + Top-K with the
    previous step's per-row threshold as a hint, and attention; every step
    is compared with the oracle on the grown cache (indices bit-exact,
    attention within the bars).  Queries drift slowly from step to step, as
    consecutive decode queries do, so the hint is often usable."""
    wl0 = dsa_synth.latent("incremental", "decode", [5000, 20000, 40000], seed=73, topk=2048)
    steps = 8
    # a cache with room for the appended tokens: the workload of the final
    # lengths; the first steps see shorter sequences (seq_lens grows)
    wl = dsa_synth.latent("incremental", "decode", [L + steps for L in wl0.seq_lens], seed=73,
                          topk=2048)
    say(f"[incremental decode] {wl0.seq_lens} + {steps} steps")
    dc = dsa_synth.device_case(wl)
    hc = dsa_synth.host_case(wl)
    rng = np.random.default_rng(73)
    lens = np.array(wl0.seq_lens, np.int32)
    # the pool rows of the appended positions hold other values until written
    for b, L in enumerate(lens):
        rows = _logical_rows(wl, hc.block_table, b, L + steps)[L:]
        hc.kv[rows] = 0
        hc.k_idx[rows] = 0
    dc.kv.view(-1, wl.d_qk)[torch.from_numpy(np.concatenate(
        [_logical_rows(wl, hc.block_table, b, L + steps)[L:] for b, L in enumerate(lens)])).long()
        .cuda()] = 0
    seq_lens = torch.from_numpy(lens.copy()).cuda()
    cache = dsa.Cache(dc.kv, dc.k_idx, dc.block_table, seq_lens, d_v=wl.d_v)
    st = dsa.DecodeStep(cache, wl.n_q, wl.H, wl.H_idx, wl.topk, max(wl.seq_lens), wl.d_v,
                        seed=True)
    q_idx = hc.q_idx.copy()
    for s_ in range(steps):
        # append one token per sequence at position lens[b]
        new_kv = _bf16_rows(rng, wl.n_q, wl.d_qk)
        new_ki = rng.integers(-3, 4, (wl.n_q, wl.d_idx)).astype(np.float32)
        new_ki = torch.from_numpy(new_ki).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        seq = np.arange(wl.n_q, dtype=np.int32)
        pos = lens.copy()
        dsa.cache_write(cache, torch.from_numpy(seq).cuda(), torch.from_numpy(pos).cuda(),
                        _dev_bf16(new_kv), _dev_bf16(new_ki))
        oracle.cache_write(hc.kv, hc.block_table, wl.block_size, seq, pos, new_kv)
        oracle.cache_write(hc.k_idx, hc.block_table, wl.block_size, seq, pos, new_ki)
        lens += 1
        seq_lens.copy_(torch.from_numpy(lens))
        # the query drifts: a few indexer entries change per step
        flip = rng.random(q_idx.shape) < 0.02
        q_idx[flip] = torch.from_numpy(rng.integers(-3, 4, flip.sum()).astype(np.float32)).to(
            torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        q = hc.q
        st(_dev_bf16(q), _dev_bf16(q_idx), dc.w, wl.sm_scale)
        torch.cuda.synchronize()
        ld = int(lens.max())
        sc = oracle.index_score(hc.k_idx, hc.block_table, wl.block_size, q_idx, hc.w,
                                np.arange(wl.n_q, dtype=np.int32), lens - 1, ld=ld)
        idx = oracle.topk(sc, lens, wl.topk)
        out, lse = oracle.sparse_attn(hc.kv, None, hc.block_table, wl.block_size, q,
                                      np.arange(wl.n_q, dtype=np.int32), idx, wl.sm_scale,
                                      d_v=wl.d_v)
        np.testing.assert_array_equal(st.idx.cpu().numpy(), idx, err_msg=f"step {s_}")
        mx, mn = assert_attention(st.out, st.lse, out, lse, f"step {s_}")
        say(f"   step {s_}: lengths {lens.tolist()}: Top-K exact, attention max|err| {mx:.2e}")


def test_fused_prefill_mixed_blocks_short_rows_and_reuse():
    """The fused prefill selection over queries that interleave two
    sequences inside every 4-query block, rows shorter than K (all kept, -1
    padded), the last position allowed (8191), and a second call on the same
    workspace."""
    wl = dsa_synth.latent("fused_mix", "decode", [8192, 3000], seed=61, topk=512)
    rng = np.random.default_rng(7)
    pos0 = np.concatenate([rng.integers(0, 8192, 120), [8191, 0, 1, 511, 512, 513]])
    pos1 = rng.integers(0, 3000, 126)
    q_seq = np.empty(252, np.int32)
    q_pos = np.empty(252, np.int32)
    q_seq[0::2], q_pos[0::2] = 0, pos0
    q_seq[1::2], q_pos[1::2] = 1, pos1
    dc = dsa_synth.device_case(wl)
    hc = dsa_synth.host_case(wl)
    _, q_idx, w = dsa_synth.host_query_rows(wl, 0, len(q_seq))
    sc = oracle.index_score(hc.k_idx, hc.block_table, wl.block_size, q_idx, w, q_seq, q_pos,
                            ld=8192)
    idx = oracle.topk(sc, q_pos + 1, wl.topk)
    say(f"[fused prefill] {len(q_seq)} queries over 2 sequences, K={wl.topk}")
    cache = dsa.Cache(dc.kv, dc.k_idx, dc.block_table, dc.seq_lens, v=dc.v, d_v=wl.d_v)
    ws = dsa.index_topk_prefill_workspace(len(q_seq))
    args = (cache, _dev_bf16(q_idx), torch.from_numpy(w).cuda(), torch.from_numpy(q_seq).cuda(),
            torch.from_numpy(q_pos).cuda(), wl.topk)
    for rep in range(2):
        got = dsa.index_topk_prefill(*args, workspace=ws)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(got.cpu().numpy(), idx, err_msg=f"call {rep}")
    say("   exact on both calls")


@pytest.mark.parametrize("K,bs", [(1, 64), (37, 16), (511, 64), (2048, 16)])
def test_fused_prefill_odd_K_and_rows_around_K(K, bs):
    """The fused prefill selection for K values that are not multiples of the
    wave width, rows with exactly K - 1, K and K + 1 candidates (all kept,
    all kept, one dropped), a partial last block of queries and both block
    sizes, against the oracle."""
    wl = dsa_synth.latent(f"fused_k{K}", "decode", [8192, 2500], seed=63 + K % 7, topk=K,
                          block_size=bs)
    rng = np.random.default_rng(K)
    near = [p for p in (K - 2, K - 1, K) if 0 <= p < 8192]
    pos0 = np.concatenate([near, rng.integers(0, 8192, 40 - len(near)), [8191]])
    pos1 = rng.integers(0, 2500, 12)
    q_seq = np.concatenate([np.zeros(len(pos0), np.int32), np.ones(len(pos1), np.int32)])
    q_pos = np.concatenate([pos0, pos1]).astype(np.int32)
    dc = dsa_synth.device_case(wl)
    hc = dsa_synth.host_case(wl)
    _, q_idx, w = dsa_synth.host_query_rows(wl, 0, len(q_seq))
    sc = oracle.index_score(hc.k_idx, hc.block_table, wl.block_size, q_idx, w, q_seq, q_pos,
                            ld=8192)
    idx = oracle.topk(sc, q_pos + 1, K)
    say(f"[fused prefill] K={K}, block size {bs}, {len(q_seq)} queries")
    cache = dsa.Cache(dc.kv, dc.k_idx, dc.block_table, dc.seq_lens, v=dc.v, d_v=wl.d_v)
    got = dsa.index_topk_prefill(cache, _dev_bf16(q_idx), torch.from_numpy(w).cuda(),
                                 torch.from_numpy(q_seq).cuda(), torch.from_numpy(q_pos).cuda(), K)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(got.cpu().numpy(), idx)
    say("   exact")


def test_fused_prefill_debug_build_flags_positions_past_8192():
    D = dsa.debug_lib()
    wl = dsa_synth.latent("fused_dbg", "decode", [9000], seed=62, topk=64)
    dc = dsa_synth.device_case(wl)
    cache = dsa.Cache(dc.kv, dc.k_idx, dc.block_table, dc.seq_lens, v=dc.v, d_v=wl.d_v)
    assert dsa.check_device_errors(library=D) == 0
    # eight queries of the one sequence (the decode case has a single query row)
    q8 = dc.q_idx[:1].repeat(8, 1, 1).contiguous()
    w8 = dc.w[:1].repeat(8, 1).contiguous()
    q_seq = torch.zeros(8, dtype=torch.int32, device="cuda")
    ok = torch.arange(8184, 8192, dtype=torch.int32, device="cuda")  # up to 8192 candidates
    good = dsa.index_topk_prefill(cache, q8, w8, q_seq, ok, wl.topk, library=D)
    assert dsa.check_device_errors(library=D) == 0
    rel = dsa.index_topk_prefill(cache, q8, w8, q_seq, ok, wl.topk)
    torch.cuda.synchronize()
    assert torch.equal(good, rel)
    bad = torch.arange(8190, 8198, dtype=torch.int32, device="cuda")  # 8193 .. 8198 candidates
    dsa.index_topk_prefill(cache, q8, w8, q_seq, bad, wl.topk, library=D)
    assert dsa.check_device_errors(library=D) == 7
    assert dsa.check_device_errors(library=D) == 0
