"""Pins of the oracle to things other than itself: a hand-worked example,
closed forms, library routines on special cases, invariants and brute force
on tiny inputs.  A plausible slip in the oracle (a dropped ReLU, a wrong head
weight, a transposed operand, a wrong block-table lookup, a tie broken the
wrong way, a missed padding entry) fails at least one test here.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_worked.json")


def bf16_bits(x):
    """float array -> uint16 bf16 bits (values used here are exact in bf16)."""
    t = torch.as_tensor(np.asarray(x, dtype=np.float32)).to(torch.bfloat16)
    assert np.array_equal(t.float().numpy(), np.asarray(x, dtype=np.float32), equal_nan=True), \
        "inexact"
    return t.view(torch.int16).numpy().view(np.uint16)


def bf16_float(bits):
    return torch.from_numpy(np.asarray(bits, dtype=np.uint16).view(np.int16)).view(
        torch.bfloat16).double().numpy()


def to_pool(logical, block_table, block_size, n_blocks, fill=np.nan):
    """Scatter logical rows [n_seq][L][d] into a paged pool [n_blocks*bs, d] the
    way the paged-cache layout states it: position p of sequence b goes to
    block block_table[b][p // bs], slot p % bs.  Other rows get `fill`."""
    d = logical[0].shape[-1]
    pool = np.full((n_blocks * block_size, d), fill, dtype=np.float32)
    for b, rows in enumerate(logical):
        for p in range(rows.shape[0]):
            pool[block_table[b][p // block_size] * block_size + p % block_size] = rows[p]
    return pool


def random_table(rng, n_seq, blocks_each, extra=0):
    n_blocks = n_seq * blocks_each + extra
    perm = rng.permutation(n_blocks).astype(np.int32)
    return perm[: n_seq * blocks_each].reshape(n_seq, blocks_each), n_blocks


# ----------------------------------------------------------------------------- hand example

def test_hand_worked_index_score_and_topk(oracle_lib):
    g = json.load(open(GOLDEN))["index_score"]
    bt = np.array(g["block_table"], dtype=np.int32)
    pool = to_pool([np.array(g["logical_k_idx"], dtype=np.float32)], bt, g["block_size"], 2)
    sc = oracle_lib.index_score(bf16_bits(pool), bt, g["block_size"],
                                bf16_bits(np.array([g["q_idx"]], dtype=np.float32)),
                                np.array([g["w"]], dtype=np.float32), np.array([0]),
                                np.array([g["q_pos"]]))
    assert sc[0].tolist() == g["scores"]
    for k, want in g["topk"].items():
        got = oracle_lib.topk(sc, np.array([4]), int(k))
        assert got[0].tolist() == want, k


def test_hand_worked_attention(oracle_lib):
    g = json.load(open(GOLDEN))["attention"]
    bt = np.array(g["block_table"], dtype=np.int32)
    kp = to_pool([np.array(g["logical_k"], dtype=np.float32)], bt, g["block_size"], 2)
    vp = to_pool([np.array(g["logical_v"], dtype=np.float32)], bt, g["block_size"], 2)
    out, lse = oracle_lib.sparse_attn(bf16_bits(kp), bf16_bits(vp), bt, g["block_size"],
                                      bf16_bits(np.array([g["q"]], dtype=np.float32)),
                                      np.array([0]), np.array([g["idx"]], dtype=np.int32),
                                      math.log(3.0))
    np.testing.assert_allclose(out[0, 0], g["out"], rtol=0, atol=1e-6)
    assert abs(lse[0, 0] - math.log(4.0)) < 1e-6


# ----------------------------------------------------------------------------- index score

def _score_setup(rng, n_seq=3, L=37, bs=8, H=5, d=16, lo=-3, hi=3, n_q_per_seq=2):
    blocks_each = (L + bs - 1) // bs
    bt, n_blocks = random_table(rng, n_seq, blocks_each, extra=2)
    keys = [rng.integers(lo, hi + 1, size=(L, d)).astype(np.float32) for _ in range(n_seq)]
    pool = to_pool(keys, bt, bs, n_blocks)
    n_q = n_seq * n_q_per_seq
    q_seq = np.repeat(np.arange(n_seq), n_q_per_seq).astype(np.int32)
    q_pos = rng.integers(0, L, size=n_q).astype(np.int32)
    q_pos[0] = L - 1
    q = rng.integers(lo, hi + 1, size=(n_q, H, d)).astype(np.float32)
    w = rng.integers(1, 5, size=(n_q, H)).astype(np.float32)
    return bt, keys, pool, q, w, q_seq, q_pos


def test_identity_activation_is_a_matmul(oracle_lib):
    """With the activation switched off the score is (sum_h w_h q_h) . k: a
    library matmul on the unpaged keys pins contraction, head weights and the
    block-table lookup."""
    rng = np.random.default_rng(11)
    bt, keys, pool, q, w, q_seq, q_pos = _score_setup(rng)
    bs = 8
    sc = oracle_lib.index_score(bf16_bits(pool), bt, bs, bf16_bits(q), w, q_seq, q_pos,
                                relu=False, ld=37)
    for i in range(q.shape[0]):
        ref = keys[q_seq[i]] @ (w[i] @ q[i])  # numpy matmul
        n = q_pos[i] + 1
        np.testing.assert_array_equal(sc[i, :n], ref[:n].astype(np.float32))
        assert np.isnan(sc[i, n:]).all(), "entries past the query position must stay untouched"


def test_relu_identities(oracle_lib):
    """relu(x) - relu(-x) = x and relu(x) + relu(-x) = |x| pin the per-head
    ReLU against per-head library matmuls."""
    rng = np.random.default_rng(12)
    bt, keys, pool, q, w, q_seq, q_pos = _score_setup(rng)
    bs = 8
    kw = dict(ld=37)
    plus = oracle_lib.index_score(bf16_bits(pool), bt, bs, bf16_bits(q), w, q_seq, q_pos, **kw)
    minus = oracle_lib.index_score(bf16_bits(pool), bt, bs, bf16_bits(-q), w, q_seq, q_pos, **kw)
    for i in range(q.shape[0]):
        n = q_pos[i] + 1
        per_head = keys[q_seq[i]][:n] @ q[i].T          # [n, H] numpy matmul
        np.testing.assert_array_equal(plus[i, :n] - minus[i, :n], per_head @ w[i])
        np.testing.assert_array_equal(plus[i, :n] + minus[i, :n], np.abs(per_head) @ w[i])
        assert (plus[i, :n] >= 0).all()


def test_scores_exact_integers_and_bounded(oracle_lib):
    rng = np.random.default_rng(13)
    bt, keys, pool, q, w, q_seq, q_pos = _score_setup(rng, H=64, d=128, L=70, bs=16)
    sc = oracle_lib.index_score(bf16_bits(pool), bt, 16, bf16_bits(q), w, q_seq, q_pos, ld=70)
    for i in range(q.shape[0]):
        row = sc[i, : q_pos[i] + 1]
        assert (row == np.round(row)).all()
        assert row.max() <= 64 * 4 * 128 * 9 < 2 ** 24


def test_scores_invariant_under_block_table(oracle_lib):
    rng = np.random.default_rng(14)
    L, bs, d = 45, 4, 8
    keys = [rng.integers(-3, 4, size=(L, d)).astype(np.float32)]
    q = rng.integers(-3, 4, size=(1, 3, d)).astype(np.float32)
    w = rng.integers(1, 5, size=(1, 3)).astype(np.float32)
    res = []
    for seed in range(3):
        bt, nb = random_table(np.random.default_rng(seed), 1, 12, extra=5)
        pool = to_pool(keys, bt, bs, nb)
        res.append(oracle_lib.index_score(bf16_bits(pool), bt, bs, bf16_bits(q), w, [0], [L - 1]))
    np.testing.assert_array_equal(res[0], res[1])
    np.testing.assert_array_equal(res[0], res[2])


# ----------------------------------------------------------------------------- top-k

def brute_topk(scores, n, K):
    """Repeatedly take the best remaining candidate (largest score, lowest
    position on ties); then list ascending and pad."""
    left = list(range(n))
    kept = []
    for _ in range(min(K, n)):
        best = left[0]
        for s in left[1:]:
            if scores[s] > scores[best]:
                best = s
        kept.append(best)
        left.remove(best)
    return sorted(kept) + [-1] * (K - len(kept))


@pytest.mark.parametrize("seed", range(6))
def test_topk_brute_force_with_heavy_ties(oracle_lib, seed):
    rng = np.random.default_rng(100 + seed)
    n_q, ld = 7, 80
    scores = rng.integers(0, 6, size=(n_q, ld)).astype(np.float32)   # many ties
    n_valid = rng.integers(1, ld + 1, size=n_q).astype(np.int32)
    for K in (1, 3, 16, 79, 80, 100):
        got = oracle_lib.topk(scores, n_valid, K)
        for i in range(n_q):
            assert got[i].tolist() == brute_topk(scores[i], n_valid[i], K), (i, K)


def test_topk_invariants_random_floats(oracle_lib):
    rng = np.random.default_rng(7)
    n_q, ld, K = 5, 5000, 257
    scores = np.round(rng.normal(size=(n_q, ld)) * 20).astype(np.float32)
    n_valid = np.array([5000, 4000, 257, 100, 3333], dtype=np.int32)
    idx = oracle_lib.topk(scores, n_valid, K)
    for i in range(n_q):
        n = n_valid[i]
        kept = idx[i][idx[i] >= 0]
        assert len(kept) == min(n, K) and (idx[i][len(kept):] == -1).all()
        assert (np.diff(kept) > 0).all() and kept.max() < n
        if n > K:
            rest = np.setdiff1d(np.arange(n), kept)
            tau = scores[i, kept].min()
            assert scores[i, rest].max() <= tau
            ties = np.flatnonzero(scores[i, :n] == tau)
            kept_ties = np.intersect1d(kept, ties)
            np.testing.assert_array_equal(kept_ties, ties[: len(kept_ties)])


def test_topk_special_cases(oracle_lib):
    n = 300
    equal = np.full((1, n), 5.0, dtype=np.float32)
    assert oracle_lib.topk(equal, [n], 64)[0].tolist() == list(range(64))
    inc = np.arange(n, dtype=np.float32)[None]
    assert oracle_lib.topk(inc, [n], 64)[0].tolist() == list(range(n - 64, n))
    dec = inc[:, ::-1].copy()
    assert oracle_lib.topk(dec, [n], 64)[0].tolist() == list(range(64))
    short = oracle_lib.topk(inc, [10], 64)[0]
    assert short.tolist() == list(range(10)) + [-1] * 54
    rng = np.random.default_rng(3)
    r = rng.integers(0, 50, size=(4, n)).astype(np.float32)
    got = oracle_lib.topk(r, [n] * 4, 1)
    assert got[:, 0].tolist() == np.argmax(r, axis=1).tolist()   # first maximum
    signed0 = np.array([[0.0, -0.0, 0.0, -0.0, -1.0]], dtype=np.float32)
    assert oracle_lib.topk(signed0, [5], 2)[0].tolist() == [0, 1]


# ----------------------------------------------------------------------------- attention

def _attn_setup(rng, n_seq=2, L=29, bs=4, d_qk=24, d_v=16, H=3):
    blocks_each = (L + bs - 1) // bs
    bt, n_blocks = random_table(rng, n_seq, blocks_each, extra=3)
    kl = [rng.normal(size=(L, d_qk)).astype(np.float32) for _ in range(n_seq)]
    vl = [rng.normal(size=(L, d_v)).astype(np.float32) for _ in range(n_seq)]
    kl = [bf16_float(bf16_bits_round(x)).astype(np.float32) for x in kl]
    vl = [bf16_float(bf16_bits_round(x)).astype(np.float32) for x in vl]
    kp = to_pool(kl, bt, bs, n_blocks)
    vp = to_pool(vl, bt, bs, n_blocks)
    return bt, kl, vl, kp, vp


def bf16_bits_round(x):
    return torch.as_tensor(np.asarray(x, dtype=np.float32)).to(torch.bfloat16).view(
        torch.int16).numpy().view(np.uint16)


def test_select_all_equals_dense_causal_attention(oracle_lib):
    """Keeping every candidate (K >= n) must give textbook causal attention:
    torch's scaled_dot_product_attention in float64 with a causal mask."""
    rng = np.random.default_rng(21)
    L, bs, H, d_qk, d_v = 29, 4, 3, 24, 16
    bt, kl, vl, kp, vp = _attn_setup(rng, n_seq=1, L=L, bs=bs, d_qk=d_qk, d_v=d_v, H=H)
    q = bf16_bits_round(rng.normal(size=(L, H, d_qk)))
    K = 32
    idx = np.array([list(range(t + 1)) + [-1] * (K - t - 1) for t in range(L)], dtype=np.int32)
    scale = 1.0 / math.sqrt(d_qk)
    out, lse = oracle_lib.sparse_attn(bf16_bits_round(kp), bf16_bits_round(vp), bt, bs, q,
                                      np.zeros(L, np.int32), idx, scale)
    Q = torch.from_numpy(bf16_float(q)).permute(1, 0, 2)          # [H, L, d]
    Kt = torch.from_numpy(kl[0].astype(np.float64))[None].expand(H, L, d_qk)
    Vt = torch.from_numpy(vl[0].astype(np.float64))[None].expand(H, L, d_v)
    ref = torch.nn.functional.scaled_dot_product_attention(Q, Kt, Vt, is_causal=True,
                                                           scale=scale)
    np.testing.assert_allclose(out, ref.permute(1, 0, 2).numpy(), rtol=0, atol=1e-6)
    logits = (Q @ Kt.transpose(1, 2)) * scale
    mask = torch.triu(torch.ones(L, L, dtype=torch.bool), 1)
    ref_lse = torch.logsumexp(logits.masked_fill(mask, -math.inf), dim=-1)   # [H, L]
    np.testing.assert_allclose(lse, ref_lse.T.numpy(), rtol=0, atol=1e-5)


def test_random_selection_equals_masked_softmax(oracle_lib):
    rng = np.random.default_rng(22)
    L, bs, H, d_qk, d_v, K = 29, 4, 3, 24, 16, 9
    bt, kl, vl, kp, vp = _attn_setup(rng, n_seq=2, L=L, bs=bs, d_qk=d_qk, d_v=d_v, H=H)
    n_q = 4
    q_seq = np.array([0, 1, 1, 0], np.int32)
    q = bf16_bits_round(rng.normal(size=(n_q, H, d_qk)))
    idx = np.full((n_q, K), -1, np.int32)
    for i in range(n_q):
        m = rng.integers(1, K + 1)
        idx[i, :m] = np.sort(rng.choice(L, size=m, replace=False))
    scale = 0.3
    out, lse = oracle_lib.sparse_attn(bf16_bits_round(kp), bf16_bits_round(vp), bt, bs, q, q_seq,
                                      idx, scale)
    for i in range(n_q):
        sel = idx[i][idx[i] >= 0]
        mask = torch.full((L,), -math.inf, dtype=torch.float64)
        mask[torch.from_numpy(sel).long()] = 0.0
        Kt = torch.from_numpy(kl[q_seq[i]].astype(np.float64))
        Vt = torch.from_numpy(vl[q_seq[i]].astype(np.float64))
        Qi = torch.from_numpy(bf16_float(q[i]))
        logits = (Qi @ Kt.T) * scale + mask
        p = torch.softmax(logits, dim=-1)
        np.testing.assert_allclose(out[i], (p @ Vt).numpy(), rtol=0, atol=1e-6)
        np.testing.assert_allclose(lse[i], torch.logsumexp(logits, -1).numpy(), rtol=0, atol=1e-5)


def test_attention_closed_forms(oracle_lib):
    rng = np.random.default_rng(23)
    L, bs, H, d_qk, d_v, K = 29, 4, 2, 24, 16, 6
    bt, kl, vl, kp, vp = _attn_setup(rng, n_seq=1, L=L, bs=bs, d_qk=d_qk, d_v=d_v, H=H)
    kb, vb = bf16_bits_round(kp), bf16_bits_round(vp)
    sel = np.array([[2, 5, 11, 17, 28, -1]], np.int32)
    # q = 0: uniform weights -> mean of the kept V rows, lse = ln |S|
    zero_q = np.zeros((1, H, d_qk), np.uint16)
    out, lse = oracle_lib.sparse_attn(kb, vb, bt, bs, zero_q, [0], sel, 0.5)
    np.testing.assert_allclose(out[0, 0], vl[0][[2, 5, 11, 17, 28]].mean(0), atol=1e-6)
    np.testing.assert_allclose(lse, math.log(5.0), atol=1e-6)
    # one kept position: output is that V row, lse is its logit
    q = bf16_bits_round(rng.normal(size=(1, H, d_qk)))
    one = np.array([[17, -1, -1, -1, -1, -1]], np.int32)
    out, lse = oracle_lib.sparse_attn(kb, vb, bt, bs, q, [0], one, 0.5)
    np.testing.assert_allclose(out[0, 1], vl[0][17], atol=1e-6)
    np.testing.assert_allclose(lse[0, 1], 0.5 * bf16_float(q[0, 1]) @ kl[0][17], atol=1e-5)
    # every V row equal to c: output is c whatever the weights
    c = bf16_float(bf16_bits_round(rng.normal(size=d_v)))
    vconst = to_pool([np.tile(c, (L, 1))], bt, bs, vp.shape[0] // bs)
    out, _ = oracle_lib.sparse_attn(kb, bf16_bits_round(vconst), bt, bs, q, [0], sel, 0.5)
    np.testing.assert_allclose(out[0], np.tile(c, (H, 1)), atol=1e-6)
    # two kept positions: sigmoid weights
    two = np.array([[5, 11, -1, -1, -1, -1]], np.int32)
    out, _ = oracle_lib.sparse_attn(kb, vb, bt, bs, q, [0], two, 0.5)
    qf = bf16_float(q[0, 0])
    a = 1.0 / (1.0 + math.exp(-0.5 * (qf @ kl[0][5] - qf @ kl[0][11])))
    np.testing.assert_allclose(out[0, 0], a * vl[0][5] + (1 - a) * vl[0][11], atol=1e-6)
    # no kept position: zeros and -inf
    none = np.full((1, K), -1, np.int32)
    out, lse = oracle_lib.sparse_attn(kb, vb, bt, bs, q, [0], none, 0.5)
    assert (out == 0).all() and np.isneginf(lse).all()


def test_latent_value_is_prefix_of_key_row(oracle_lib):
    """With no separate V pool, V is the first d_v columns of each K row."""
    rng = np.random.default_rng(24)
    bt, kl, vl, kp, vp = _attn_setup(rng, n_seq=1, L=29, bs=4, d_qk=24, d_v=16, H=2)
    kb = bf16_bits_round(kp)
    q = bf16_bits_round(rng.normal(size=(1, 2, 24)))
    sel = np.array([[0, 3, 9, 28]], np.int32)
    a, la = oracle_lib.sparse_attn(kb, None, bt, 4, q, [0], sel, 0.2, d_v=16)
    b, lb = oracle_lib.sparse_attn(kb, np.ascontiguousarray(kb[:, :16]), bt, 4, q, [0], sel, 0.2)
    np.testing.assert_array_equal(a, b)
    np.testing.assert_array_equal(la, lb)


# ----------------------------------------------------------------------------- cache write

def test_hand_worked_cache_write(oracle_lib):
    g = json.load(open(GOLDEN))["cache_write"]
    pool = np.zeros((g["pool_rows"], 2), np.uint16)
    toks = g["tokens"]
    oracle_lib.cache_write(pool, np.array(g["block_table"], np.int32), g["block_size"],
                           [t["seq"] for t in toks], [t["pos"] for t in toks],
                           np.array([t["row"] for t in toks], np.uint16))
    want = np.zeros_like(pool)
    for r, row in g["written_rows"].items():
        want[int(r)] = row
    np.testing.assert_array_equal(pool, want)


def test_cache_write_then_attention_reads_the_same_rows(oracle_lib):
    """Rows written token by token through a shuffled block table, then read
    back by the oracle's attention (C code, its own gather), give the same
    result as the rows laid out contiguously with an identity table."""
    rng = np.random.default_rng(31)
    L, bs, d_qk, d_v, H = 23, 4, 24, 16, 2
    blocks = (L + bs - 1) // bs
    bt, n_blocks = random_table(rng, 2, blocks, extra=2)
    k = bf16_bits_round(rng.normal(size=(L, d_qk)))
    v = bf16_bits_round(rng.normal(size=(L, d_v)))
    kpool = np.full((n_blocks * bs, d_qk), 0x7fc0, np.uint16)   # NaN: a stray read shows
    vpool = np.full((n_blocks * bs, d_v), 0x7fc0, np.uint16)
    order = rng.permutation(L)                                  # any write order
    seq = np.ones(L, np.int32)
    oracle_lib.cache_write(kpool, bt, bs, seq, order, k[order])
    oracle_lib.cache_write(vpool, bt, bs, seq, order, v[order])
    q = bf16_bits_round(rng.normal(size=(L, H, d_qk)))
    idx = np.tile(np.arange(L, dtype=np.int32), (L, 1))
    for t in range(L):
        idx[t, t + 1:] = -1
    got, lg = oracle_lib.sparse_attn(kpool, vpool, bt, bs, q, np.ones(L, np.int32), idx, 0.3)
    ident = np.arange(blocks, dtype=np.int32).reshape(1, blocks)
    kc = np.zeros((blocks * bs, d_qk), np.uint16)
    vc = np.zeros((blocks * bs, d_v), np.uint16)
    kc[:L], vc[:L] = k, v
    want, lw = oracle_lib.sparse_attn(kc, vc, ident, bs, q, np.zeros(L, np.int32), idx, 0.3)
    np.testing.assert_array_equal(got, want)
    np.testing.assert_array_equal(lg, lw)
    # sequence 0's blocks and the spare blocks were not touched
    touched = {int(b) * bs + s for b in bt[1] for s in range(bs)}
    for r in range(n_blocks * bs):
        if r not in touched:
            assert (kpool[r] == 0x7fc0).all() and (vpool[r] == 0x7fc0).all()


def test_cache_write_skips_tokens_outside_the_table(oracle_lib):
    pool = np.zeros((8, 1), np.uint16)
    bt = np.array([[0, 1], [2, 3]], np.int32)
    oracle_lib.cache_write(pool, bt, 2, [2, -1, 0, 0], [0, 0, -1, 4], np.ones((4, 1), np.uint16))
    assert not pool.any()
