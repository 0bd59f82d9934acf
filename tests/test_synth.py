"""The seeded input generator: determinism, value ranges, block tables, and
that paged filling stores each logical value where the block table says."""
import numpy as np
import pytest


def test_hash_is_deterministic_and_spreads(synth):
    L = synth.lib()
    a = [L.synth_hash(5, 2, i, 7, 9) for i in range(2000)]
    b = [L.synth_hash(5, 2, i, 7, 9) for i in range(2000)]
    assert a == b
    assert len(set(a)) == 2000
    bits = np.array(a, dtype=np.uint64)
    ones = np.array([((bits >> k) & 1).mean() for k in range(32)])
    assert (abs(ones - 0.5) < 0.06).all()


def test_value_ranges(synth):
    ints = synth.host_dense(synth.KIND_INT_BF16, 3, synth.TID_QIDX, 0, 50, 16, 32, -3, 3)
    vals = (ints.astype(np.uint32) << 16).view(np.float32)
    assert set(np.unique(vals).tolist()) == set(range(-3, 4))
    w = synth.host_dense(synth.KIND_INT_F32, 3, synth.TID_W, 0, 400, 64, 1, 1, 4)
    assert set(np.unique(w).tolist()) == {1.0, 2.0, 3.0, 4.0}
    z = synth.host_dense(synth.KIND_NORMAL_BF16, 3, synth.TID_Q, 0, 64, 128, 128)
    zf = (z.astype(np.uint32) << 16).view(np.float32)
    assert abs(zf.mean()) < 0.01 and abs(zf.std() - 1.0) < 0.01
    assert np.isfinite(zf).all() and abs(zf).max() < 4.5


def test_normal_table_is_symmetric_and_sorted(synth):
    t = synth.normal_table()
    f = (t.astype(np.uint32) << 16).view(np.float32)
    assert (np.diff(f) >= 0).all()
    np.testing.assert_array_equal(f, -f[::-1])


def test_block_tables(synth):
    for n in (1, 2, 3, 4):
        wl = synth.workload(n)
        bt = synth.block_table(wl)
        used = np.concatenate([bt[b, :nb] for b, nb in enumerate(wl.blocks_per_seq)])
        assert sorted(used.tolist()) == list(range(wl.pool_blocks))
        np.testing.assert_array_equal(bt, synth.block_table(wl))


def test_workload_shapes(synth):
    w1 = synth.workload(1)
    assert (w1.n_q, w1.seq_lens, w1.block_size, w1.pool_blocks) == (1, (1024,), 16, 64)
    assert (w1.H, w1.d_qk, w1.d_v, w1.H_idx, w1.d_idx, w1.topk) == (8, 64, 64, 4, 32, 64)
    w2 = synth.workload(2)
    assert (w2.n_q, w2.pool_blocks, w2.d_qk, w2.d_v, w2.H, w2.H_idx, w2.d_idx) == (
        32, 16384, 576, 512, 128, 64, 128)
    w3 = synth.workload(3)
    assert (w3.phase, w3.n_q, w3.pool_blocks) == ("prefill", 8192, 128)
    w4 = synth.workload(4)
    assert w4.n_q == 64 and min(w4.seq_lens) >= 4096 and max(w4.seq_lens) <= 131072
    assert w4.seq_lens == synth.workload(4).seq_lens
    w5 = synth.workload(5)
    assert (w5.n_q, w5.pool_blocks, w5.seq_lens[0]) == (8, 131072, 1 << 20)


def test_paged_fill_matches_logical_values(synth):
    """Reading the pool through the block table gives the values the generator
    assigns to (sequence, position, column), whatever the table."""
    wl = synth.small_mqa("t", "decode", [50, 33, 17], seed=9, block_size=8)
    case = synth.host_case(wl)
    for b, L in enumerate(wl.seq_lens):
        logical = synth.host_dense(synth.KIND_INT_BF16, wl.seed, synth.TID_KIDX, b, 1, L,
                                   wl.d_idx, -3, 3)[0]
        kvl = synth.host_dense(synth.KIND_NORMAL_BF16, wl.seed, synth.TID_KV, b, 1, L,
                               wl.d_qk)[0]
        rows = case.block_table[b, np.arange(L) // 8] * 8 + np.arange(L) % 8
        np.testing.assert_array_equal(case.k_idx[rows], logical)
        np.testing.assert_array_equal(case.kv[rows], kvl)
    # slots past each sequence's end stay poisoned (NaN)
    used = np.zeros(case.k_idx.shape[0], bool)
    for b, L in enumerate(wl.seq_lens):
        used[case.block_table[b, np.arange(L) // 8] * 8 + np.arange(L) % 8] = True
    assert (case.k_idx[~used] == synth.BF16_NAN).all()


def test_sequence_pool_matches_full_case(synth):
    wl = synth.latent("t", "decode", [200, 130], seed=4, topk=16, block_size=64)
    full = synth.host_case(wl)
    lbt, k_idx, kv, _ = synth.host_sequence_pools(wl, 1, kv_positions=[0, 5, 129])
    L = wl.seq_lens[1]
    rows_full = full.block_table[1, np.arange(L) // 64] * 64 + np.arange(L) % 64
    rows_loc = lbt[0, np.arange(L) // 64] * 64 + np.arange(L) % 64
    np.testing.assert_array_equal(k_idx[rows_loc], full.k_idx[rows_full])
    for p in (0, 5, 129):
        np.testing.assert_array_equal(kv[rows_loc[p]], full.kv[rows_full[p]])
