"""The bench's roofline arithmetic against figures worked out by hand from
the workload definitions (no GPU): algorithmic bytes of a decode step and of
its index-score launch, algorithmic flops of the causal prefill."""
import bench
import dsa_synth


def test_batched_decode_bytes():
    # 32 sequences x 32768 positions, block size 64, 128 heads on a 576-wide
    # latent row (512 value columns), indexer 64 x 128, Top-K 2048
    k_idx = 32 * 32768 * 128 * 2          # every candidate's indexer key
    gather = 32 * 2048 * 576 * 2          # the kept latent rows
    q = 32 * 128 * 576 * 2
    q_idx = 32 * 64 * 128 * 2 + 32 * 64 * 4   # indexer queries + head weights
    table = 32 * (32768 // 64) * 4        # block-table entries
    idx = 2 * 32 * 2048 * 4               # kept positions, written and read
    out = 32 * 128 * 512 * 2 + 32 * 128 * 4   # output + log-sum-exp
    step, launch = bench.decode_bytes(dsa_synth.workload(2))
    assert step == k_idx + gather + q + q_idx + table + idx + out == 353_984_512
    assert launch == k_idx + q_idx + table == 269_033_472


def test_million_token_index_launch_bytes():
    # 8 sequences x 2^20 positions: 0.27 GB of indexer keys per sequence
    k_idx = 8 * 2**20 * 128 * 2
    q_idx = 8 * 64 * 128 * 2 + 8 * 64 * 4
    table = 8 * (2**20 // 64) * 4
    _, launch = bench.decode_bytes(dsa_synth.workload(5))
    assert launch == k_idx + q_idx + table == 2_148_141_056


def test_ragged_decode_counts_each_sequence_by_its_length():
    wl = dsa_synth.workload(4)
    L = wl.seq_lens
    step, launch = bench.decode_bytes(wl)
    assert launch == (sum(L) * 256 + 64 * 64 * 128 * 2 + 64 * 64 * 4
                      + sum((x + 63) // 64 for x in L) * 4)
    kept = sum(min(2048, x) for x in L)
    assert step - launch == (kept * 1152 + 64 * 128 * 576 * 2 + 2 * 64 * 2048 * 4
                             + 64 * 128 * 512 * 2 + 64 * 128 * 4)


def test_prefill_flops():
    # indexer: 2 * 128 dims * 64 heads per causal pair; attention:
    # 2 * 128 heads * (576 + 512) per kept pair, min(2048, t + 1) kept for query t
    T = 8192
    pairs = T * (T + 1) // 2
    kept = 2048 * 2049 // 2 + (T - 2048) * 2048
    fi, fa = bench.prefill_flops(dsa_synth.workload(3))
    assert kept == 14_681_088
    assert fi == 2 * 128 * 64 * pairs == 549_822_922_752
    assert fa == 2 * 128 * (576 + 512) * kept == 4_089_094_078_464
