"""Seeded synthetic inputs for the DSA workloads (shared by the oracle side and
the GPU side of every parity test and by the benchmark).

Nothing here computes any part of the attention method.  The module only
describes workloads (shapes, sizes, seeds) and fills host or device buffers
with pseudo-random values that are a pure function of (seed, tensor id,
logical coordinates); see ``synth.hip`` for the generator's definition.

Value recipes (all inclusive integer ranges):
  * attention q, K/V rows: bf16 N(0,1) (65536-quantile table, see
    ``normal_table``);
  * indexer q_idx, k_idx: bf16 integers uniform on [-3, 3];
  * indexer head weights w: fp32 integers uniform on [1, 4];
  * block tables: one seeded Fisher-Yates permutation of the physical pool,
    handed out to the sequences in order, so sequences interleave at random;
  * ragged lengths: integers uniform on [lo, hi].
Cache values are keyed by (sequence, logical position, column), so a
different block table moves values around without changing them.
"""
from __future__ import annotations

import ctypes
import dataclasses
import math
import os
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdsa_synth.so")

# tensor ids: part of every hash key, so tensors never share a stream
TID_Q, TID_KV, TID_V, TID_KIDX, TID_QIDX, TID_W, TID_BT, TID_LEN = 1, 2, 3, 4, 5, 6, 7, 8
KIND_NORMAL_BF16, KIND_INT_BF16, KIND_INT_F32 = 0, 1, 2
BF16_NAN = 0x7FC0

_lib = None
_table = None


def build(verbose: bool = False) -> str:
    """Compile libdsa_synth.so (host and gfx950 device code from one source)."""
    import subprocess

    cmd = ["/opt/rocm/bin/hipcc", "--offload-arch=gfx950", "-O3", "-fPIC", "-shared",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           os.path.join(_HERE, "synth.hip"), "-o", LIB_PATH + ".tmp"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("building libdsa_synth.so failed:\n" + r.stderr)
    os.replace(LIB_PATH + ".tmp", LIB_PATH)
    if verbose:
        print("built", LIB_PATH)
    return LIB_PATH


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: run __graft_entry__.build() first")
        L = ctypes.CDLL(LIB_PATH)
        c_i64, c_u32, c_int, c_vp = ctypes.c_int64, ctypes.c_uint32, ctypes.c_int, ctypes.c_void_p
        L.synth_hash.restype = c_u32
        L.synth_hash.argtypes = [c_u32] * 5
        L.synth_dense_host.argtypes = [c_vp, c_int, c_u32, c_u32, c_i64, c_i64, c_int, c_int,
                                       c_int, c_int, c_vp]
        L.synth_paged_host.argtypes = [c_vp, c_i64, c_int, c_u32, c_u32, c_int, c_i64, c_i64,
                                       c_int, c_vp, c_int, c_int, c_int, c_vp]
        L.synth_dense_device.argtypes = L.synth_dense_host.argtypes + [c_vp]
        L.synth_paged_device.argtypes = L.synth_paged_host.argtypes + [c_vp]
        L.synth_permutation.argtypes = [c_vp, c_int, c_u32, c_u32]
        L.synth_uniform_ints.argtypes = [c_vp, c_int, c_u32, c_u32, c_int, c_int]
        for f in (L.synth_dense_host, L.synth_paged_host, L.synth_dense_device,
                  L.synth_paged_device, L.synth_permutation, L.synth_uniform_ints):
            f.restype = c_int
        _lib = L
    return _lib


def normal_table() -> np.ndarray:
    """bf16 bits of the N(0,1) quantiles at (i + 1/2) / 65536, i = 0..65535."""
    global _table
    if _table is None:
        from scipy.special import ndtri
        import torch

        p = (np.arange(65536, dtype=np.float64) + 0.5) / 65536.0
        z = torch.from_numpy(ndtri(p).astype(np.float32)).to(torch.bfloat16)
        _table = z.view(torch.int16).numpy().view(np.uint16).copy()
    return _table


def _check(rc: int, what: str):
    if rc != 0:
        raise RuntimeError(f"{what} failed with code {rc}")


# --------------------------------------------------------------------------- workloads

@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic DSA workload.

    phase "decode": query i is the last token (position seq_lens[i]-1) of
    sequence i.  phase "prefill": one sequence; query t is position t and every
    position of the sequence is a query.
    """
    name: str
    phase: str
    seq_lens: tuple
    block_size: int
    H: int
    d_qk: int
    d_v: int
    separate_v: bool
    H_idx: int
    d_idx: int
    topk: int
    sm_scale: float
    seed: int
    table_seed: int = -1   # seed of the block-table shuffle; -1: use `seed`

    @property
    def n_seq(self) -> int:
        return len(self.seq_lens)

    @property
    def n_q(self) -> int:
        return self.n_seq if self.phase == "decode" else self.seq_lens[0]

    @property
    def blocks_per_seq(self) -> list:
        return [(L + self.block_size - 1) // self.block_size for L in self.seq_lens]

    @property
    def pool_blocks(self) -> int:
        return sum(self.blocks_per_seq)

    @property
    def max_blocks(self) -> int:
        return max(self.blocks_per_seq)

    @property
    def kv_cols(self) -> int:
        return self.d_qk

    def query_seq_pos(self):
        """(seq, pos) of every query, as int32 arrays."""
        if self.phase == "decode":
            seq = np.arange(self.n_seq, dtype=np.int32)
            pos = np.asarray(self.seq_lens, dtype=np.int32) - 1
        else:
            T = self.seq_lens[0]
            seq = np.zeros(T, dtype=np.int32)
            pos = np.arange(T, dtype=np.int32)
        return seq, pos

    def query_key(self, i: int) -> int:
        """The logical coordinate that keys query i's values in the generator."""
        return i


def ragged_lengths(n: int, lo: int, hi: int, seed: int) -> tuple:
    out = np.zeros(n, dtype=np.int32)
    _check(lib().synth_uniform_ints(out.ctypes.data, n, seed, TID_LEN, lo, hi), "lengths")
    return tuple(int(x) for x in out)


def latent(name, phase, seq_lens, seed, topk=2048, block_size=64, H=128, H_idx=64,
           table_seed=-1) -> Workload:
    """The 576-wide shared-latent shape: V is the first 512 columns of each K row."""
    return Workload(name=name, phase=phase, seq_lens=tuple(seq_lens), block_size=block_size,
                    H=H, d_qk=576, d_v=512, separate_v=False, H_idx=H_idx, d_idx=128,
                    topk=topk, sm_scale=1.0 / math.sqrt(576.0), seed=seed, table_seed=table_seed)


def small_mqa(name, phase, seq_lens, seed, topk=64, block_size=16, table_seed=-1) -> Workload:
    """The small shape: 8 query heads on one K and one V head of width 64."""
    return Workload(name=name, phase=phase, seq_lens=tuple(seq_lens), block_size=block_size,
                    H=8, d_qk=64, d_v=64, separate_v=True, H_idx=4, d_idx=32, topk=topk,
                    sm_scale=1.0 / 8.0, seed=seed, table_seed=table_seed)


def workload(n: int) -> Workload:
    """The five reference workloads (seed n for workload n)."""
    if n == 1:   # tiny decode: 1 query at position 1023, 64 blocks of 16
        return small_mqa("tiny_decode_L1024", "decode", [1024], seed=1)
    if n == 2:   # batched decode: 32 x 32768
        return latent("batched_decode_B32_L32768", "decode", [32768] * 32, seed=2)
    if n == 3:   # causal prefill of 8192 tokens
        return latent("causal_prefill_T8192", "prefill", [8192], seed=3)
    if n == 4:   # ragged decode: 64 lengths uniform on [4096, 131072]
        return latent("ragged_decode_B64_L4K-128K", "decode",
                      ragged_lengths(64, 4096, 131072, seed=4), seed=4)
    if n == 5:   # million-token decode: 8 x 1048576
        return latent("million_decode_B8_L1M", "decode", [1 << 20] * 8, seed=5)
    raise ValueError(n)


def block_table(wl: Workload) -> np.ndarray:
    """[n_seq, max_blocks] int32; entries past a sequence's last block are 0."""
    perm = np.zeros(wl.pool_blocks, dtype=np.int32)
    tseed = wl.seed if wl.table_seed < 0 else wl.table_seed
    _check(lib().synth_permutation(perm.ctypes.data, wl.pool_blocks, tseed, TID_BT), "perm")
    bt = np.zeros((wl.n_seq, wl.max_blocks), dtype=np.int32)
    off = 0
    for b, nb in enumerate(wl.blocks_per_seq):
        bt[b, :nb] = perm[off:off + nb]
        off += nb
    return bt


# --------------------------------------------------------------------------- host fill

def host_dense(kind, seed, tid, a0, na, nb, nc, lo=0, hi=0) -> np.ndarray:
    dt = np.float32 if kind == KIND_INT_F32 else np.uint16
    out = np.empty((na, nb, nc), dtype=dt)
    tab = normal_table()
    _check(lib().synth_dense_host(out.ctypes.data, kind, seed, tid, a0, na, nb, nc, lo, hi,
                                  tab.ctypes.data), "dense")
    return out


def host_paged(pool: np.ndarray, kind, seed, tid, seq, pos0, npos, bt_row: np.ndarray, bs,
               lo=0, hi=0, nc: Optional[int] = None):
    """Fill logical rows [pos0, pos0+npos) of one sequence into a [rows, cols] pool."""
    assert pool.flags.c_contiguous and bt_row.dtype == np.int32
    bt_row = np.ascontiguousarray(bt_row)
    ncols = pool.shape[-1] if nc is None else nc
    tab = normal_table()
    _check(lib().synth_paged_host(pool.ctypes.data, pool.shape[-1], kind, seed, tid, seq, pos0,
                                  npos, ncols, bt_row.ctypes.data, bs, lo, hi, tab.ctypes.data),
           "paged")


@dataclasses.dataclass
class HostCase:
    """All inputs of a workload in host memory (numpy; bf16 as uint16 bits)."""
    wl: Workload
    block_table: np.ndarray      # [n_seq, max_blocks] int32
    seq_lens: np.ndarray         # [n_seq] int32
    kv: np.ndarray               # [pool_blocks*bs, d_qk] uint16 (K rows; latent rows)
    v: Optional[np.ndarray]      # [pool_blocks*bs, d_v] uint16 or None (V = kv[:, :d_v])
    k_idx: np.ndarray            # [pool_blocks*bs, d_idx] uint16
    q: np.ndarray                # [n_q, H, d_qk] uint16
    q_idx: np.ndarray            # [n_q, H_idx, d_idx] uint16
    w: np.ndarray                # [n_q, H_idx] float32
    q_seq: np.ndarray            # [n_q] int32
    q_pos: np.ndarray            # [n_q] int32


def host_case(wl: Workload, with_kv: bool = True, poison: bool = True) -> HostCase:
    """Generate a whole workload on the host.  Unused pool slots hold NaN."""
    bt = block_table(wl)
    rows = wl.pool_blocks * wl.block_size
    fill = BF16_NAN if poison else 0
    kv = np.full((rows if with_kv else 0, wl.d_qk), fill, dtype=np.uint16)
    v = np.full((rows if with_kv else 0, wl.d_v), fill, dtype=np.uint16) if wl.separate_v else None
    k_idx = np.full((rows, wl.d_idx), fill, dtype=np.uint16)
    for b, L in enumerate(wl.seq_lens):
        host_paged(k_idx, KIND_INT_BF16, wl.seed, TID_KIDX, b, 0, L, bt[b], wl.block_size, -3, 3)
        if with_kv:
            host_paged(kv, KIND_NORMAL_BF16, wl.seed, TID_KV, b, 0, L, bt[b], wl.block_size)
            if v is not None:
                host_paged(v, KIND_NORMAL_BF16, wl.seed, TID_V, b, 0, L, bt[b], wl.block_size)
    n_q = wl.n_q
    q = host_dense(KIND_NORMAL_BF16, wl.seed, TID_Q, 0, n_q, wl.H, wl.d_qk)
    q_idx = host_dense(KIND_INT_BF16, wl.seed, TID_QIDX, 0, n_q, wl.H_idx, wl.d_idx, -3, 3)
    w = host_dense(KIND_INT_F32, wl.seed, TID_W, 0, n_q, wl.H_idx, 1, 1, 4).reshape(n_q, wl.H_idx)
    q_seq, q_pos = wl.query_seq_pos()
    return HostCase(wl, bt, np.asarray(wl.seq_lens, dtype=np.int32), kv, v, k_idx, q, q_idx, w,
                    q_seq, q_pos)


def host_query_rows(wl: Workload, i0: int, n: int):
    """q, q_idx, w of queries [i0, i0+n) only (for sampled checks at full size)."""
    q = host_dense(KIND_NORMAL_BF16, wl.seed, TID_Q, i0, n, wl.H, wl.d_qk)
    q_idx = host_dense(KIND_INT_BF16, wl.seed, TID_QIDX, i0, n, wl.H_idx, wl.d_idx, -3, 3)
    w = host_dense(KIND_INT_F32, wl.seed, TID_W, i0, n, wl.H_idx, 1, 1, 4).reshape(n, wl.H_idx)
    return q, q_idx, w


def host_kept_pool(wl: Workload, seq: int, positions: Sequence[int]):
    """K/V rows of only the listed positions of one sequence, in a compact
    pool addressed with block size 1: returns (table [1, L] int32, kv [m,
    d_qk], v [m, d_v] or None) where table[0, p] is the pool row of a listed
    position p (0 for the others, which must not be read).  Values are the
    ones every other fill gives (keyed by sequence, position and column)."""
    L = wl.seq_lens[seq]
    keep = sorted(set(int(x) for x in positions if x >= 0))
    table = np.zeros((1, L), dtype=np.int32)
    table[0, keep] = np.arange(len(keep), dtype=np.int32)
    m = max(1, len(keep))
    kv = np.full((m, wl.d_qk), BF16_NAN, dtype=np.uint16)
    v = np.full((m, wl.d_v), BF16_NAN, dtype=np.uint16) if wl.separate_v else None
    for p in keep:
        host_paged(kv, KIND_NORMAL_BF16, wl.seed, TID_KV, seq, p, 1, table[0], 1)
        if v is not None:
            host_paged(v, KIND_NORMAL_BF16, wl.seed, TID_V, seq, p, 1, table[0], 1)
    return table, kv, v


def host_sequence_pools(wl: Workload, seq: int, kv_positions: Optional[Sequence[int]] = None):
    """k_idx for every position of one sequence, plus K/V rows for only the
    positions listed (others NaN), laid out in a private pool whose block
    table is that sequence's own row.  Used for sampled checks at sizes where
    the whole cache does not fit in host memory."""
    bt = block_table(wl)[seq:seq + 1]
    nb = wl.blocks_per_seq[seq]
    # remap this sequence's blocks onto 0..nb-1, keeping their order in the pool
    phys = bt[0, :nb]
    order = np.argsort(phys, kind="stable")
    local = np.empty(nb, dtype=np.int32)
    local[order] = np.arange(nb, dtype=np.int32)
    lbt = np.zeros((1, wl.max_blocks), dtype=np.int32)
    lbt[0, :nb] = local
    rows = nb * wl.block_size
    L = wl.seq_lens[seq]
    k_idx = np.full((rows, wl.d_idx), BF16_NAN, dtype=np.uint16)
    host_paged(k_idx, KIND_INT_BF16, wl.seed, TID_KIDX, seq, 0, L, lbt[0], wl.block_size, -3, 3)
    if kv_positions is None:  # indexer keys only
        return lbt, k_idx, None, None
    kv = np.full((rows, wl.d_qk), BF16_NAN, dtype=np.uint16)
    v = np.full((rows, wl.d_v), BF16_NAN, dtype=np.uint16) if wl.separate_v else None
    if kv_positions is not None:
        for p in sorted(set(int(x) for x in kv_positions if x >= 0)):
            host_paged(kv, KIND_NORMAL_BF16, wl.seed, TID_KV, seq, p, 1, lbt[0], wl.block_size)
            if v is not None:
                host_paged(v, KIND_NORMAL_BF16, wl.seed, TID_V, seq, p, 1, lbt[0], wl.block_size)
    return lbt, k_idx, kv, v


# --------------------------------------------------------------------------- device fill

@dataclasses.dataclass
class DeviceCase:
    """All inputs of a workload in device memory (torch tensors)."""
    wl: Workload
    block_table: "torch.Tensor"  # [n_seq, max_blocks] int32
    seq_lens: "torch.Tensor"     # [n_seq] int32
    kv: "torch.Tensor"           # [pool_blocks, bs, d_qk] bf16
    v: "Optional[torch.Tensor]"  # [pool_blocks, bs, d_v] bf16 or None
    k_idx: "torch.Tensor"        # [pool_blocks, bs, d_idx] bf16
    q: "torch.Tensor"            # [n_q, H, d_qk] bf16
    q_idx: "torch.Tensor"        # [n_q, H_idx, d_idx] bf16
    w: "torch.Tensor"            # [n_q, H_idx] float32


def device_case(wl: Workload, device="cuda", poison: bool = True) -> DeviceCase:
    """Generate a whole workload directly in device memory (same values as
    ``host_case``).  Unused pool slots hold NaN when ``poison``."""
    import torch

    L = lib()
    stream = torch.cuda.current_stream(device).cuda_stream
    tab = torch.from_numpy(normal_table().view(np.int16)).to(device)
    bt_h = block_table(wl)
    bt = torch.from_numpy(bt_h).to(device)
    nb, bs = wl.pool_blocks, wl.block_size
    fill = float("nan") if poison else 0.0
    kv = torch.full((nb, bs, wl.d_qk), fill, dtype=torch.bfloat16, device=device)
    v = (torch.full((nb, bs, wl.d_v), fill, dtype=torch.bfloat16, device=device)
         if wl.separate_v else None)
    k_idx = torch.full((nb, bs, wl.d_idx), fill, dtype=torch.bfloat16, device=device)
    chunk = 1 << 16
    for b, Lb in enumerate(wl.seq_lens):
        row = bt[b]
        for p0 in range(0, Lb, chunk):
            n = min(chunk, Lb - p0)
            _check(L.synth_paged_device(k_idx.data_ptr(), wl.d_idx, KIND_INT_BF16, wl.seed,
                                        TID_KIDX, b, p0, n, wl.d_idx, row.data_ptr(), bs, -3, 3,
                                        tab.data_ptr(), stream), "paged k_idx")
            _check(L.synth_paged_device(kv.data_ptr(), wl.d_qk, KIND_NORMAL_BF16, wl.seed, TID_KV,
                                        b, p0, n, wl.d_qk, row.data_ptr(), bs, 0, 0,
                                        tab.data_ptr(), stream), "paged kv")
            if v is not None:
                _check(L.synth_paged_device(v.data_ptr(), wl.d_v, KIND_NORMAL_BF16, wl.seed,
                                            TID_V, b, p0, n, wl.d_v, row.data_ptr(), bs, 0, 0,
                                            tab.data_ptr(), stream), "paged v")
    n_q = wl.n_q
    q = torch.empty((n_q, wl.H, wl.d_qk), dtype=torch.bfloat16, device=device)
    q_idx = torch.empty((n_q, wl.H_idx, wl.d_idx), dtype=torch.bfloat16, device=device)
    w = torch.empty((n_q, wl.H_idx), dtype=torch.float32, device=device)
    _check(L.synth_dense_device(q.data_ptr(), KIND_NORMAL_BF16, wl.seed, TID_Q, 0, n_q, wl.H,
                                wl.d_qk, 0, 0, tab.data_ptr(), stream), "q")
    _check(L.synth_dense_device(q_idx.data_ptr(), KIND_INT_BF16, wl.seed, TID_QIDX, 0, n_q,
                                wl.H_idx, wl.d_idx, -3, 3, tab.data_ptr(), stream), "q_idx")
    _check(L.synth_dense_device(w.data_ptr(), KIND_INT_F32, wl.seed, TID_W, 0, n_q, wl.H_idx, 1,
                                1, 4, tab.data_ptr(), stream), "w")
    torch.cuda.synchronize(device)
    seq_lens = torch.tensor(wl.seq_lens, dtype=torch.int32, device=device)
    return DeviceCase(wl, bt, seq_lens, kv, v, k_idx, q, q_idx, w)
