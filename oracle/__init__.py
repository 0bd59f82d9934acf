"""The oracle: plain CPU statement of the DSA hot path (index score, Top-K,
exact sparse attention over a block-paged cache), in C with double
accumulation (``dsa_oracle.c``), plus this ctypes wrapper.

TEST INFRASTRUCTURE ONLY: imported by the test suite, the smoke check and the
benchmark's CPU-baseline leg, never by the GPU library.  It shares no code
with the GPU path.

Arrays are numpy; bf16 tensors are uint16 bit patterns.

Pins (see tests/test_oracle_pins.py): every function is checked against
closed forms, library routines on special cases, invariants and brute force
on tiny inputs.  No function here is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# DSA_ORACLE_LIB names another build of dsa_oracle.c to load instead (the
# mutation check of the pins builds deliberately broken copies)
LIB_PATH = os.environ.get("DSA_ORACLE_LIB") or os.path.join(_HERE, "libdsa_oracle.so")
_lib = None
SOURCES = ["dsa_oracle.c", "moe_oracle.c"]


def build(verbose: bool = False) -> str:
    """Compile the oracle (gcc -O2 -fopenmp)."""
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-Wall",
           *[os.path.join(_HERE, f) for f in SOURCES], "-o", LIB_PATH + ".tmp", "-lm"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("building the oracle failed:\n" + r.stderr)
    os.replace(LIB_PATH + ".tmp", LIB_PATH)
    if verbose:
        print("built", LIB_PATH)
    return LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, dbl = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_double
        L.oracle_index_score.argtypes = [vp, i64, vp, i32, i32, i32, vp, vp, vp, vp, i32, i32, i32,
                                         vp, i64]
        L.oracle_index_score.restype = None
        L.oracle_topk.argtypes = [vp, i64, vp, i32, i32, vp]
        L.oracle_topk.restype = None
        L.oracle_sparse_attn.argtypes = [vp, i64, vp, i64, vp, i32, i32, i32, i32, vp, vp, vp, i32,
                                         i32, i32, dbl, vp, vp]
        L.oracle_sparse_attn.restype = None
        u8 = ctypes.c_uint8
        L.oracle_fp4_value.argtypes = [u8]
        L.oracle_fp4_value.restype = dbl
        L.oracle_e8m0_value.argtypes = [u8]
        L.oracle_e8m0_value.restype = dbl
        L.oracle_e4m3_value.argtypes = [u8]
        L.oracle_e4m3_value.restype = dbl
        L.oracle_e4m3_encode.argtypes = [dbl]
        L.oracle_e4m3_encode.restype = u8
        L.oracle_mxfp4_to_fp8.argtypes = [vp, vp, vp, i32, i32, i32, vp]
        L.oracle_mxfp4_to_fp8.restype = None
        L.oracle_moe_gemm.argtypes = [vp, vp, vp, i32, vp, vp, i32, i32, vp, vp]
        L.oracle_moe_gemm.restype = None
        _lib = L
    return _lib


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a, a.ctypes.data


def index_score(k_idx, block_table, block_size, q_idx, w, q_seq, q_pos, relu=True, ld=None):
    """scores[i, s] = sum_h w[i,h] * relu(q_idx[i,h,:] . k_idx(seq_i, s)) for s <= q_pos[i].

    k_idx: [rows, d_idx] (or [blocks, bs, d_idx]) uint16 pool; block_table
    [n_seq, max_blocks] int32; q_idx [n_q, H_idx, d_idx] uint16; w [n_q, H_idx]
    float32.  Returns float32 [n_q, ld]; entries past q_pos[i] are NaN."""
    k_idx = np.ascontiguousarray(k_idx, dtype=np.uint16)
    d_idx = k_idx.shape[-1]
    k_idx = k_idx.reshape(-1, d_idx)
    bt, bt_p = _c(block_table, np.int32)
    qi, qi_p = _c(q_idx, np.uint16)
    w_, w_p = _c(w, np.float32)
    qs, qs_p = _c(q_seq, np.int32)
    qp, qp_p = _c(q_pos, np.int32)
    n_q, H_idx = qi.shape[0], qi.shape[1]
    assert qi.shape[2] == d_idx and w_.shape == (n_q, H_idx)
    if ld is None:
        ld = int(qp.max()) + 1 if n_q else 1
    out = np.full((n_q, ld), np.nan, dtype=np.float32)
    _load().oracle_index_score(k_idx.ctypes.data, d_idx, bt_p, bt.shape[1], block_size, d_idx,
                               qi_p, w_p, qs_p, qp_p, n_q, H_idx, 1 if relu else 0,
                               out.ctypes.data, ld)
    return out


def topk(scores, n_valid, K):
    """idx[i, :] = positions of the K largest of scores[i, :n_valid[i]] (ties:
    lower position first), ascending, padded with -1.  int32 [n_q, K]."""
    sc, sc_p = _c(scores, np.float32)
    nv, nv_p = _c(n_valid, np.int32)
    n_q = sc.shape[0]
    assert nv.shape == (n_q,) and (nv <= sc.shape[1]).all()
    idx = np.empty((n_q, K), dtype=np.int32)
    _load().oracle_topk(sc_p, sc.shape[1], nv_p, n_q, K, idx.ctypes.data)
    return idx


def sparse_attn(k_pool, v_pool, block_table, block_size, q, q_seq, idx, sm_scale, d_v=None):
    """Exact softmax attention of every (query, head) over its kept positions.

    k_pool [rows, d_qk] uint16; v_pool [rows, >= d_v] uint16 or None (then
    V = first d_v columns of k_pool); q [n_q, H, d_qk] uint16; idx [n_q, K]
    int32.  Returns (out float32 [n_q, H, d_v], lse float32 [n_q, H])."""
    k_pool = np.ascontiguousarray(k_pool, dtype=np.uint16)
    d_qk = k_pool.shape[-1]
    k_pool = k_pool.reshape(-1, d_qk)
    if v_pool is None:
        v_pool = k_pool
        assert d_v is not None
    else:
        v_pool = np.ascontiguousarray(v_pool, dtype=np.uint16)
        v_pool = v_pool.reshape(-1, v_pool.shape[-1])
        d_v = v_pool.shape[-1] if d_v is None else d_v
    bt, bt_p = _c(block_table, np.int32)
    q_, q_p = _c(q, np.uint16)
    qs, qs_p = _c(q_seq, np.int32)
    ix, ix_p = _c(idx, np.int32)
    n_q, H = q_.shape[0], q_.shape[1]
    assert q_.shape[2] == d_qk and ix.shape[0] == n_q
    out = np.empty((n_q, H, d_v), dtype=np.float32)
    lse = np.empty((n_q, H), dtype=np.float32)
    _load().oracle_sparse_attn(k_pool.ctypes.data, k_pool.shape[1], v_pool.ctypes.data,
                               v_pool.shape[1], bt_p, bt.shape[1], block_size, d_qk, d_v, q_p, qs_p,
                               ix_p, n_q, H, ix.shape[1], float(sm_scale), out.ctypes.data,
                               lse.ctypes.data)
    return out, lse


def cache_write(pool, block_table, block_size, seq, pos, new):
    """Paged cache write, in place: token i of sequence seq[i] at logical
    position pos[i] goes to physical row block_table[seq[i], pos[i] //
    block_size] * block_size + pos[i] % block_size of `pool` (viewed as
    [rows, width]); new[i] fills the first new.shape[1] columns of that row.
    Tokens whose sequence, position or block lies outside the table or the
    pool are skipped.  Page "Day-0 Adaptation of Trillion-Parameter MoE
    Models on Domestic GPUs", section 3 item (2) (paged layout); page
    "Day-0 Adaptation of Ultra-Large-Scale MoE Models on Heterogeneous AI
    Accelerators", section 4 (the written layout is the read layout)."""
    rows = pool.reshape(-1, pool.shape[-1])
    bt = np.asarray(block_table)
    n_seq, max_blocks = bt.shape
    n_rows = rows.shape[0]
    for i in range(len(seq)):
        b, p = int(seq[i]), int(pos[i])
        if b < 0 or b >= n_seq or p < 0 or p // block_size >= max_blocks:
            continue
        blk = int(bt[b, p // block_size])
        r = blk * block_size + p % block_size
        if blk < 0 or r >= n_rows:
            continue
        rows[r, :new.shape[1]] = new[i]


def decode_step(case, K=None):
    """The whole decode path on a host case from dsa_synth: scores, Top-K, attention."""
    wl = case.wl
    K = wl.topk if K is None else K
    ld = int(case.q_pos.max()) + 1
    sc = index_score(case.k_idx, case.block_table, wl.block_size, case.q_idx, case.w, case.q_seq,
                     case.q_pos, ld=ld)
    idx = topk(sc, case.q_pos + 1, K)
    out, lse = sparse_attn(case.kv, case.v, case.block_table, wl.block_size, case.q, case.q_seq,
                           idx, wl.sm_scale, d_v=wl.d_v)
    return sc, idx, out, lse


# ----------------------------------------------------------------------------- MoE experts
# (web pages "Day-0 Adaptation of Trillion-Parameter MoE Models on Domestic
# GPUs", section 4; "Technical Path for Day-0 Adaptation of Trillion-Parameter
# Models on Domestic GPUs", section 3.2: MXFP4 expert weights converted to FP8
# just before the expert matrix product)

def fp4_value(code: int) -> float:
    """FP4 E2M1 code (0..15) -> value."""
    return _load().oracle_fp4_value(code)


def e8m0_value(code: int) -> float:
    """E8M0 scale code -> 2^(code-127) (NaN for 255)."""
    return _load().oracle_e8m0_value(code)


def e4m3_value(code: int) -> float:
    """FP8 E4M3 (OCP E4M3FN) code -> value."""
    return _load().oracle_e4m3_value(code)


def e4m3_encode(x: float) -> int:
    """Real -> E4M3 code: round to nearest even, saturate at +-448."""
    return _load().oracle_e4m3_encode(float(x))


def mxfp4_to_fp8(codes, scales, expert_ids, N, K):
    """E4M3 codes [E, N, K] of the listed experts' MXFP4 weights
    (codes [experts, N, K/2] uint8, scales [experts, N, K/32] uint8)."""
    c, c_p = _c(codes, np.uint8)
    s_, s_p = _c(scales, np.uint8)
    ids, ids_p = _c(expert_ids, np.int32)
    out = np.empty((len(ids), N, K), dtype=np.uint8)
    _load().oracle_mxfp4_to_fp8(c_p, s_p, ids_p, len(ids), N, K, out.ctypes.data)
    return out


def moe_gemm(x, row_offsets, expert_ids, codes, scales, N, K):
    """y[r, n] = sum_k x[r, k] w8[n, k] for the rows of each listed expert
    (x: E4M3 codes [M, K] uint8; row_offsets [E+1]).  fp32 [M, N]."""
    x_, x_p = _c(x, np.uint8)
    ro, ro_p = _c(row_offsets, np.int32)
    ids, ids_p = _c(expert_ids, np.int32)
    c, c_p = _c(codes, np.uint8)
    s_, s_p = _c(scales, np.uint8)
    M = x_.shape[0]
    y = np.zeros((M, N), dtype=np.float32)
    w8 = np.empty((N, K), dtype=np.uint8)
    _load().oracle_moe_gemm(x_p, ro_p, ids_p, len(ids), c_p, s_p, N, K, w8.ctypes.data,
                            y.ctypes.data)
    return y
