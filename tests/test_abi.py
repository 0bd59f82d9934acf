"""The C ABI without a GPU: libdsa.so loads, exports every function that
include/dsa.h and include/dsa_moe.h declare, and rejects bad arguments on the host before any
launch (on a machine with no GPU, well-formed calls stop at the device check)."""
import ctypes
import os
import re

import pytest

import sparse_attention_long_dsa_amd as dsa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in ("dsa.h", "dsa_moe.h")]


def declared_functions():
    names = set()
    for h in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"\b(dsa_\w+)\s*\(", text))
    return sorted(names)


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(dsa.LIB_PATH):
        dsa.build()
    return dsa.lib()


def test_header_declares_the_calls():
    names = declared_functions()
    for f in ("dsa_index_score", "dsa_topk", "dsa_sparse_attn_decode", "dsa_sparse_attn_prefill",
              "dsa_moe_gemm_mxfp4", "dsa_mxfp4_to_fp8", "dsa_moe_gemm_fp8",
              "dsa_moe_gemm_staged"):
        assert f in names


def test_library_exports_every_declared_symbol(L):
    cdll = ctypes.CDLL(dsa.LIB_PATH)
    for name in declared_functions():
        assert hasattr(cdll, name), name


def test_status_strings(L):
    for code in range(8):
        assert L.dsa_status_string(code)
    assert L.dsa_status_string(99) == b"unknown status"


FAKE = 0x10000  # never dereferenced: every call below returns before any device work


def cache(**kw):
    c = dict(kv=FAKE, kv_row_stride=576, v=None, v_row_stride=0, k_idx=FAKE, k_idx_row_stride=128,
             block_table=FAKE, seq_lens=FAKE, n_seq=2, max_blocks_per_seq=4, num_blocks=8,
             block_size=64, d_qk=576, d_v=512, d_idx=128)
    c.update(kw)
    return dsa.PagedCache(**c)


def score(L, c, phase=dsa.DSA_DECODE, q=FAKE, w=FAKE, q_seq=None, q_pos=None, n_q=2, H=64,
          out=FAKE, ld=256):
    return L.dsa_index_score(ctypes.byref(c), phase, q, w, q_seq, q_pos, n_q, H, out, ld, None, 0,
                             None)


def test_index_score_validation(L):
    assert L.dsa_index_score_ws(dsa.DSA_DECODE, 64, 1 << 17) == 0    # no workspace needed
    assert L.dsa_index_score_ws(dsa.DSA_PREFILL, 8192, 8192) == 0
    assert score(L, cache(), q=None) == 1
    assert score(L, cache(k_idx=None)) == 1
    assert score(L, cache(block_table=None)) == 1
    assert score(L, cache(seq_lens=None)) == 1                # decode without per-query arrays
    assert L.dsa_index_score(None, 1, FAKE, FAKE, None, None, 2, 64, FAKE, 256, None, 0,
                             None) == 1
    assert score(L, cache(), q_seq=FAKE) == 1                 # one array without the other
    assert score(L, cache(), q_pos=FAKE) == 1
    assert score(L, cache(), phase=dsa.DSA_PREFILL) == 1      # prefill needs both arrays
    assert score(L, cache(), n_q=3) == 2                      # decode: n_q must equal n_seq
    assert score(L, cache(), n_q=3, q_seq=FAKE, q_pos=FAKE) == 5   # ... unless per-query arrays
    assert score(L, cache(), ld=0) == 2
    assert score(L, cache(), phase=7) == 2
    assert score(L, cache(), H=32) == 3
    assert score(L, cache(d_idx=64, k_idx_row_stride=64)) == 3
    assert score(L, cache(k_idx_row_stride=100)) == 2        # stride below width
    assert score(L, cache()) == 5                            # well formed: no gfx950 here
    assert score(L, cache(seq_lens=None), q_seq=FAKE, q_pos=FAKE) == 5
    assert score(L, cache(), phase=dsa.DSA_PREFILL, n_q=200, q_seq=FAKE, q_pos=FAKE) == 5
    assert score(L, cache(d_idx=32, k_idx_row_stride=32), H=4) == 5
    assert score(L, cache(k_idx=FAKE + 8)) == 3              # 16-byte alignment
    assert score(L, cache(), q=FAKE + 4) == 3
    assert score(L, cache(block_size=8)) == 3                # 16-position key groups


def test_topk_validation(L):
    ws = L.dsa_topk_workspace_size(4, 1 << 20, 2048)
    assert ws >= 4 * (1 << 20) * 8
    assert L.dsa_topk_workspace_size(4, 8192, 2048) == 0     # short rows need no workspace
    f = L.dsa_topk
    assert f(None, 100, 4, 8, FAKE, 0, FAKE, None, 0, None) == 1
    assert f(FAKE, 100, 4, 8, FAKE, 0, None, None, 0, None) == 1
    assert f(FAKE, 100, 4, 0, FAKE, 0, FAKE, None, 0, None) == 2
    assert f(FAKE, 100, 4, 2049, FAKE, 0, FAKE, None, 0, None) == 2
    assert f(FAKE, 100, 0, 8, FAKE, 0, FAKE, None, 0, None) == 2
    assert f(FAKE, 100, 4, 8, None, 97, FAKE, None, 0, None) == 2   # causal rows past ld
    assert f(FAKE, 1 << 20, 4, 2048, FAKE, 0, FAKE, None, 0, None) == 4
    assert f(FAKE, 1 << 20, 4, 2048, FAKE, 0, FAKE, FAKE, ws - 1, None) == 4
    assert f(FAKE, 1 << 20, 4, 2048, FAKE, 0, FAKE, FAKE, ws, None) == 5
    assert f(FAKE, 100, 4, 8, None, 96, FAKE, None, 0, None) == 5
    assert f(FAKE, (1 << 24) + 1, 4, 8, FAKE, 0, FAKE, FAKE, 1 << 40, None) == 2   # ld bound


def test_index_topk_validation(L):
    f = L.dsa_index_topk_decode
    ws = L.dsa_index_topk_decode_ws(2, 1 << 17, 2048)
    assert ws >= 2 * (1 << 17) // 16 * 8                     # two group maxima per 16 positions
    assert L.dsa_index_topk_decode_ws(2, 1 << 20, 2048) >= 2 * (1 << 20) * 8   # long rows
    c = cache()

    def call(c=c, q=FAKE, q_seq=None, q_pos=None, n_q=2, H=64, K=2048, sc=FAKE, ld=1 << 17,
             idx=FAKE, flags=0, w=FAKE, ws_bytes=ws):
        return f(ctypes.byref(c), q, FAKE, q_seq, q_pos, n_q, H, K, sc, ld, idx, flags, w,
                 ws_bytes, None)

    assert call() == 5                                       # well formed: no gfx950 here
    assert call(q=None) == 1
    assert call(idx=None) == 1
    assert call(q_seq=FAKE) == 1
    assert call(c=cache(seq_lens=None)) == 1
    assert call(c=cache(seq_lens=None), q_seq=FAKE, q_pos=FAKE, n_q=5,
                ws_bytes=L.dsa_index_topk_decode_ws(5, 1 << 17, 2048)) == 5
    assert call(n_q=3) == 2
    assert call(K=0) == 2 and call(K=2049) == 2
    assert call(ld=(1 << 17) + 2) == 2                       # ld must be a multiple of 4
    assert call(flags=8) == 2
    assert call(flags=2 | 4) == 2                            # score-only and select-only
    assert call(flags=1) == 5 and call(flags=2) == 5 and call(flags=4) == 5
    assert call(H=32) == 3
    assert call(sc=FAKE + 4) == 3
    assert call(w=None) == 4
    assert call(ws_bytes=ws - 1) == 4


def test_index_topk_prefill_validation(L):
    f = L.dsa_index_topk_prefill
    ws = L.dsa_index_topk_prefill_ws(8192)
    assert ws == 256 * 16 * 8192 * 4                         # 512 KB per resident workgroup
    assert L.dsa_index_topk_prefill_ws(1 << 20) == ws        # bounded whatever n_q
    assert L.dsa_index_topk_prefill_ws(1) == 16 * 8192 * 4   # one 16-query block
    assert L.dsa_index_topk_prefill_ws(33) == 3 * 16 * 8192 * 4
    assert L.dsa_index_topk_prefill_ws(0) == 0

    def call(c=None, q=FAKE, w=FAKE, q_seq=FAKE, q_pos=FAKE, n_q=100, H=64, K=2048, idx=FAKE,
             work=FAKE, ws_bytes=ws):
        c = c or cache()
        return f(ctypes.byref(c), q, w, q_seq, q_pos, n_q, H, K, idx, work, ws_bytes, None)

    assert call() == 5                                       # well formed: no gfx950 here
    assert call(c=cache(seq_lens=None)) == 5                 # lengths are not read
    assert call(q=None) == 1 and call(w=None) == 1 and call(idx=None) == 1
    assert call(q_seq=None) == 1 and call(q_pos=None) == 1   # per-query arrays required
    assert call(work=None) == 1
    assert call(c=cache(k_idx=None)) == 1 and call(c=cache(block_table=None)) == 1
    assert f(None, FAKE, FAKE, FAKE, FAKE, 100, 64, 2048, FAKE, FAKE, ws, None) == 1
    assert call(n_q=0) == 2
    assert call(K=0) == 2 and call(K=2049) == 2
    assert call(c=cache(k_idx_row_stride=100)) == 2          # stride below width
    assert call(ws_bytes=L.dsa_index_topk_prefill_ws(100) - 1) == 4
    assert call(ws_bytes=L.dsa_index_topk_prefill_ws(100)) == 5
    assert call(H=32) == 3                                   # indexer shape (64, 128) only
    assert call(c=cache(d_idx=64, k_idx_row_stride=64)) == 3
    assert call(c=cache(k_idx_row_stride=132)) == 3          # rows of whole 16-byte chunks
    assert call(c=cache(block_size=8)) == 3 and call(c=cache(block_size=24)) == 3
    assert call(c=cache(k_idx=FAKE + 8)) == 3                # 16-byte alignment
    assert call(q=FAKE + 4) == 3 and call(work=FAKE + 4) == 3


def test_attention_validation(L):
    dec = L.dsa_sparse_attn_decode
    pre = L.dsa_sparse_attn_prefill
    ws = L.dsa_sparse_attn_decode_workspace_size(2, 128, 2048, 512)
    assert ws > 0
    c = cache()
    assert dec(ctypes.byref(c), None, FAKE, 2, 128, 2048, 0.1, FAKE, None, FAKE, ws, None) == 1
    assert dec(ctypes.byref(c), FAKE, FAKE, 3, 128, 2048, 0.1, FAKE, None, FAKE, ws, None) == 2
    assert dec(ctypes.byref(c), FAKE, FAKE, 2, 64, 2048, 0.1, FAKE, None, FAKE, ws, None) == 3
    assert dec(ctypes.byref(c), FAKE, FAKE, 2, 128, 4096, 0.1, FAKE, None, FAKE, ws, None) == 2
    assert dec(ctypes.byref(c), FAKE, FAKE, 2, 128, 2048, 0.1, FAKE, None, FAKE, ws - 1, None) == 4
    assert dec(ctypes.byref(c), FAKE, FAKE, 2, 128, 2048, 0.1, FAKE, None, FAKE, ws, None) == 5
    # any finite softmax scale is accepted (zero and negative too); inf / nan are not
    for scale in (0.0, -0.5, 1e30):
        assert dec(ctypes.byref(c), FAKE, FAKE, 2, 128, 2048, scale, FAKE, None, FAKE, ws,
                   None) == 5
    for scale in (float("inf"), float("-inf"), float("nan")):
        assert dec(ctypes.byref(c), FAKE, FAKE, 2, 128, 2048, scale, FAKE, None, FAKE, ws,
                   None) == 2
        assert pre(ctypes.byref(c), FAKE, FAKE, FAKE, FAKE, 100, 128, 2048, scale, FAKE, None,
                   None) == 2
    sep = cache(v=FAKE, v_row_stride=64, d_qk=64, d_v=64, kv_row_stride=64)
    assert dec(ctypes.byref(sep), FAKE, FAKE, 2, 8, 64, 0.1, FAKE, None, FAKE, 1 << 30, None) == 5
    assert dec(ctypes.byref(cache(v=FAKE, v_row_stride=512)), FAKE, FAKE, 2, 128, 2048, 0.1, FAKE,
               None, FAKE, ws, None) == 3                    # latent shape wants V inside K rows
    assert pre(ctypes.byref(c), FAKE, FAKE, FAKE, FAKE, 100, 128, 2048, 0.1, FAKE, None,
               None) == 5
    assert pre(ctypes.byref(c), FAKE, None, FAKE, FAKE, 100, 128, 2048, 0.1, FAKE, None,
               None) == 1                                   # per-query arrays are required
    assert pre(ctypes.byref(c), FAKE, FAKE, None, FAKE, 100, 128, 2048, 0.1, FAKE, None,
               None) == 1
    assert pre(ctypes.byref(c), None, FAKE, FAKE, FAKE, 100, 128, 2048, 0.1, FAKE, None,
               None) == 1
    assert pre(ctypes.byref(c), FAKE, FAKE, FAKE, FAKE, 0, 128, 2048, 0.1, FAKE, None, None) == 2
    # 16-byte alignment of the vector-loaded buffers
    for bad in (dict(kv=FAKE + 2),):
        assert dec(ctypes.byref(cache(**bad)), FAKE, FAKE, 2, 128, 2048, 0.1, FAKE, None, FAKE,
                   ws, None) == 3
    assert dec(ctypes.byref(c), FAKE + 8, FAKE, 2, 128, 2048, 0.1, FAKE, None, FAKE, ws, None) == 3
    assert dec(ctypes.byref(c), FAKE, FAKE, 2, 128, 2048, 0.1, FAKE + 4, None, FAKE, ws, None) == 3
    assert dec(ctypes.byref(c), FAKE, FAKE, 2, 128, 2048, 0.1, FAKE, None, FAKE + 4, ws, None) == 3
    assert pre(ctypes.byref(c), FAKE + 2, FAKE, FAKE, FAKE, 100, 128, 2048, 0.1, FAKE, None,
               None) == 3


def test_static_decode_validation(L):
    f = L.dsa_sparse_attn_decode_static
    c = cache()
    assert f(ctypes.byref(c), FAKE, FAKE, 2, 128, 2048, 0.1, FAKE, None, None) == 5  # fits
    assert f(ctypes.byref(c), None, FAKE, 2, 128, 2048, 0.1, FAKE, None, None) == 1
    assert f(ctypes.byref(c), FAKE, FAKE, 3, 128, 2048, 0.1, FAKE, None, None) == 2
    # 200 queries x 2 splits of fp16 partials need more than the 48 MiB array
    assert L.dsa_sparse_attn_decode_workspace_size(200, 128, 2048, 512) > 48 << 20
    big = cache(n_seq=200)
    assert f(ctypes.byref(big), FAKE, FAKE, 200, 128, 2048, 0.1, FAKE, None, None) == 4
    assert L.dsa_sparse_attn_decode_workspace_size(64, 128, 2048, 512) <= 48 << 20
    ok = cache(n_seq=64)
    assert f(ctypes.byref(ok), FAKE, FAKE, 64, 128, 2048, 0.1, FAKE, None, None) == 5


def test_device_error_check(L):
    # release build: no checks compiled in
    assert L.dsa_check_device_errors(None) == 3
    # the debug build exports the same symbols; without a GPU its calls stop
    # at the device check like the release build's
    if not os.path.exists(dsa.DEBUG_LIB_PATH):
        dsa.build(debug=True)
    D = dsa.debug_lib()
    assert score(D, cache()) == 5
    assert score(D, cache(), q=None) == 1


def test_cache_write_validation(L):
    f = L.dsa_cache_write
    c = cache()
    assert f(ctypes.byref(c), FAKE, FAKE, 4, FAKE, None, FAKE, None) == 5     # well formed
    assert f(ctypes.byref(c), FAKE, FAKE, 0, FAKE, None, FAKE, None) == 5     # device checked first
    assert f(None, FAKE, FAKE, 4, FAKE, None, FAKE, None) == 1
    assert f(ctypes.byref(c), None, FAKE, 4, FAKE, None, FAKE, None) == 1
    assert f(ctypes.byref(c), FAKE, FAKE, 4, None, None, FAKE, None) == 1
    assert f(ctypes.byref(c), FAKE, FAKE, 4, FAKE, FAKE, FAKE, None) == 1     # v_new without a V pool
    sep = cache(v=FAKE, v_row_stride=64, d_qk=64, d_v=64, kv_row_stride=64)
    assert f(ctypes.byref(sep), FAKE, FAKE, 4, FAKE, None, FAKE, None) == 1   # V pool needs v_new
    assert f(ctypes.byref(sep), FAKE, FAKE, 4, FAKE, FAKE, FAKE, None) == 5
    assert f(ctypes.byref(c), FAKE, FAKE, -1, FAKE, None, FAKE, None) == 2
    assert f(ctypes.byref(cache(kv_row_stride=500)), FAKE, FAKE, 4, FAKE, None, FAKE, None) == 2
    assert f(ctypes.byref(cache(d_qk=570, kv_row_stride=576)), FAKE, FAKE, 4, FAKE, None, FAKE,
             None) == 3
    assert f(ctypes.byref(c), FAKE, FAKE, 4, FAKE + 8, None, FAKE, None) == 3  # alignment


def weights(**kw):
    w = dict(codes=FAKE, scales=FAKE, num_experts=8, N=64, K=256)
    w.update(kw)
    return dsa.Mxfp4Weights(**w)


def test_moe_validation(L):
    f = L.dsa_moe_gemm_mxfp4
    w = weights()

    def gemm(w=w, x=FAKE, ids=FAKE, offs=FAKE, n_act=4, M=16, max_rows=4, y=FAKE):
        return f(ctypes.byref(w) if w is not None else None, x, ids, offs, n_act, M, max_rows, y,
                 None)

    assert gemm() == 5                                  # well formed: stops at the device check
    assert gemm(w=None) == 1
    assert gemm(x=None) == 1 and gemm(ids=None) == 1 and gemm(offs=None) == 1 and gemm(y=None) == 1
    assert gemm(w=weights(codes=None)) == 1
    assert gemm(n_act=0) == 2 and gemm(n_act=65536) == 2 and gemm(M=-1) == 2
    assert gemm(w=weights(num_experts=0)) == 2
    assert gemm(w=weights(K=200)) == 3                  # K not a multiple of 128
    assert gemm(w=weights(N=40)) == 3                   # N not a multiple of 16
    assert gemm(x=FAKE + 8) == 3 and gemm(w=weights(codes=FAKE + 4)) == 3
    assert gemm(w=weights(scales=FAKE + 2)) == 3
    c = L.dsa_mxfp4_to_fp8
    assert c(ctypes.byref(w), FAKE, 4, FAKE, None) == 5
    assert c(ctypes.byref(w), FAKE, 4, None, None) == 1
    assert c(ctypes.byref(w), None, 4, FAKE, None) == 1
    assert c(ctypes.byref(w), FAKE, 0, FAKE, None) == 2
    g = L.dsa_moe_gemm_fp8
    assert g(FAKE, 64, 256, FAKE, FAKE, 4, 16, 4, FAKE, None) == 5
    assert g(None, 64, 256, FAKE, FAKE, 4, 16, 4, FAKE, None) == 1
    assert g(FAKE, 64, 250, FAKE, FAKE, 4, 16, 4, FAKE, None) == 3
    assert g(FAKE, 0, 256, FAKE, FAKE, 4, 16, 4, FAKE, None) == 2
    assert L.dsa_moe_staged_ws(64, 256, 3) == 2 * 3 * 64 * 256
    assert L.dsa_moe_staged_ws(64, 256, 0) == 0
    s = L.dsa_moe_gemm_staged
    ev = (ctypes.c_void_p * 5)(FAKE, FAKE, FAKE, FAKE, FAKE)
    ws = L.dsa_moe_staged_ws(64, 256, 1)

    def staged(ws_bytes=ws, stream=None, conv=FAKE, events=ev):
        return s(ctypes.byref(w), FAKE, FAKE, FAKE, 4, 16, 4, FAKE, FAKE, ws_bytes, stream, conv,
                 events)

    assert staged() == 5
    assert staged(ws_bytes=ws - 1) == 4                 # not even one expert a half
    assert staged(events=None) == 1
    assert staged(events=(ctypes.c_void_p * 5)(FAKE, None, FAKE, FAKE, FAKE)) == 1
    assert staged(events=(ctypes.c_void_p * 5)(FAKE, FAKE, FAKE, FAKE, None)) == 1
    assert staged(conv=None) == 2                       # conversion stream == product stream
