"""DSA sparse attention on MI355X (gfx950): Python binding of libdsa.so.

Argument marshalling only.  Every step of the hot path (index score, Top-K,
paged gather, sparse attention) runs in the library's HIP kernels; torch
provides device memory and the current stream.  There is no fallback: if
libdsa.so is missing or cannot load, importing the functions below raises.

The C ABI is declared in include/dsa.h; the names here match it:
  index_score        -> dsa_index_score
  index_topk_prefill -> dsa_index_topk_prefill
  topk               -> dsa_topk
  sparse_attn_decode -> dsa_sparse_attn_decode
  sparse_attn_prefill-> dsa_sparse_attn_prefill
  cache_write        -> dsa_cache_write
  check_device_errors-> dsa_check_device_errors
and the MoE expert calls of include/dsa_moe.h:
  moe_gemm_mxfp4     -> dsa_moe_gemm_mxfp4
  mxfp4_to_fp8       -> dsa_mxfp4_to_fp8
  moe_gemm_fp8       -> dsa_moe_gemm_fp8
  moe_gemm_staged    -> dsa_moe_gemm_staged (MoeStaged holds its workspace,
                        second stream and events)
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdsa.so")
# the same sources built with DSA_DEBUG_BOUNDS: kernels check the device data
# the host cannot see (block-table entries, lengths, positions, kept indices)
DEBUG_LIB_PATH = os.path.join(_HERE, "libdsa_debug.so")
SOURCES = ["index_score.hip", "topk.hip", "sparse_attn.hip", "sparse_attn_latent.hip",
           "cache_write.hip", "moe.hip"]
HIPCC_FLAGS = ["--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17",
               # keep packed-fp32 instructions out of the generated code
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]

DSA_PREFILL, DSA_DECODE = 0, 1
DSA_MXFP4_ROW_MAJOR, DSA_MXFP4_TILED = 0, 1
DSA_TOPK_SEED_PREVIOUS, DSA_INDEX_TOPK_SCORE_ONLY, DSA_INDEX_TOPK_SELECT_ONLY = 1, 2, 4
STATUS = {0: "DSA_OK", 1: "DSA_ERR_NULL", 2: "DSA_ERR_SHAPE", 3: "DSA_ERR_UNSUPPORTED",
          4: "DSA_ERR_WORKSPACE", 5: "DSA_ERR_DEVICE", 6: "DSA_ERR_HIP", 7: "DSA_ERR_BOUNDS"}


# Per-source extra flags.  The attention kernel keeps its MFMA accumulators
# in arch VGPRs: with accumulators in AGPRs the compiler copies all of O
# between the two register files on every tile.
# the small-head kernel keeps its accumulators in ordinary VGPRs; the
# latent kernel needs the accumulation registers for its 512 x 32 output
EXTRA_FLAGS = {"sparse_attn.hip": ["-mllvm", "--amdgpu-mfma-vgpr-form"]}


def build(verbose: bool = False, debug: bool = False) -> str:
    """Compile libdsa.so (or, with debug=True, libdsa_debug.so: the same
    sources with DSA_DEBUG_BOUNDS) in-tree with hipcc for gfx950, one object
    per source, compiled in parallel."""
    import tempfile

    path = DEBUG_LIB_PATH if debug else LIB_PATH
    flags = HIPCC_FLAGS + (["-DDSA_DEBUG_BOUNDS"] if debug else [])
    with tempfile.TemporaryDirectory() as tmp:
        procs = []
        for src in SOURCES:
            obj = os.path.join(tmp, src + ".o")
            cmd = ["/opt/rocm/bin/hipcc", *flags, *EXTRA_FLAGS.get(src, []), "-c",
                   os.path.join(_HERE, "csrc", src), "-o", obj]
            procs.append((src, obj, subprocess.Popen(cmd, stdout=subprocess.PIPE,
                                                     stderr=subprocess.PIPE, text=True)))
        objs = []
        for src, obj, p in procs:
            _, err = p.communicate()
            if p.returncode != 0:
                raise RuntimeError(f"compiling {src} failed:\n" + err)
            objs.append(obj)
        cmd = ["/opt/rocm/bin/hipcc", *flags, "-shared", *objs, "-o", path + ".tmp"]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"linking {os.path.basename(path)} failed:\n" + r.stderr)
    os.replace(path + ".tmp", path)
    if verbose:
        print("built", path)
    return path


PROBE_SRC = os.path.join(_HERE, "probe", "hbm_probe.hip")
PROBE_LIB = os.path.join(_HERE, "probe", "libdsa_hbm_probe.so")


def build_probe(verbose: bool = False) -> str:
    """Compile the HBM streaming-read probe (a measurement aid, not part of
    the hot path) into its own small library."""
    cmd = ["/opt/rocm/bin/hipcc", *HIPCC_FLAGS, "-shared", PROBE_SRC, "-o", PROBE_LIB + ".tmp"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("building the HBM probe failed:\n" + r.stderr)
    os.replace(PROBE_LIB + ".tmp", PROBE_LIB)
    if verbose:
        print("built", PROBE_LIB)
    return PROBE_LIB


class Mxfp4Weights(ctypes.Structure):
    """Mirror of dsa_mxfp4_weights_t."""
    _fields_ = [("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("num_experts", ctypes.c_int32), ("N", ctypes.c_int32), ("K", ctypes.c_int32),
                ("layout", ctypes.c_int32)]


class PagedCache(ctypes.Structure):
    """Mirror of dsa_paged_cache_t."""
    _fields_ = [("kv", ctypes.c_void_p), ("kv_row_stride", ctypes.c_int64),
                ("v", ctypes.c_void_p), ("v_row_stride", ctypes.c_int64),
                ("k_idx", ctypes.c_void_p), ("k_idx_row_stride", ctypes.c_int64),
                ("block_table", ctypes.c_void_p), ("seq_lens", ctypes.c_void_p),
                ("n_seq", ctypes.c_int32), ("max_blocks_per_seq", ctypes.c_int32),
                ("num_blocks", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("d_qk", ctypes.c_int32), ("d_v", ctypes.c_int32), ("d_idx", ctypes.c_int32)]


_lib = None
_debug_lib = None


def _configure(L):
    vp, i32, i64, f32, sz = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float,
                             ctypes.c_size_t)
    pc = ctypes.POINTER(PagedCache)
    L.dsa_index_score.argtypes = [pc, i32, vp, vp, vp, vp, i32, i32, vp, i64, vp, sz, vp]
    L.dsa_index_score_ws.argtypes = [i32, i32, i64]
    L.dsa_index_score_ws.restype = sz
    L.dsa_index_topk_decode_ws.argtypes = [i32, i64, i32]
    L.dsa_index_topk_decode_ws.restype = sz
    L.dsa_index_topk_decode.argtypes = [pc, vp, vp, vp, vp, i32, i32, i32, vp, i64, vp, i32, vp,
                                        sz, vp]
    L.dsa_index_topk_prefill_ws.argtypes = [i32]
    L.dsa_index_topk_prefill_ws.restype = sz
    L.dsa_index_topk_prefill.argtypes = [pc, vp, vp, vp, vp, i32, i32, i32, vp, vp, sz, vp]
    L.dsa_topk_workspace_size.argtypes = [i32, i64, i32]
    L.dsa_topk_workspace_size.restype = sz
    L.dsa_topk.argtypes = [vp, i64, i32, i32, vp, i32, vp, vp, sz, vp]
    L.dsa_sparse_attn_decode_workspace_size.argtypes = [i32, i32, i32, i32]
    L.dsa_sparse_attn_decode_workspace_size.restype = sz
    L.dsa_sparse_attn_decode.argtypes = [pc, vp, vp, i32, i32, i32, f32, vp, vp, vp, sz, vp]
    L.dsa_sparse_attn_decode_static.argtypes = [pc, vp, vp, i32, i32, i32, f32, vp, vp, vp]
    L.dsa_sparse_attn_prefill.argtypes = [pc, vp, vp, vp, vp, i32, i32, i32, f32, vp, vp, vp]
    L.dsa_cache_write.argtypes = [pc, vp, vp, i32, vp, vp, vp, vp]
    L.dsa_check_device_errors.argtypes = [vp]
    pw = ctypes.POINTER(Mxfp4Weights)
    L.dsa_mxfp4_pack.argtypes = [pw, vp, vp, vp]
    L.dsa_moe_gemm_mxfp4.argtypes = [pw, vp, vp, vp, i32, i32, i32, vp, vp]
    L.dsa_mxfp4_to_fp8.argtypes = [pw, vp, i32, vp, vp]
    L.dsa_moe_gemm_fp8.argtypes = [vp, i32, i32, vp, vp, i32, i32, i32, vp, vp]
    L.dsa_moe_staged_ws.argtypes = [i32, i32, i32]
    L.dsa_moe_staged_ws.restype = sz
    L.dsa_moe_gemm_staged.argtypes = [pw, vp, vp, vp, i32, i32, i32, vp, vp, sz, vp, vp, vp]
    L.dsa_status_string.argtypes = [i32]
    L.dsa_status_string.restype = ctypes.c_char_p
    for f in (L.dsa_index_score, L.dsa_topk, L.dsa_index_topk_decode, L.dsa_index_topk_prefill,
              L.dsa_sparse_attn_decode,
              L.dsa_sparse_attn_decode_static, L.dsa_sparse_attn_prefill, L.dsa_cache_write,
              L.dsa_check_device_errors, L.dsa_mxfp4_pack, L.dsa_moe_gemm_mxfp4, L.dsa_mxfp4_to_fp8,
              L.dsa_moe_gemm_fp8, L.dsa_moe_gemm_staged):
        f.restype = i32
    return L


def lib():
    """The loaded libdsa.so (raises if it is missing: there is no fallback)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
        _lib = _configure(ctypes.CDLL(LIB_PATH))
    return _lib


def debug_lib():
    """The loaded libdsa_debug.so (the DSA_DEBUG_BOUNDS build)."""
    global _debug_lib
    if _debug_lib is None:
        if not os.path.exists(DEBUG_LIB_PATH):
            raise RuntimeError(f"{DEBUG_LIB_PATH} is missing: build it with "
                               "__graft_entry__.build()")
        _debug_lib = _configure(ctypes.CDLL(DEBUG_LIB_PATH))
    return _debug_lib


class DsaError(RuntimeError):
    def __init__(self, code: int, call: str, library=None):
        msg = (library or lib()).dsa_status_string(code).decode()
        super().__init__(f"{call}: {STATUS.get(code, code)} ({msg})")
        self.code = code


def _check(code: int, call: str, library=None):
    if code != 0:
        raise DsaError(code, call, library)


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _nbytes(t) -> int:
    """Size in bytes of a workspace tensor of any dtype."""
    return t.numel() * t.element_size()


def _stream(stream=None):
    import torch

    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _need(t, dtype, name):
    import torch

    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


class Cache:
    """A block-paged cache in device memory (tensors are referenced, not copied).

    kv:          bf16 [num_blocks, block_size, d_qk] key rows (latent rows when v is None)
    k_idx:       bf16 [num_blocks, block_size, d_idx] indexer keys
    block_table: int32 [n_seq, max_blocks_per_seq]
    seq_lens:    int32 [n_seq]
    v:           bf16 [num_blocks, block_size, d_v] or None (V = kv[..., :d_v])
    """

    def __init__(self, kv, k_idx, block_table, seq_lens, v=None, d_v=None):
        import torch

        _need(kv, torch.bfloat16, "kv")
        _need(k_idx, torch.bfloat16, "k_idx")
        _need(block_table, torch.int32, "block_table")
        _need(seq_lens, torch.int32, "seq_lens")
        if v is not None:
            _need(v, torch.bfloat16, "v")
        nb, bs, d_qk = kv.shape
        if d_v is None:
            d_v = v.shape[-1] if v is not None else 512
        self.tensors = (kv, k_idx, block_table, seq_lens, v)
        self.c = PagedCache(kv.data_ptr(), d_qk, _ptr(v), v.shape[-1] if v is not None else 0,
                            k_idx.data_ptr(), k_idx.shape[-1], block_table.data_ptr(),
                            seq_lens.data_ptr(), block_table.shape[0], block_table.shape[1], nb,
                            bs, d_qk, d_v, k_idx.shape[-1])

    @property
    def n_seq(self):
        return self.c.n_seq


def index_score(cache: Cache, q_idx, w, phase: int, q_seq=None, q_pos=None,
                ld: Optional[int] = None, out=None, stream=None, library=None):
    """dsa_index_score: fp32 scores [n_q, ld].  q_seq / q_pos: int32 [n_q]
    device tensors (query i = position q_pos[i] of sequence q_seq[i]), or
    both None in DSA_DECODE (query i = last cached token of sequence i)."""
    import torch

    L = library or lib()
    _need(q_idx, torch.bfloat16, "q_idx")
    _need(w, torch.float32, "w")
    if q_seq is not None:
        _need(q_seq, torch.int32, "q_seq")
    if q_pos is not None:
        _need(q_pos, torch.int32, "q_pos")
    n_q, H_idx, _ = q_idx.shape
    if ld is None:
        ld = out.shape[1] if out is not None else None
    if out is None:
        out = torch.empty((n_q, ld), dtype=torch.float32, device=q_idx.device)
    _need(out, torch.float32, "scores")
    _check(L.dsa_index_score(ctypes.byref(cache.c), phase, q_idx.data_ptr(), w.data_ptr(),
                             _ptr(q_seq), _ptr(q_pos), n_q, H_idx, out.data_ptr(), out.shape[1],
                             None, 0, _stream(stream)), "dsa_index_score", L)
    return out


def index_topk_workspace(n_q: int, ld: int, K: int, device="cuda"):
    import torch

    n = lib().dsa_index_topk_decode_ws(n_q, ld, K)
    return torch.empty(max(n, 1), dtype=torch.uint8, device=device)


def index_topk_decode(cache: Cache, q_idx, w, K: int, scores, idx, workspace, q_seq=None,
                      q_pos=None, flags: int = 0, stream=None, library=None):
    """dsa_index_topk_decode: scores [n_q, ld] and kept positions [n_q, K] in
    one call (index kernel with group maxima, then one Top-K kernel)."""
    import torch

    L = library or lib()
    _need(q_idx, torch.bfloat16, "q_idx")
    _need(w, torch.float32, "w")
    _need(scores, torch.float32, "scores")
    _need(idx, torch.int32, "idx")
    n_q, H_idx, _ = q_idx.shape
    _check(L.dsa_index_topk_decode(ctypes.byref(cache.c), q_idx.data_ptr(), w.data_ptr(),
                                   _ptr(q_seq), _ptr(q_pos), n_q, H_idx, K, scores.data_ptr(),
                                   scores.shape[1], idx.data_ptr(), flags, workspace.data_ptr(),
                                   _nbytes(workspace), _stream(stream)), "dsa_index_topk_decode", L)
    return scores, idx


def index_topk_prefill_workspace(n_q: int, device="cuda"):
    import torch

    n = lib().dsa_index_topk_prefill_ws(n_q)
    return torch.empty(max(n, 1), dtype=torch.uint8, device=device)


def index_topk_prefill(cache: Cache, q_idx, w, q_seq, q_pos, K: int, idx=None, workspace=None,
                       stream=None, library=None):
    """dsa_index_topk_prefill: int32 kept positions [n_q, K] of prefill
    queries (position q_pos[i] of sequence q_seq[i]), no score matrix."""
    import torch

    L = library or lib()
    _need(q_idx, torch.bfloat16, "q_idx")
    _need(w, torch.float32, "w")
    _need(q_seq, torch.int32, "q_seq")
    _need(q_pos, torch.int32, "q_pos")
    n_q, H_idx, _ = q_idx.shape
    if idx is None:
        idx = torch.empty((n_q, K), dtype=torch.int32, device=q_idx.device)
    _need(idx, torch.int32, "idx")
    if workspace is None:
        workspace = index_topk_prefill_workspace(n_q, q_idx.device)
    _check(L.dsa_index_topk_prefill(ctypes.byref(cache.c), q_idx.data_ptr(), w.data_ptr(),
                                    q_seq.data_ptr(), q_pos.data_ptr(), n_q, H_idx, K,
                                    idx.data_ptr(), workspace.data_ptr(), _nbytes(workspace),
                                    _stream(stream)), "dsa_index_topk_prefill", L)
    return idx


def check_device_errors(stream=None, library=None) -> int:
    """dsa_check_device_errors: the status (DSA_OK, DSA_ERR_BOUNDS, or
    DSA_ERR_UNSUPPORTED in a release build)."""
    L = library or lib()
    return L.dsa_check_device_errors(_stream(stream))


def topk_workspace(n_q: int, ld: int, K: int, device="cuda"):
    import torch

    n = lib().dsa_topk_workspace_size(n_q, ld, K)
    return torch.empty(max(n, 1), dtype=torch.uint8, device=device)


def topk(scores, K: int, n_valid=None, causal_base: int = 0, out=None, workspace=None,
         stream=None, library=None):
    """dsa_topk: int32 [n_q, K] ascending kept positions, -1 padded."""
    import torch

    L = library or lib()
    _need(scores, torch.float32, "scores")
    n_q, ld = scores.shape
    if n_valid is not None:
        _need(n_valid, torch.int32, "n_valid")
    if out is None:
        out = torch.empty((n_q, K), dtype=torch.int32, device=scores.device)
    _need(out, torch.int32, "idx")
    if workspace is None:
        workspace = topk_workspace(n_q, ld, K, scores.device)
    _check(L.dsa_topk(scores.data_ptr(), ld, n_q, K, _ptr(n_valid), causal_base,
                      out.data_ptr(), workspace.data_ptr(), _nbytes(workspace), _stream(stream)),
           "dsa_topk", L)
    return out


def decode_workspace(B: int, H: int, K: int, d_v: int, device="cuda"):
    import torch

    n = lib().dsa_sparse_attn_decode_workspace_size(B, H, K, d_v)
    return torch.empty(max(n, 1), dtype=torch.uint8, device=device)


def sparse_attn_decode(cache: Cache, q, idx, sm_scale: float, out=None, lse=None,
                       workspace=None, want_lse: bool = True, stream=None, library=None):
    """dsa_sparse_attn_decode: (bf16 out [B, H, d_v], fp32 lse [B, H])."""
    import torch

    L = library or lib()
    _need(q, torch.bfloat16, "q")
    _need(idx, torch.int32, "idx")
    B, H, _ = q.shape
    K = idx.shape[1]
    d_v = cache.c.d_v
    if out is None:
        out = torch.empty((B, H, d_v), dtype=torch.bfloat16, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((B, H), dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = decode_workspace(B, H, K, d_v, q.device)
    _check(L.dsa_sparse_attn_decode(ctypes.byref(cache.c), q.data_ptr(), idx.data_ptr(), B, H,
                                    K, float(sm_scale), out.data_ptr(), _ptr(lse),
                                    workspace.data_ptr(), _nbytes(workspace), _stream(stream)),
           "dsa_sparse_attn_decode", L)
    return out, lse


def sparse_attn_decode_static(cache: Cache, q, idx, sm_scale: float, out=None, lse=None,
                              want_lse: bool = True, stream=None, library=None):
    """dsa_sparse_attn_decode_static: as sparse_attn_decode, with the split
    partials in the library's static device array (no workspace)."""
    import torch

    L = library or lib()
    _need(q, torch.bfloat16, "q")
    _need(idx, torch.int32, "idx")
    B, H, _ = q.shape
    K = idx.shape[1]
    d_v = cache.c.d_v
    if out is None:
        out = torch.empty((B, H, d_v), dtype=torch.bfloat16, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((B, H), dtype=torch.float32, device=q.device)
    _check(L.dsa_sparse_attn_decode_static(ctypes.byref(cache.c), q.data_ptr(), idx.data_ptr(),
                                           B, H, K, float(sm_scale), out.data_ptr(), _ptr(lse),
                                           _stream(stream)), "dsa_sparse_attn_decode_static", L)
    return out, lse


def sparse_attn_prefill(cache: Cache, q, q_seq, q_pos, idx, sm_scale: float, out=None,
                        lse=None, want_lse: bool = True, stream=None, library=None):
    """dsa_sparse_attn_prefill: (bf16 out [T, H, d_v], fp32 lse [T, H]).
    q_seq, q_pos: int32 [T] device tensors (query t = position q_pos[t] of
    sequence q_seq[t])."""
    import torch

    L = library or lib()
    _need(q, torch.bfloat16, "q")
    _need(idx, torch.int32, "idx")
    _need(q_seq, torch.int32, "q_seq")
    _need(q_pos, torch.int32, "q_pos")
    T, H, _ = q.shape
    K = idx.shape[1]
    d_v = cache.c.d_v
    if out is None:
        out = torch.empty((T, H, d_v), dtype=torch.bfloat16, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((T, H), dtype=torch.float32, device=q.device)
    _check(L.dsa_sparse_attn_prefill(ctypes.byref(cache.c), q.data_ptr(), q_seq.data_ptr(),
                                     q_pos.data_ptr(), idx.data_ptr(), T, H, K, float(sm_scale),
                                     out.data_ptr(), _ptr(lse), _stream(stream)),
           "dsa_sparse_attn_prefill", L)
    return out, lse


def cache_write(cache: Cache, seq, pos, kv_new, k_idx_new, v_new=None, stream=None,
                library=None):
    """dsa_cache_write: store new tokens' rows into the paged pools in place.

    seq, pos: int32 [n]; kv_new: bf16 [n, d_qk]; k_idx_new: bf16 [n, d_idx];
    v_new: bf16 [n, d_v] exactly when the cache has a separate V pool."""
    import torch

    _need(seq, torch.int32, "seq")
    _need(pos, torch.int32, "pos")
    _need(kv_new, torch.bfloat16, "kv_new")
    _need(k_idx_new, torch.bfloat16, "k_idx_new")
    if v_new is not None:
        _need(v_new, torch.bfloat16, "v_new")
    n = seq.shape[0]
    L = library or lib()
    _check(L.dsa_cache_write(ctypes.byref(cache.c), seq.data_ptr(), pos.data_ptr(), n,
                             kv_new.data_ptr(), _ptr(v_new), k_idx_new.data_ptr(),
                             _stream(stream)), "dsa_cache_write", L)


class DecodeStep:
    """One decode step over a batch (index score -> Top-K -> sparse attention)
    with every buffer allocated once up front.  fused=True runs the index
    score and Top-K as one dsa_index_topk_decode call; fused=False as the two
    separate calls.  seed=True passes DSA_TOPK_SEED_PREVIOUS from the second
    call on (the previous step's per-row threshold as a hint)."""

    def __init__(self, cache: Cache, B: int, H: int, H_idx: int, K: int, ld: int, d_v: int,
                 device="cuda", fused: bool = True, seed: bool = False):
        import torch

        self.cache, self.K, self.fused, self.seed = cache, K, fused, seed
        ld = (ld + 63) // 64 * 64  # aligned score rows: 16-byte loads in Top-K
        self.scores = torch.empty((B, ld), dtype=torch.float32, device=device)
        self.idx = torch.empty((B, K), dtype=torch.int32, device=device)
        self.out = torch.empty((B, H, d_v), dtype=torch.bfloat16, device=device)
        self.lse = torch.empty((B, H), dtype=torch.float32, device=device)
        self.ws_topk = (index_topk_workspace(B, ld, K, device) if fused else
                        topk_workspace(B, ld, K, device))
        self.ws_attn = decode_workspace(B, H, K, d_v, device)
        self.calls = 0

    def select(self, q_idx, w, stream=None, library=None):
        """Index score and Top-K of the step (self.scores, self.idx)."""
        c = self.cache
        if self.fused:
            flags = DSA_TOPK_SEED_PREVIOUS if self.seed and self.calls > 0 else 0
            index_topk_decode(c, q_idx, w, self.K, self.scores, self.idx, self.ws_topk,
                              flags=flags, stream=stream, library=library)
        else:
            index_score(c, q_idx, w, DSA_DECODE, out=self.scores, stream=stream, library=library)
            topk(self.scores, self.K, n_valid=c.tensors[3], out=self.idx, workspace=self.ws_topk,
                 stream=stream, library=library)
        self.calls += 1

    def attend(self, q, sm_scale: float, stream=None, library=None):
        sparse_attn_decode(self.cache, q, self.idx, sm_scale, out=self.out, lse=self.lse,
                           workspace=self.ws_attn, stream=stream, library=library)

    def __call__(self, q, q_idx, w, sm_scale: float, stream=None, library=None):
        self.select(q_idx, w, stream=stream, library=library)
        self.attend(q, sm_scale, stream=stream, library=library)
        return self.out, self.lse


class PrefillStep:
    """Causal prefill of positions pos0 .. pos0+T-1 of sequence `seq` (or, with
    q_seq / q_pos given, of any queries: q_seq[t], q_pos[t]).  fused=True
    selects with dsa_index_topk_prefill (no score matrix)."""

    def __init__(self, cache: Cache, T: int, H: int, K: int, d_v: int, pos0: int = 0,
                 seq: int = 0, q_seq=None, q_pos=None, device="cuda", fused: bool = False):
        import torch

        self.cache, self.K, self.T, self.fused = cache, K, T, fused
        if q_pos is None:
            q_pos = torch.arange(pos0, pos0 + T, dtype=torch.int32, device=device)
            q_seq = torch.full((T,), seq, dtype=torch.int32, device=device)
        self.q_seq, self.q_pos = q_seq, q_pos
        self.n_valid = q_pos + 1  # candidates of each row: positions 0 .. q_pos
        ld = (int(q_pos.max().item()) + 1 + 63) // 64 * 64  # aligned score rows
        self.scores = torch.empty((T, ld), dtype=torch.float32, device=device)
        self.idx = torch.empty((T, K), dtype=torch.int32, device=device)
        self.out = torch.empty((T, H, d_v), dtype=torch.bfloat16, device=device)
        self.lse = torch.empty((T, H), dtype=torch.float32, device=device)
        self.ws_topk = topk_workspace(T, ld, K, device)
        self.ws_fused = index_topk_prefill_workspace(T, device) if fused else None

    def select(self, q_idx, w, stream=None, library=None):
        """Index score and Top-K of the chunk (self.idx; self.scores too
        unless fused)."""
        c = self.cache
        if self.fused:
            index_topk_prefill(c, q_idx, w, self.q_seq, self.q_pos, self.K, idx=self.idx,
                               workspace=self.ws_fused, stream=stream, library=library)
            return
        index_score(c, q_idx, w, DSA_PREFILL, q_seq=self.q_seq, q_pos=self.q_pos,
                    out=self.scores, stream=stream, library=library)
        topk(self.scores, self.K, n_valid=self.n_valid, out=self.idx, workspace=self.ws_topk,
             stream=stream, library=library)

    def __call__(self, q, q_idx, w, sm_scale: float, stream=None, library=None):
        c = self.cache
        self.select(q_idx, w, stream=stream, library=library)
        sparse_attn_prefill(c, q, self.q_seq, self.q_pos, self.idx, sm_scale, out=self.out,
                            lse=self.lse, stream=stream, library=library)
        return self.out, self.lse


class Experts:
    """One layer's MXFP4 expert weights in device memory (referenced, not
    copied): codes uint8 [num_experts, N, K/2] (element 2i in the low
    nibble), scales uint8 [num_experts, N, K/32] (E8M0), in row-major
    (DSA_MXFP4_ROW_MAJOR) or tiled (DSA_MXFP4_TILED) byte order."""

    def __init__(self, codes, scales, layout: int = DSA_MXFP4_ROW_MAJOR):
        import torch

        _need(codes, torch.uint8, "codes")
        _need(scales, torch.uint8, "scales")
        E, N, K2 = codes.shape
        if scales.shape != (E, N, 2 * K2 // 32):
            raise ValueError(f"scales must be [{E}, {N}, {2 * K2 // 32}], got {tuple(scales.shape)}")
        self.tensors = (codes, scales)
        self.w = Mxfp4Weights(codes.data_ptr(), scales.data_ptr(), E, N, 2 * K2, layout)

    @property
    def N(self):
        return self.w.N

    @property
    def K(self):
        return self.w.K

    def tiled(self, stream=None, library=None) -> "Experts":
        """dsa_mxfp4_pack: a tiled copy of row-major weights."""
        import torch

        L = library or lib()
        codes, scales = self.tensors
        c2, s2 = torch.empty_like(codes), torch.empty_like(scales)
        _check(L.dsa_mxfp4_pack(ctypes.byref(self.w), c2.data_ptr(), s2.data_ptr(),
                                _stream(stream)), "dsa_mxfp4_pack", L)
        return Experts(c2, s2, DSA_MXFP4_TILED)


def _routing(x, expert_ids, row_offsets):
    import torch

    _need(x, torch.uint8, "x")
    _need(row_offsets, torch.int32, "row_offsets")
    if expert_ids is not None:
        _need(expert_ids, torch.int32, "expert_ids")
    return row_offsets.shape[0] - 1, x.shape[0]


def moe_gemm_mxfp4(experts: Experts, x, expert_ids, row_offsets, max_rows: int, out=None,
                   stream=None, library=None):
    """dsa_moe_gemm_mxfp4: fp32 y [M, N] = x (E4M3 codes [M, K]) times the
    routed experts' weights, converted to E4M3 in registers."""
    import torch

    L = library or lib()
    n_act, M = _routing(x, expert_ids, row_offsets)
    if out is None:
        out = torch.empty((M, experts.N), dtype=torch.float32, device=x.device)
    _need(out, torch.float32, "y")
    _check(L.dsa_moe_gemm_mxfp4(ctypes.byref(experts.w), x.data_ptr(), expert_ids.data_ptr(),
                                row_offsets.data_ptr(), n_act, M, max_rows, out.data_ptr(),
                                _stream(stream)), "dsa_moe_gemm_mxfp4", L)
    return out


def mxfp4_to_fp8(experts: Experts, expert_ids, out=None, stream=None, library=None):
    """dsa_mxfp4_to_fp8: uint8 E4M3 codes [n_act, N, K] of the listed experts."""
    import torch

    L = library or lib()
    _need(expert_ids, torch.int32, "expert_ids")
    n_act = expert_ids.shape[0]
    if out is None:
        out = torch.empty((n_act, experts.N, experts.K), dtype=torch.uint8,
                          device=expert_ids.device)
    _need(out, torch.uint8, "w8")
    _check(L.dsa_mxfp4_to_fp8(ctypes.byref(experts.w), expert_ids.data_ptr(), n_act,
                              out.data_ptr(), _stream(stream)), "dsa_mxfp4_to_fp8", L)
    return out


def moe_gemm_fp8(w8, x, row_offsets, max_rows: int, out=None, stream=None, library=None):
    """dsa_moe_gemm_fp8: fp32 y [M, N] from converted weights w8 [n_act, N, K]."""
    import torch

    L = library or lib()
    _need(w8, torch.uint8, "w8")
    n_act, M = _routing(x, None, row_offsets)
    _, N, K = w8.shape
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=x.device)
    _need(out, torch.float32, "y")
    _check(L.dsa_moe_gemm_fp8(w8.data_ptr(), N, K, x.data_ptr(), row_offsets.data_ptr(), n_act,
                              M, max_rows, out.data_ptr(), _stream(stream)), "dsa_moe_gemm_fp8", L)
    return out


_hip = None


def _hip_runtime():
    global _hip
    if _hip is None:
        _hip = ctypes.CDLL("libamdhip64.so")
        _hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        _hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
    return _hip


class MoeStaged:
    """The staged expert pipeline's state that every layer shares: one FP8
    workspace of two halves (chunk_experts experts each), a second stream
    for the conversions and the five events that order them against the
    products and the halves' reuse (dsa_moe_gemm_staged).  Call it once per
    layer, in layer order."""

    def __init__(self, N: int, K: int, chunk_experts: int, device="cuda"):
        import torch

        n = lib().dsa_moe_staged_ws(N, K, chunk_experts)
        self.workspace = torch.empty(n, dtype=torch.uint8, device=device)
        self.conv_stream = torch.cuda.Stream(device=device)
        H = _hip_runtime()
        self._events = (ctypes.c_void_p * 5)()
        for i in range(5):
            ev = ctypes.c_void_p()
            if H.hipEventCreateWithFlags(ctypes.byref(ev), 2) != 0:  # hipEventDisableTiming
                raise RuntimeError("hipEventCreateWithFlags failed")
            self._events[i] = ev.value

    def __call__(self, experts: Experts, x, expert_ids, row_offsets, max_rows: int, out=None,
                 stream=None, library=None):
        import torch

        L = library or lib()
        n_act, M = _routing(x, expert_ids, row_offsets)
        if out is None:
            out = torch.empty((M, experts.N), dtype=torch.float32, device=x.device)
        _need(out, torch.float32, "y")
        _check(L.dsa_moe_gemm_staged(ctypes.byref(experts.w), x.data_ptr(), expert_ids.data_ptr(),
                                     row_offsets.data_ptr(), n_act, M, max_rows, out.data_ptr(),
                                     self.workspace.data_ptr(), _nbytes(self.workspace),
                                     _stream(stream), ctypes.c_void_p(self.conv_stream.cuda_stream),
                                     self._events), "dsa_moe_gemm_staged", L)
        return out

    def __del__(self):
        try:
            import torch

            torch.cuda.synchronize()
            H = _hip_runtime()
            for ev in self._events:
                if ev:
                    H.hipEventDestroy(ctypes.c_void_p(ev))
        except Exception:
            pass
