"""Benchmark of the DSA hot path on one MI355X.

A step is one pass of the whole path over one batch: index score -> Top-K ->
sparse attention (decode: split-K + merge).  The headline workload is the
ragged long-context decode (64 sequences, lengths uniform on [4096, 131072],
block size 64, 128 query heads on a 576-wide latent KV row, indexer 64 x 128,
Top-K 2048); tokens/s counts one new token per sequence per step.  The other
two full-size decode batches (32 x 32768 and 8 x 1048576) and the 8192-token
causal prefill are measured in the same run and reported as sub-objects.

Timing: inputs are seeded synthetic data generated directly in HBM before
timing.  Before every timed step a 512 MiB scratch buffer is written and
another one read (outside the timed events), so no step finds the previous
step's data in the caches, nor dirty lines of the flush to write back.
Each step is bracketed by HIP events on the stream the kernels run on; the
reported step time is the median over the timed steps.  A second pass of the
same number of steps puts events between the calls for the per-call
breakdown (the dominant kernel's time for the roofline comes from it).  The
achievable HBM read bandwidth is measured by a streaming-read probe kernel
and reported beside the 8 TB/s datasheet figure.

Prints one JSON line (see --help for the options).

Helper modes for the roofline's "traffic" figure (rocprofv3 counters):
  bench.py --calibrate-copy     a plain 1 GiB device copy (counter calibration)
  bench.py --write-traffic KERNEL WORKLOAD F W CF CW
                                fold rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE
                                CSVs of the step (F, W) and of the copy (CF, CW)
                                into profiles/traffic_KERNEL.json
"""
import argparse
import ctypes
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0           # MI355X HBM3E, GB/s (datasheet)
MFMA_BF16_PEAK_TF = 2500.0      # MI355X dense bf16 MFMA, TFLOP/s (datasheet)
# 256 CUs x 4 SIMDs x 1024 bf16 flop/clk x 2.4 GHz: the clock-derived dense
# peak, slightly above the datasheet's rounded figure; prefill utilisation is
# reported against it (the more conservative of the two)
MFMA_BF16_CLOCK_PEAK_TF = 2516.6
FLUSH_BYTES = 512 << 20         # scratch written before every timed step
PROBE_BYTES = 2 << 30           # streaming-read probe buffer
CSRC = os.path.join(ROOT, "sparse_attention_long_dsa_amd", "csrc")
# kernel -> the sources its counter figures were taken on
KERNEL_SOURCES = {
    "index_score_decode": ["index_score.hip", "common.h"],
    "topk_fused": ["topk.hip", "common.h"],
    "sparse_attn_latent": ["sparse_attn_latent.hip", "attn_common.h", "common.h"],
    "latent_combine": ["sparse_attn_latent.hip", "attn_common.h", "common.h"],
    "topk": ["topk.hip", "common.h"],
    "moe_decode": ["moe.hip", "common.h"],
    "moe_prefill": ["moe.hip", "common.h"],
}
# the kernel-name fragment of each key in a counter CSV (default: the key)
KERNEL_NAME_PART = {"moe_decode": "moe_gemm_kernel<2, 1, 2, true, true>",
                    "moe_prefill": "moe_gemm_big_kernel"}


def traffic_file(kernel):
    return os.path.join(ROOT, "profiles", f"traffic_{kernel}.json")


def decode_bytes(wl):
    """Algorithmic bytes of one decode step and of its index-score launch."""
    L = wl.seq_lens
    B, K = wl.n_q, wl.topk
    kidx = sum(L) * wl.d_idx * 2
    kept = sum(min(K, x) for x in L)
    gather = kept * wl.d_qk * 2 + (kept * wl.d_v * 2 if wl.separate_v else 0)
    q = B * wl.H * wl.d_qk * 2
    qidx = B * wl.H_idx * wl.d_idx * 2 + B * wl.H_idx * 4
    bt = sum((x + wl.block_size - 1) // wl.block_size for x in L) * 4
    idx = 2 * B * K * 4
    out = B * wl.H * wl.d_v * 2 + B * wl.H * 4
    step = kidx + gather + q + qidx + bt + idx + out
    index_launch = kidx + qidx + bt
    return step, index_launch


def attn_bytes(wl):
    """Algorithmic bytes of the decode attention: kept rows, q, the index
    array, block-table entries of the kept rows, the output."""
    L = wl.seq_lens
    B, K = wl.n_q, wl.topk
    kept = sum(min(K, x) for x in L)
    return (kept * wl.d_qk * 2 + B * wl.H * wl.d_qk * 2 + B * K * 4 + kept * 4
            + B * wl.H * wl.d_v * 2 + B * wl.H * 4)


def prefill_flops(wl):
    T, K = wl.seq_lens[0], wl.topk
    pairs = T * (T + 1) // 2
    kept = sum(min(K, t + 1) for t in range(T))
    return 2 * wl.d_idx * wl.H_idx * pairs, 2 * wl.H * (wl.d_qk + wl.d_v) * kept


def sha(paths):
    h = hashlib.sha256()
    for p in paths:
        h.update(open(p, "rb").read())
    return h.hexdigest()


def traffic_for(kernel, workload):
    """HBM bytes per launch of `kernel` from the committed counter summary,
    or None when missing, taken on another workload or on different sources."""
    f = traffic_file(kernel)
    if not os.path.exists(f):
        return None
    t = json.load(open(f))
    srcs = [os.path.join(CSRC, s) for s in KERNEL_SOURCES[kernel]]
    if t.get("source_sha256") != sha(srcs) or t.get("workload") != workload:
        return None
    return t.get("bytes_per_launch")


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def probe_lib():
    import sparse_attention_long_dsa_amd as dsa

    if not os.path.exists(dsa.PROBE_LIB):
        raise RuntimeError(f"{dsa.PROBE_LIB} is missing: build it with __graft_entry__.build()")
    L = ctypes.CDLL(dsa.PROBE_LIB)
    L.hbm_read_probe.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int,
                                 ctypes.c_int, ctypes.c_void_p]
    L.hbm_read_probe.restype = ctypes.c_int
    return L


class Timer:
    """Event-timed steps with a cache flush before each step.

    The flush writes a 512 MiB scratch buffer (evicting L2 and the 256 MB
    last-level cache) and then reads another 512 MiB buffer, so that the
    written lines are written back before the step starts rather than
    inside it; the step then finds only clean, unrelated lines cached.
    `calls` is the list of the step's calls (each a no-argument function
    that launches on the current stream).  Pass A brackets each whole step
    with one event pair; pass B records an event between consecutive calls
    for the breakdown."""

    def __init__(self):
        import torch

        self.torch = torch
        self.stream = torch.cuda.current_stream()
        self.flush_buf = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device="cuda")
        self.read_buf = torch.zeros(FLUSH_BYTES, dtype=torch.uint8, device="cuda")
        self.sink = torch.empty(4096 * 256, dtype=torch.int32, device="cuda")
        self.probe = probe_lib()
        self.n_flush = 0

    def flush(self):
        self.n_flush += 1
        self.flush_buf.fill_(self.n_flush & 0xFF)
        rc = self.probe.hbm_read_probe(self.read_buf.data_ptr(), FLUSH_BYTES,
                                       self.sink.data_ptr(), 4096, 0,
                                       ctypes.c_void_p(self.stream.cuda_stream))
        if rc != 0:
            raise RuntimeError(f"hbm_read_probe failed ({rc})")

    def run(self, calls, steps, warmup, breakdown=None):
        """Pass A times `calls` as whole steps; pass B times each call of
        `breakdown` (default: `calls`) on its own within a step."""
        torch = self.torch
        for _ in range(warmup):
            for c in calls:
                c()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(steps)]
        t0 = time.perf_counter()
        for i in range(steps):
            self.flush()
            ev[i][0].record(self.stream)
            for c in calls:
                c()
            ev[i][1].record(self.stream)
        torch.cuda.synchronize()
        wall_ms = (time.perf_counter() - t0) * 1e3 / steps
        step_ms = [a.elapsed_time(b) for a, b in ev]
        # pass B: per-call breakdown
        parts = breakdown or calls
        evb = [[torch.cuda.Event(enable_timing=True) for _ in range(len(parts) + 1)]
               for _ in range(steps)]
        for i in range(steps):
            self.flush()
            evb[i][0].record(self.stream)
            for j, c in enumerate(parts):
                c()
                evb[i][j + 1].record(self.stream)
        torch.cuda.synchronize()
        per_call = [statistics.median(e[j].elapsed_time(e[j + 1]) for e in evb)
                    for j in range(len(parts))]
        return {"median_ms": statistics.median(step_ms), "min_ms": min(step_ms),
                "max_ms": max(step_ms), "wall_ms_incl_flush": wall_ms, "per_call_ms": per_call}


def bench_decode(n, timer, steps, warmup, log):
    import torch

    import dsa_synth
    import sparse_attention_long_dsa_amd as dsa

    wl = dsa_synth.workload(n)
    t0 = time.time()
    dc = dsa_synth.device_case(wl, poison=False)
    log(f"generated {wl.name} (B={wl.n_q}, sum(L)={sum(wl.seq_lens)}) in HBM in "
        f"{time.time() - t0:.1f}s")
    cache = dsa.Cache(dc.kv, dc.k_idx, dc.block_table, dc.seq_lens, v=dc.v, d_v=wl.d_v)
    st = dsa.DecodeStep(cache, wl.n_q, wl.H, wl.H_idx, wl.topk, max(wl.seq_lens), wl.d_v)

    def stage(flags):
        return lambda: dsa.index_topk_decode(cache, dc.q_idx, dc.w, wl.topk, st.scores, st.idx,
                                             st.ws_topk, flags=flags)

    attend = lambda: st.attend(dc.q, wl.sm_scale)  # noqa: E731
    # the step: the fused index score + Top-K call, then the attention call;
    # breakdown: the fused call's two launches timed apart (same arguments)
    r = timer.run([stage(0), attend], steps, warmup,
                  breakdown=[stage(dsa.DSA_INDEX_TOPK_SCORE_ONLY),
                             stage(dsa.DSA_INDEX_TOPK_SELECT_ONLY), attend])
    step_bytes, index_bytes = decode_bytes(wl)
    ms = r["median_ms"]
    idx_ms, topk_ms, attn_ms = r["per_call_ms"]
    res = {
        "workload": wl.name, "batch": wl.n_q, "sum_ctx": sum(wl.seq_lens),
        "max_ctx": max(wl.seq_lens), "tokens_per_s": round(wl.n_q / (ms * 1e-3), 1),
        "ms_per_step": round(ms, 4), "ms_min": round(r["min_ms"], 4),
        "ms_max": round(r["max_ms"], 4), "wall_ms_per_step_incl_flush": round(r["wall_ms_incl_flush"], 4),
        "index_ms": round(idx_ms, 4), "topk_ms": round(topk_ms, 4), "attn_ms": round(attn_ms, 4),
        "algorithmic_bytes": step_bytes, "index_algorithmic_bytes": index_bytes,
        "hbm_gbs_step": round(step_bytes / (ms * 1e-3) / 1e9, 1),
        "hbm_frac_step": round(step_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "index_gbs": round(index_bytes / (idx_ms * 1e-3) / 1e9, 1),
        "attn_gbs": round(attn_bytes(wl) / (attn_ms * 1e-3) / 1e9, 1),
    }
    del dc, cache, st
    torch.cuda.empty_cache()
    return res, wl


def bench_prefill(timer, reps, warmup, log):
    import torch

    import dsa_synth
    import sparse_attention_long_dsa_amd as dsa

    wl = dsa_synth.workload(3)
    dc = dsa_synth.device_case(wl, poison=False)
    cache = dsa.Cache(dc.kv, dc.k_idx, dc.block_table, dc.seq_lens, v=dc.v, d_v=wl.d_v)
    T = wl.seq_lens[0]
    st = dsa.PrefillStep(cache, T, wl.H, wl.topk, wl.d_v)
    calls = [lambda: dsa.index_score(cache, dc.q_idx, dc.w, dsa.DSA_PREFILL, q_seq=st.q_seq,
                                     q_pos=st.q_pos, out=st.scores),
             lambda: dsa.topk(st.scores, wl.topk, n_valid=st.n_valid, out=st.idx,
                              workspace=st.ws_topk),
             lambda: dsa.sparse_attn_prefill(cache, dc.q, st.q_seq, st.q_pos, st.idx,
                                             wl.sm_scale, out=st.out, lse=st.lse)]
    r = timer.run(calls, reps, warmup)
    # the same step with the fused selection (index score + Top-K, no score matrix)
    stf = dsa.PrefillStep(cache, T, wl.H, wl.topk, wl.d_v, fused=True)
    rf = timer.run([lambda: stf.select(dc.q_idx, dc.w),
                    lambda: dsa.sparse_attn_prefill(cache, dc.q, stf.q_seq, stf.q_pos, stf.idx,
                                                    wl.sm_scale, out=stf.out, lse=stf.lse)],
                   reps, warmup)
    torch.cuda.synchronize()
    same = bool(torch.equal(stf.idx, st.idx))
    fi, fa = prefill_flops(wl)
    ms, msf = r["median_ms"], rf["median_ms"]
    parts, pf = r["per_call_ms"], rf["per_call_ms"]
    peak = MFMA_BF16_CLOCK_PEAK_TF
    res = {
        "workload": wl.name, "tokens_per_s": round(T / (msf * 1e-3), 1),
        "ms_per_step": round(msf, 4), "reps": reps, "ms_min": round(rf["min_ms"], 4),
        "select_ms": round(pf[0], 4), "attn_ms": round(pf[1], 4),
        "select_equal_to_separate": same,
        "flops": fi + fa, "mfma_peak_tflops": peak,
        "mfma_util": round((fi + fa) / (msf * 1e-3) / 1e12 / peak, 4),
        "attn_mfma_util": round(fa / (pf[1] * 1e-3) / 1e12 / peak, 4),
        "select_index_mfma_util": round(fi / (pf[0] * 1e-3) / 1e12 / peak, 4),
        "separate": {"ms_per_step": round(ms, 4), "ms_min": round(r["min_ms"], 4),
                     "index_ms": round(parts[0], 4), "topk_ms": round(parts[1], 4),
                     "attn_ms": round(parts[2], 4),
                     "index_mfma_util": round(fi / (parts[0] * 1e-3) / 1e12 / peak, 4),
                     "score_matrix_bytes": int(st.scores.numel()) * 4}}
    del stf
    # the cache write of the whole sequence: its own rows written back from a
    # contiguous copy (gathered untimed), so the pools end up unchanged
    stream = torch.cuda.current_stream()
    pos = torch.arange(T, dtype=torch.int32, device=dc.kv.device)
    seq = torch.zeros_like(pos)
    bt = dc.block_table[0].long()
    rows = bt[pos.long() // wl.block_size] * wl.block_size + pos.long() % wl.block_size
    kv_rows = dc.kv.reshape(-1, wl.d_qk)[rows].contiguous()
    kidx_rows = dc.k_idx.reshape(-1, wl.d_idx)[rows].contiguous()
    dsa.cache_write(cache, seq, pos, kv_rows, kidx_rows)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n_cw = 20
    a.record(stream)
    for _ in range(n_cw):
        dsa.cache_write(cache, seq, pos, kv_rows, kidx_rows)
    b.record(stream)
    torch.cuda.synchronize()
    cw_eager_ms = a.elapsed_time(b) / n_cw  # includes the Python launch of each call
    g = torch.cuda.CUDAGraph()  # the same launches replayed from a HIP graph: device time
    with torch.cuda.graph(g):
        for _ in range(n_cw):
            dsa.cache_write(cache, seq, pos, kv_rows, kidx_rows)
    g.replay()
    torch.cuda.synchronize()
    a.record(stream)
    g.replay()
    b.record(stream)
    torch.cuda.synchronize()
    cw_ms = a.elapsed_time(b) / n_cw
    del g
    cw_bytes = 2 * T * 2 * (wl.d_qk + wl.d_idx) + 2 * T * 4 + T * 4
    cw = {"workload": f"{wl.name}: {T} tokens' latent and indexer rows",
          "ms": round(cw_ms, 4), "ms_eager": round(cw_eager_ms, 4), "bytes": cw_bytes,
          "gbs": round(cw_bytes / (cw_ms * 1e-3) / 1e9, 1),
          "frac": round(cw_bytes / (cw_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    del dc, cache, st, kv_rows, kidx_rows, calls
    torch.cuda.empty_cache()
    return res, cw


FP8_MFMA_PEAK_TF = 5000.0  # MI355X dense FP8 matrix peak (TFLOP/s)


def moe_layer_bytes(wl, n_act, M):
    """Algorithmic HBM bytes of one expert-layer product: the listed
    experts' MXFP4 weights once (codes + scales, 17/32 byte an element), the
    token rows once (E4M3) and the fp32 result once."""
    return n_act * wl.N * wl.K * 17 // 32 + M * wl.K + M * wl.N * 4


def bench_moe(timer, steps, warmup, log):
    """The MoE expert product of one layer (MXFP4 weights converted to FP8
    just before use) at the decode and prefill batch sizes: the fused call on
    tiled weights (the headline of each), and beside it the fused call on
    row-major weights, the conversion alone and the staged two-stream
    pipeline."""
    import torch

    import sparse_attention_long_dsa_amd as dsa
    from dsa_synth import moe as synth

    out = {}
    for make in (synth.decode_layer, synth.prefill_layer):
        wl = make()
        ids, offs, max_rows = synth.routing(wl)
        n_act, M = len(ids), int(offs[-1])
        codes, scales = synth.device_weights(wl)
        x = synth.device_tokens(wl)
        d_ids = torch.from_numpy(ids).cuda()
        d_offs = torch.from_numpy(offs).cuda()
        rowmajor = dsa.Experts(codes, scales)
        tiled = rowmajor.tiled()
        y = torch.empty((M, wl.N), dtype=torch.float32, device="cuda")
        staged = dsa.MoeStaged(wl.N, wl.K, 16)
        w8 = torch.empty((16, wl.N, wl.K), dtype=torch.uint8, device="cuda")
        torch.cuda.synchronize()
        calls = [lambda: dsa.moe_gemm_mxfp4(tiled, x, d_ids, d_offs, max_rows, out=y)]
        parts = [calls[0],
                 lambda: dsa.moe_gemm_mxfp4(rowmajor, x, d_ids, d_offs, max_rows, out=y),
                 lambda: dsa.mxfp4_to_fp8(tiled, d_ids[:16], out=w8),
                 lambda: staged(tiled, x, d_ids, d_offs, max_rows, out=y)]
        r = timer.run(calls, steps, warmup, breakdown=parts)
        ms = r["median_ms"]
        nbytes = moe_layer_bytes(wl, n_act, M)
        flops = 2 * M * wl.N * wl.K
        conv_bytes = 16 * wl.N * wl.K * (17 / 32 + 1)
        e = {"workload": wl.name, "experts_listed": n_act, "rows": M, "max_rows": max_rows,
             "N": wl.N, "K": wl.K, "scale_codes": [wl.scale_lo, wl.scale_hi],
             "ms": round(ms, 4), "ms_min": round(r["min_ms"], 4),
             "ms_rowmajor_weights": round(r["per_call_ms"][1], 4),
             "ms_convert_16_experts": round(r["per_call_ms"][2], 4),
             "convert_gbs": round(conv_bytes / (r["per_call_ms"][2] * 1e-3) / 1e9, 1),
             "ms_staged_pipeline": round(r["per_call_ms"][3], 4),
             "algorithmic_bytes": nbytes, "flops": flops,
             "gbs": round(nbytes / (ms * 1e-3) / 1e9, 1),
             "hbm_frac": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
             "tflops": round(flops / (ms * 1e-3) / 1e12, 1),
             "fp8_mfma_frac": round(flops / (ms * 1e-3) / 1e12 / FP8_MFMA_PEAK_TF, 4),
             "traffic": traffic_for("moe_decode" if make is synth.decode_layer
                                    else "moe_prefill", wl.name)}
        log(f"{wl.name}: {ms:.3f} ms, {e['gbs']} GB/s, {e['tflops']} TFLOP/s")
        out[make.__name__] = e
        del codes, scales, x, rowmajor, tiled, y, staged, w8, calls, parts
        torch.cuda.empty_cache()
    return out


def hbm_probe(log):
    """Achievable HBM read bandwidth: the streaming-read probe over a 2 GiB
    buffer, a few grid sizes, the best median of 5 reads each."""
    import torch

    L = probe_lib()
    buf = torch.ones(PROBE_BYTES // 4, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    best = None
    modes = {0: "ordinary loads", 1: "non-temporal loads", 2: "per-workgroup regions"}
    for grid, nt in ((1024, 1), (2048, 1), (4096, 1), (8192, 1), (4096, 0), (4096, 2),
                     (8192, 2), (16384, 2)):
        sink = torch.empty(grid * 256, dtype=torch.int32, device="cuda")
        times = []
        for rep in range(6):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            rc = L.hbm_read_probe(buf.data_ptr(), PROBE_BYTES, sink.data_ptr(), grid, nt,
                                  ctypes.c_void_p(stream.cuda_stream))
            b.record(stream)
            if rc != 0:
                raise RuntimeError(f"hbm_read_probe failed ({rc})")
            torch.cuda.synchronize()
            if rep > 0:
                times.append(a.elapsed_time(b))
        gbs = PROBE_BYTES / (statistics.median(times) * 1e-3) / 1e9
        log(f"hbm probe: grid {grid} x 256, {modes[nt]}: {gbs:.0f} GB/s")
        if best is None or gbs > best[0]:
            best = (gbs, grid, nt)
    del buf
    torch.cuda.empty_cache()
    return {"kernel": "hbm_read_kernel / hbm_read_chunk_kernel (streaming read, 16 B a lane, "
                      "8 loads in flight; best of grid sizes and patterns)",
            "bytes": PROBE_BYTES, "gbs": round(best[0], 1), "grid_blocks": best[1],
            "pattern": modes[best[2]], "frac_of_peak": round(best[0] / HBM_PEAK_GBS, 4)}


def cpu_baseline(wl, budget_s, log):
    """The oracle, as it stands, on a bounded sample of the decode batch:
    whole sequences (scores over all positions, Top-K, attention) until the
    time budget is used.  Reported in the same unit (tokens/s)."""
    import dsa_synth
    import oracle

    done, spent = 0, 0.0
    for b in range(wl.n_q):
        L = wl.seq_lens[b]
        lbt, k_idx, _, _ = dsa_synth.host_sequence_pools(wl, b)
        q, q_idx, w = dsa_synth.host_query_rows(wl, b, 1)
        t0 = time.perf_counter()
        sc = oracle.index_score(k_idx, lbt, wl.block_size, q_idx, w, [0], [L - 1], ld=L)
        idx = oracle.topk(sc, [L], wl.topk)
        t1 = time.perf_counter()
        table, kv, v = dsa_synth.host_kept_pool(wl, b, idx[0])
        t2 = time.perf_counter()
        oracle.sparse_attn(kv, v, table, 1, q, [0], idx, wl.sm_scale, d_v=wl.d_v)
        spent += (t1 - t0) + (time.perf_counter() - t2)
        done += 1
        if spent >= budget_s:
            break
    cores = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    log(f"cpu oracle: {done} sequences in {spent:.1f}s on {cores} threads")
    return {"value": done / spent, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "cpu_model": cpu_model(), "nproc": os.cpu_count(),
            "sample": f"{done} of {wl.n_q} sequences of the same batch (first ones, "
                      f"{sum(wl.seq_lens[:done])} cached positions), one decode token each: "
                      f"index score over every position, Top-K, attention; input generation "
                      f"not timed"}


COPY_BYTES = 1 << 30  # plain-copy calibration size


def calibrate_copy():
    """A plain device-to-device copy of COPY_BYTES, three times: the counter
    reading of this kernel is the scale for FETCH_SIZE / WRITE_SIZE."""
    import torch

    torch.cuda.set_device(0)
    a = torch.ones(COPY_BYTES, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": COPY_BYTES}))


def _pmc_per_dispatch(csv_path, counter, name_part):
    """Mean per-dispatch value of `counter` for kernels whose name contains
    name_part, from a rocprofv3 --pmc counter_collection.csv."""
    import csv

    vals = {}
    for r in csv.DictReader(open(csv_path)):
        if name_part in r["Kernel_Name"] and r["Counter_Name"] == counter:
            vals.setdefault(r["Dispatch_Id"], 0.0)
            vals[r["Dispatch_Id"]] += float(r["Counter_Value"])
    if not vals:
        raise SystemExit(f"no {counter} rows for {name_part} in {csv_path}")
    return sum(vals.values()) / len(vals)


def write_traffic(kernel, workload, fetch_csv, write_csv, copy_fetch_csv, copy_write_csv,
                  cname="copyBuffer"):
    """Fold two counter runs of a kernel and two of the plain copy into
    profiles/traffic_KERNEL.json (HBM bytes per launch).  `cname` names the
    copy kernel (the runtime's device-to-device copy)."""
    part = KERNEL_NAME_PART.get(kernel, kernel)
    f = _pmc_per_dispatch(fetch_csv, "FETCH_SIZE", part)
    w = _pmc_per_dispatch(write_csv, "WRITE_SIZE", part)
    cf = _pmc_per_dispatch(copy_fetch_csv, "FETCH_SIZE", cname)
    cw = _pmc_per_dispatch(copy_write_csv, "WRITE_SIZE", cname)
    f_scale, w_scale = COPY_BYTES / cf, COPY_BYTES / cw  # bytes per counter unit
    srcs = [os.path.join(CSRC, s) for s in KERNEL_SOURCES[kernel]]
    out = {"kernel": kernel, "workload": workload,
           "fetch_raw": f, "write_raw": w, "copy_fetch_raw": cf, "copy_write_raw": cw,
           "fetch_bytes": f * f_scale, "write_bytes": w * w_scale,
           "bytes_per_launch": f * f_scale + w * w_scale, "source_sha256": sha(srcs)}
    with open(traffic_file(kernel), "w") as fh:
        json.dump(out, fh, indent=1)
    print(json.dumps(out))


def main():
    if len(sys.argv) > 1 and sys.argv[1] == "--calibrate-copy":
        return calibrate_copy()
    if len(sys.argv) > 1 and sys.argv[1] == "--write-traffic":
        return write_traffic(*sys.argv[2:])
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=4, help="headline decode workload: 1, 2, 4 or 5")
    ap.add_argument("--prefill-reps", type=int, default=10)
    ap.add_argument("--no-prefill", action="store_true", help="skip the 8192-token prefill")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the other full-size decode batches")
    ap.add_argument("--no-probe", action="store_true", help="skip the HBM read probe")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-moe", action="store_true",
                    help="skip the MoE expert layers (MXFP4 -> FP8 product)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    def log(*a):
        print(*a, file=sys.stderr, flush=True)

    import torch

    import sparse_attention_long_dsa_amd as dsa

    torch.cuda.set_device(0)
    dsa.lib()
    if args.config not in (1, 2, 4, 5):
        sys.exit("--config must name a decode workload (1, 2, 4 or 5)")
    timer = Timer()
    probe = None if args.no_probe else hbm_probe(log)
    d, wl = bench_decode(args.config, timer, args.steps, args.warmup, log)
    ms = d["ms_per_step"]
    step_bytes, index_bytes = d["algorithmic_bytes"], d["index_algorithmic_bytes"]
    achieved = index_bytes / (d["index_ms"] * 1e-3) / 1e9
    metric = ("decode tokens/s at 128K ctx (ragged 4K-128K, B=64, Top-K 2048)" if args.config == 4
              else f"decode tokens/s ({wl.name}, Top-K {wl.topk})")
    roof = {"kernel": "index_score_decode (the step's dominant kernel; whole step in "
                      "roofline_step)", "bound": "hbm",
            "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic_for("index_score_decode", wl.name),
            "launch_ms": d["index_ms"], "algorithmic_bytes": index_bytes}
    step_gbs = step_bytes / (ms * 1e-3) / 1e9
    roof_step = {"bound": "hbm", "achieved": round(step_gbs, 1), "peak": HBM_PEAK_GBS,
                 "unit": "GB/s", "frac": round(step_gbs / HBM_PEAK_GBS, 4),
                 "algorithmic_bytes": step_bytes, "ms": ms}
    if probe:
        roof["achievable"] = probe["gbs"]
        roof["frac_of_achievable"] = round(achieved / probe["gbs"], 4)
        roof_step["achievable"] = probe["gbs"]
        roof_step["frac_of_achievable"] = round(step_gbs / probe["gbs"], 4)
    res = {
        "metric": metric,
        "value": d["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "batch": wl.n_q, "sum_ctx": sum(wl.seq_lens),
                   "max_ctx": max(wl.seq_lens), "block_size": wl.block_size, "heads": wl.H,
                   "d_qk": wl.d_qk, "d_v": wl.d_v, "indexer": [wl.H_idx, wl.d_idx],
                   "topk": wl.topk, "seed": wl.seed},
        "timing": "median of event-timed steps; before each step 512 MiB written, then 512 MiB read (cache flush)",
        "hbm_gbs_step": d["hbm_gbs_step"],
        "hbm_frac_step": d["hbm_frac_step"],
        "roofline": roof,
        "roofline_step": roof_step,
        "decode": d,
    }
    if probe:
        res["hbm_probe"] = probe
    if not args.no_extra:
        res["decode_configs"] = {}
        for n in (2, 4, 5):
            if n == args.config:
                continue
            e, ewl = bench_decode(n, timer, args.steps, args.warmup, log)
            if probe:
                e["hbm_frac_of_achievable"] = round(e["hbm_gbs_step"] / probe["gbs"], 4)
            res["decode_configs"][ewl.name] = e
    if not args.no_prefill:
        p, cw = bench_prefill(timer, args.prefill_reps, 2, log)
        res["prefill"] = p
        res["cache_write"] = cw
    if not args.no_moe:
        moe = bench_moe(timer, args.steps, args.warmup, log)
        dec, pre = moe["decode_layer"], moe["prefill_layer"]
        res["moe"] = {
            "decode_layer": dict(dec, roofline={
                "bound": "hbm", "achieved": dec["gbs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": dec["hbm_frac"], "traffic": dec["traffic"],
                **({"achievable": probe["gbs"],
                    "frac_of_achievable": round(dec["gbs"] / probe["gbs"], 4)} if probe else {})}),
            "prefill_layer": dict(pre, roofline={
                "bound": "mfma", "achieved": pre["tflops"], "peak": FP8_MFMA_PEAK_TF,
                "unit": "TFLOP/s", "frac": pre["fp8_mfma_frac"], "traffic": pre["traffic"]})}
    if not args.no_cpu:
        res["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds, log)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
