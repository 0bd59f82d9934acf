"""Benchmark of the DSA hot path on one MI355X.

A step is one pass of the whole path over one batch: index score -> Top-K ->
sparse attention (decode: split-K + merge).  The default workload is the
ragged long-context decode (64 sequences, lengths uniform on [4096, 131072],
block size 64, 128 query heads on a 576-wide latent KV row, indexer 64 x 128,
Top-K 2048); tokens/s counts one new token per sequence per step.  The 8192
token causal prefill is measured too and reported in the "prefill" object.

Inputs are seeded synthetic data generated directly in HBM before timing.
Prints one JSON line (see --help for the options).

Two helper modes feed the roofline's "traffic" figure:
  bench.py --calibrate-copy     a plain 1 GiB device copy (counter calibration)
  bench.py --write-traffic F W CF CW
                                fold rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE
                                CSVs of the step (F, W) and of the copy (CF, CW)
                                into profiles/index_score_decode_traffic.json
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0      # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TF = 2500.0  # MI355X dense bf16 MFMA, TFLOP/s
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "index_score_decode_traffic.json")
# the decode index kernel's sources (its file and the shared device helpers)
INDEX_SRC = [os.path.join(ROOT, "sparse_attention_long_dsa_amd", "csrc", f)
             for f in ("index_score.hip", "common.h")]


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


def traffic_for(workload):
    """HBM bytes per index-score launch from the committed counter summary,
    or None when missing, taken on another workload or on a different kernel
    source."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    t = json.load(open(TRAFFIC_FILE))
    if t.get("source_sha256") != sha(INDEX_SRC) or t.get("workload") != workload:
        return None
    return t.get("bytes_per_launch")


def time_decode(wl, steps, warmup, log):
    import torch

    import dsa_synth
    import sparse_attention_long_dsa_amd as dsa

    t0 = time.time()
    dc = dsa_synth.device_case(wl, poison=False)
    log(f"generated {wl.name} in HBM in {time.time() - t0:.1f}s")
    cache = dsa.Cache(dc.kv, dc.k_idx, dc.block_table, dc.seq_lens, v=dc.v, d_v=wl.d_v)
    step = dsa.DecodeStep(cache, wl.n_q, wl.H, wl.H_idx, wl.topk, max(wl.seq_lens), wl.d_v)
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        step(dc.q, dc.q_idx, dc.w, wl.sm_scale)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        # the index-score kernel is launched on this stream; events bracket it
        ev[i][0].record(stream)
        dsa.index_score(cache, dc.q_idx, dc.w, dsa.DSA_DECODE, out=step.scores)
        ev[i][1].record(stream)
        dsa.topk(step.scores, wl.topk, n_valid=dc.seq_lens, out=step.idx,
                 workspace=step.ws_topk)
        dsa.sparse_attn_decode(cache, dc.q, step.idx, wl.sm_scale, out=step.out, lse=step.lse,
                               workspace=step.ws_attn)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    idx_ms = sum(a.elapsed_time(b) for a, b in ev) / steps
    return elapsed * 1e3 / steps, idx_ms


def time_prefill(wl, steps, warmup, log):
    import torch

    import dsa_synth
    import sparse_attention_long_dsa_amd as dsa

    dc = dsa_synth.device_case(wl, poison=False)
    cache = dsa.Cache(dc.kv, dc.k_idx, dc.block_table, dc.seq_lens, v=dc.v, d_v=wl.d_v)
    T = wl.seq_lens[0]
    step = dsa.PrefillStep(cache, T, wl.H, wl.topk, wl.d_v)
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        step(dc.q, dc.q_idx, dc.w, wl.sm_scale)
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        ev[i][0].record(stream)
        dsa.index_score(cache, dc.q_idx, dc.w, dsa.DSA_PREFILL, out=step.scores)
        ev[i][1].record(stream)
        dsa.topk(step.scores, wl.topk, causal_base=0, out=step.idx, workspace=step.ws_topk)
        ev[i][2].record(stream)
        dsa.sparse_attn_prefill(cache, dc.q, step.idx, 0, 0, wl.sm_scale, out=step.out,
                                lse=step.lse)
        ev[i][3].record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    parts = [sum(e[j].elapsed_time(e[j + 1]) for e in ev) / steps for j in range(3)]
    # the cache write of the whole sequence: its own rows written back from a
    # contiguous copy (gathered untimed), so the pools end up unchanged
    pos = torch.arange(T, dtype=torch.int32, device=dc.kv.device)
    seq = torch.zeros_like(pos)
    bt = dc.block_table[0].long()
    rows = bt[pos.long() // wl.block_size] * wl.block_size + pos.long() % wl.block_size
    kv_rows = dc.kv.reshape(-1, wl.d_qk)[rows].contiguous()
    kidx_rows = dc.k_idx.reshape(-1, wl.d_idx)[rows].contiguous()
    dsa.cache_write(cache, seq, pos, kv_rows, kidx_rows)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 20
    a.record(stream)
    for _ in range(reps):
        dsa.cache_write(cache, seq, pos, kv_rows, kidx_rows)
    b.record(stream)
    torch.cuda.synchronize()
    cw_eager_ms = a.elapsed_time(b) / reps  # includes the Python launch of each call
    # the same launches replayed from a captured HIP graph: device time only
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(reps):
            dsa.cache_write(cache, seq, pos, kv_rows, kidx_rows)
    g.replay()
    torch.cuda.synchronize()
    a.record(stream)
    g.replay()
    b.record(stream)
    torch.cuda.synchronize()
    cw_ms = a.elapsed_time(b) / reps
    del g
    cw_bytes = 2 * T * 2 * (wl.d_qk + wl.d_idx) + 2 * T * 4 + T * 4
    del dc, cache, step, kv_rows, kidx_rows
    torch.cuda.empty_cache()
    return elapsed * 1e3 / steps, parts, (cw_ms, cw_eager_ms, cw_bytes)


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
        _, _, kv, v = dsa_synth.host_sequence_pools(wl, b, kv_positions=idx[0])
        t2 = time.perf_counter()
        oracle.sparse_attn(kv, v, lbt, wl.block_size, q, [0], idx, wl.sm_scale, d_v=wl.d_v)
        spent += (t1 - t0) + (time.perf_counter() - t2)
        done += 1
        if spent >= budget_s:
            break
    cores = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    log(f"cpu oracle: {done} sequences in {spent:.1f}s on {cores} threads")
    return {"value": done / spent, "unit": "tokens/s", "cores": cores, "kind": "oracle",
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


def write_traffic(fetch_csv, write_csv, copy_fetch_csv, copy_write_csv, cname="copyBuffer"):
    """Fold two counter runs of the decode step and two of the plain copy into
    profiles/index_score_decode_traffic.json (HBM bytes per launch).  `cname`
    names the copy kernel (the runtime's device-to-device copy)."""
    kname = "index_score_decode"
    f = _pmc_per_dispatch(fetch_csv, "FETCH_SIZE", kname)
    w = _pmc_per_dispatch(write_csv, "WRITE_SIZE", kname)
    cf = _pmc_per_dispatch(copy_fetch_csv, "FETCH_SIZE", cname)
    cw = _pmc_per_dispatch(copy_write_csv, "WRITE_SIZE", cname)
    f_scale, w_scale = COPY_BYTES / cf, COPY_BYTES / cw  # bytes per counter unit
    out = {"kernel": "index_score_decode", "workload": "ragged_decode_B64_L4K-128K",
           "fetch_raw": f, "write_raw": w, "copy_fetch_raw": cf, "copy_write_raw": cw,
           "fetch_bytes": f * f_scale, "write_bytes": w * w_scale,
           "bytes_per_launch": f * f_scale + w * w_scale,
           "source_sha256": sha(INDEX_SRC)}
    with open(TRAFFIC_FILE, "w") as fh:
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
    ap.add_argument("--config", type=int, default=4, help="decode workload 1, 2, 4 or 5")
    ap.add_argument("--no-prefill", action="store_true", help="skip the 8192-token prefill")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    def log(*a):
        print(*a, file=sys.stderr, flush=True)

    import torch

    import dsa_synth
    import sparse_attention_long_dsa_amd as dsa

    torch.cuda.set_device(0)
    dsa.lib()
    wl = dsa_synth.workload(args.config)
    if wl.phase != "decode":
        sys.exit("--config must name a decode workload")
    log(f"decode workload {wl.name}: B={wl.n_q} sum(L)={sum(wl.seq_lens)}")
    ms, idx_ms = time_decode(wl, args.steps, args.warmup, log)
    step_bytes, index_bytes = decode_bytes(wl)
    tok_s = wl.n_q / (ms * 1e-3)
    achieved = index_bytes / (idx_ms * 1e-3) / 1e9
    traffic = traffic_for(wl.name)
    metric = ("decode tokens/s at 128K ctx (ragged 4K-128K, B=64, Top-K 2048)" if args.config == 4
              else f"decode tokens/s ({wl.name}, Top-K {wl.topk})")
    res = {
        "metric": metric,
        "value": round(tok_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "batch": wl.n_q, "sum_ctx": sum(wl.seq_lens),
                   "max_ctx": max(wl.seq_lens), "block_size": wl.block_size, "heads": wl.H,
                   "d_qk": wl.d_qk, "d_v": wl.d_v, "indexer": [wl.H_idx, wl.d_idx],
                   "topk": wl.topk, "seed": wl.seed},
        "hbm_gbs_step": round(step_bytes / (ms * 1e-3) / 1e9, 1),
        "hbm_frac_step": round(step_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "roofline": {"kernel": "index_score_decode", "bound": "hbm",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "launch_ms": round(idx_ms, 4),
                     "algorithmic_bytes": index_bytes},
    }
    if not args.no_prefill:
        pw = dsa_synth.workload(3)
        pms, parts, (cw_ms, cw_eager_ms, cw_bytes) = time_prefill(pw, max(2, args.steps // 4), 2, log)
        fi, fa = prefill_flops(pw)
        res["prefill"] = {
            "workload": pw.name, "tokens_per_s": round(pw.seq_lens[0] / (pms * 1e-3), 1),
            "ms_per_step": round(pms, 4), "index_ms": round(parts[0], 4),
            "topk_ms": round(parts[1], 4), "attn_ms": round(parts[2], 4),
            "mfma_util": round((fi + fa) / (pms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TF, 4),
            "attn_mfma_util": round(fa / (parts[2] * 1e-3) / 1e12 / MFMA_BF16_PEAK_TF, 4),
            "index_mfma_util": round(fi / (parts[0] * 1e-3) / 1e12 / MFMA_BF16_PEAK_TF, 4),
            "flops": fi + fa}
        res["cache_write"] = {
            "workload": f"{pw.name}: {pw.seq_lens[0]} tokens' latent and indexer rows",
            "ms": round(cw_ms, 4), "ms_eager": round(cw_eager_ms, 4), "bytes": cw_bytes,
            "gbs": round(cw_bytes / (cw_ms * 1e-3) / 1e9, 1),
            "frac": round(cw_bytes / (cw_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    if not args.no_cpu:
        res["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds, log)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
