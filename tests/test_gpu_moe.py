"""GPU parity of the MoE expert product (MXFP4 weights converted to FP8 just
before use) through the C ABI against the oracle: the conversion bit-exact
for every (scale, FP4 code) pair, the three ways of running the product
bit-exact on integer-valued inputs (where fp32 accumulation is exact) and
within the fp32 accumulation bound on real-valued ones, the staged
pipeline's workspace reuse over several layers and chunks, the debug
build's checks of routing data, and sampled rows of the full-size layers.
"""
import numpy as np
import pytest
import torch

import oracle
import sparse_attention_long_dsa_amd as dsa
from dsa_synth import moe as synth
from tests.helpers import say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)
    dsa.lib()


def small(name, E, N, K, pairs, lo, hi, x_kind, seed):
    return synth.MoeWorkload(name, E, N, K, pairs, lo, hi, x_kind, seed)


def to_dev(*arrays):
    return [torch.from_numpy(np.ascontiguousarray(a)).cuda() for a in arrays]


def fp8_values(codes):
    return torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn).double().numpy()


def accumulation_bound(x, w8_list, ids_rows, K):
    """|fp32 sum - exact| <= K 2^-24 sum_k |x_k w_k| + 2^-24 |y| per entry
    (recursive fp32 summation in any order, then the oracle's own rounding)."""
    bounds = []
    for xs, w8 in zip(ids_rows, w8_list):
        bounds.append(np.abs(fp8_values(x[xs])) @ np.abs(fp8_values(w8)).T)
    return [(K + 1) * 2.0 ** -24 * b for b in bounds]


def tiled_layout_host(codes, scales):
    """The tiled byte order as the header defines it, written out with numpy
    index arithmetic (test-side; no kernel code)."""
    E, N, K2 = codes.shape
    K = 2 * K2
    c = codes.reshape(E, N // 16, 16, K // 256, 4, 2, 16)      # e, t, r, u, g, h, bytes
    c = c.transpose(0, 1, 3, 5, 4, 2, 6)                       # e, t, u, h, g, r, bytes
    s_ = scales.reshape(E, N // 16, 16, K // 256, 4, 2)        # e, t, r, u, g, h
    s_ = s_.transpose(0, 1, 3, 4, 2, 5)                        # e, t, u, g, r, h
    return (np.ascontiguousarray(c).reshape(E, N, K2),
            np.ascontiguousarray(s_).reshape(E, N, K // 32))


def run_case(wl, paths=("fused", "tiled", "fp8", "staged"), exact=True, chunk=2):
    ids, offs, max_rows = synth.routing(wl)
    codes, scales = synth.host_weights(wl)
    x = synth.host_tokens(wl)
    say(f"[moe] {wl.name} E={wl.num_experts} N={wl.N} K={wl.K} rows={wl.pairs} "
        f"n_act={len(ids)} max_rows={max_rows} scales={wl.scale_lo}..{wl.scale_hi} {wl.x_kind}")
    ref = oracle.moe_gemm(x, offs, ids, codes, scales, wl.N, wl.K)
    d_codes, d_scales, d_x, d_ids, d_offs = to_dev(codes, scales, x, ids, offs)
    ex = dsa.Experts(d_codes, d_scales)
    outs = {}
    if "fused" in paths:
        outs["fused"] = dsa.moe_gemm_mxfp4(ex, d_x, d_ids, d_offs, max_rows)
    if "tiled" in paths and wl.K % 256 == 0:
        outs["tiled"] = dsa.moe_gemm_mxfp4(ex.tiled(), d_x, d_ids, d_offs, max_rows)
    if "fp8" in paths:
        w8 = dsa.mxfp4_to_fp8(ex, d_ids)
        outs["fp8"] = dsa.moe_gemm_fp8(w8, d_x, d_offs, max_rows)
    if "staged" in paths:
        st = dsa.MoeStaged(wl.N, wl.K, chunk)
        outs["staged"] = st(ex, d_x, d_ids, d_offs, max_rows)
    torch.cuda.synchronize()
    if not exact:
        w8_ref = oracle.mxfp4_to_fp8(codes, scales, ids, wl.N, wl.K)
        rows = [slice(offs[i], offs[i + 1]) for i in range(len(ids))]
        bnd = accumulation_bound(x, list(w8_ref), rows, wl.K)
    for name, y in outs.items():
        g = y.cpu().numpy()
        if exact:
            np.testing.assert_array_equal(g, ref, err_msg=f"{wl.name} {name}")
        else:
            worst = 0.0
            for i, r in enumerate(rows):
                err = np.abs(g[r].astype(np.float64) - ref[r])
                assert (err <= bnd[i] + 1e-30).all(), f"{wl.name} {name} expert {i}"
                worst = max(worst, float((err / (bnd[i] + 1e-30)).max(initial=0.0)))
            say(f"   {name}: worst error / bound {worst:.3f}")
    if len(outs) > 1:
        first = next(iter(outs.values()))
        for name, y in outs.items():
            assert torch.equal(y, first), f"{name} differs from the other paths"
    say("   ok")
    return outs


def test_conversion_every_scale_and_code():
    # one row per block position: block b of every row has scale code b, so
    # all 256 scale codes meet all 16 FP4 codes (both nibbles)
    N, K = 32, 256 * 32
    rng = np.random.default_rng(5)
    codes = rng.integers(0, 256, (3, N, K // 2), dtype=np.uint8)
    codes[:, 0, :] = np.tile(np.arange(256, dtype=np.uint8), K // 512)
    scales = np.tile(np.arange(256, dtype=np.uint8), (3, N, 1))
    ids = np.array([2, 0, 1, 2], np.int32)
    ref = oracle.mxfp4_to_fp8(codes, scales, ids, N, K)
    d_codes, d_scales, d_ids = to_dev(codes, scales, ids)
    got = dsa.mxfp4_to_fp8(dsa.Experts(d_codes, d_scales), d_ids).cpu().numpy()
    np.testing.assert_array_equal(got, ref)


def test_pack_is_the_documented_byte_order():
    rng = np.random.default_rng(6)
    codes = rng.integers(0, 256, (3, 48, 256), dtype=np.uint8)
    scales = rng.integers(0, 256, (3, 48, 16), dtype=np.uint8)
    d_codes, d_scales = to_dev(codes, scales)
    t = dsa.Experts(d_codes, d_scales).tiled()
    c2, s2 = tiled_layout_host(codes, scales)
    np.testing.assert_array_equal(t.tensors[0].cpu().numpy(), c2)
    np.testing.assert_array_equal(t.tensors[1].cpu().numpy(), s2)
    # the conversion reads either layout to the same row-major result
    ids = torch.tensor([2, 0], dtype=torch.int32, device="cuda")
    a = dsa.mxfp4_to_fp8(dsa.Experts(d_codes, d_scales), ids)
    b = dsa.mxfp4_to_fp8(t, ids)
    assert torch.equal(a, b)


@pytest.mark.parametrize("K", [512, 384, 2048])
def test_decode_sized_integer_exact(K):
    # a few rows an expert: one 16-row tile, K with (512) and without (384)
    # the 4-step super-step
    run_case(small(f"dec_k{K}", 24, 96, K, 40, 126, 128, "int", 21 + K))


def test_mid_and_large_row_counts_integer_exact():
    # 17..32 rows (two tiles) and > 32 rows (four tiles, several passes)
    run_case(small("mid", 3, 64, 512, 80, 126, 128, "int", 31))
    run_case(small("large", 2, 48, 1024, 300, 126, 128, "int", 32))


def test_real_valued_within_accumulation_bound():
    # full E8M0 range around the exact one: FP8 subnormals and saturation
    run_case(small("real", 16, 64, 1024, 60, 100, 140, "normal", 41), exact=False)
    run_case(small("real_large", 3, 32, 512, 150, 110, 135, "normal", 42), exact=False)


def test_nan_scale_propagates():
    wl = small("nan", 4, 16, 256, 8, 126, 128, "int", 51)
    ids, offs, max_rows = synth.routing(wl)
    codes, scales = synth.host_weights(wl)
    scales[ids[0], 3, 2] = 255
    x = synth.host_tokens(wl)
    ref = oracle.moe_gemm(x, offs, ids, codes, scales, wl.N, wl.K)
    d = to_dev(codes, scales, x, ids, offs)
    y = dsa.moe_gemm_mxfp4(dsa.Experts(d[0], d[1]), d[2], d[3], d[4], max_rows).cpu().numpy()
    r = slice(offs[0], offs[1])
    assert np.isnan(ref[r, 3]).all() and np.isnan(y[r, 3]).all()
    np.testing.assert_array_equal(np.isnan(y), np.isnan(ref))
    ok = ~np.isnan(ref)
    np.testing.assert_array_equal(y[ok], ref[ok])


def test_uncovered_rows_untouched_and_empty_experts():
    wl = small("gaps", 6, 32, 256, 20, 126, 128, "int", 61)
    codes, scales = synth.host_weights(wl)
    x = synth.host_tokens(wl, rows=24)
    ids = np.array([5, 1, 3], np.int32)
    offs = np.array([2, 2, 9, 20], np.int32)  # rows 0,1 and 20..23 belong to no expert; expert 5 empty
    ref = oracle.moe_gemm(x, offs, ids, codes, scales, wl.N, wl.K)
    d = to_dev(codes, scales, x, ids, offs)
    y = torch.full((24, wl.N), float("nan"), device="cuda")
    dsa.moe_gemm_mxfp4(dsa.Experts(d[0], d[1]), d[2], d[3], d[4], 11, out=y)
    g = y.cpu().numpy()
    assert np.isnan(g[:2]).all() and np.isnan(g[20:]).all()
    np.testing.assert_array_equal(g[2:20], ref[2:20])


def test_max_rows_below_actual_count_is_still_right():
    wl = small("hint", 3, 32, 256, 90, 126, 128, "int", 71)
    ids, offs, max_rows = synth.routing(wl)
    codes, scales = synth.host_weights(wl)
    x = synth.host_tokens(wl)
    ref = oracle.moe_gemm(x, offs, ids, codes, scales, wl.N, wl.K)
    d = to_dev(codes, scales, x, ids, offs)
    for hint in (1, 16, 40):
        y = dsa.moe_gemm_mxfp4(dsa.Experts(d[0], d[1]), d[2], d[3], d[4], hint)
        np.testing.assert_array_equal(y.cpu().numpy(), ref, err_msg=f"max_rows {hint}")


def test_staged_pipeline_reuses_one_workspace_across_layers():
    # three layers with different experts, routing and widths of work; the
    # workspace holds two chunks of 2 experts, so halves are reused within a
    # layer and across layers; the conversions run on a second stream
    st = dsa.MoeStaged(64, 512, 2)
    layers = []
    for layer in range(3):
        wl = small(f"layer{layer}", 12, 64, 512, 30 + 7 * layer, 126, 128, "int", 80 + layer)
        ids, offs, max_rows = synth.routing(wl)
        codes, scales = synth.host_weights(wl)
        x = synth.host_tokens(wl)
        ref = oracle.moe_gemm(x, offs, ids, codes, scales, wl.N, wl.K)
        d = to_dev(codes, scales, x, ids, offs)
        layers.append((wl, ref, d, max_rows))
    say(f"[moe staged] 3 layers, n_act {[len(l[2][3]) for l in layers]}")
    for rep in range(2):
        outs = [st(dsa.Experts(d[0], d[1]), d[2], d[3], d[4], mr) for wl, ref, d, mr in layers]
        torch.cuda.synchronize()
        for (wl, ref, d, mr), y in zip(layers, outs):
            np.testing.assert_array_equal(y.cpu().numpy(), ref, err_msg=f"{wl.name} rep {rep}")


def test_staged_pipeline_on_a_side_stream():
    wl = small("side", 10, 32, 256, 25, 126, 128, "int", 91)
    ids, offs, max_rows = synth.routing(wl)
    codes, scales = synth.host_weights(wl)
    x = synth.host_tokens(wl)
    ref = oracle.moe_gemm(x, offs, ids, codes, scales, wl.N, wl.K)
    d = to_dev(codes, scales, x, ids, offs)
    st = dsa.MoeStaged(wl.N, wl.K, 1)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        y = st(dsa.Experts(d[0], d[1]), d[2], d[3], d[4], max_rows)
    s.synchronize()
    np.testing.assert_array_equal(y.cpu().numpy(), ref)


def test_staged_pipeline_orders_after_work_already_on_the_stream():
    # weights packed on the current stream just before the call, and a
    # workspace whose memory a just-freed tensor held: the conversions on the
    # second stream must come after both
    wl = small("order", 8, 64, 512, 30, 126, 128, "int", 95)
    ids, offs, max_rows = synth.routing(wl)
    codes, scales = synth.host_weights(wl)
    x = synth.host_tokens(wl)
    ref = oracle.moe_gemm(x, offs, ids, codes, scales, wl.N, wl.K)
    d = to_dev(codes, scales, x, ids, offs)
    for rep in range(3):
        big = torch.empty(64 << 20, dtype=torch.uint8, device="cuda").fill_(rep)
        del big  # its block returns to the allocator with the fill still pending
        st = dsa.MoeStaged(wl.N, wl.K, 2)
        y = st(dsa.Experts(d[0], d[1]).tiled(), d[2], d[3], d[4], max_rows)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(y.cpu().numpy(), ref, err_msg=f"rep {rep}")
        del st


def test_debug_build_flags_bad_routing():
    D = dsa.debug_lib()
    wl = small("dbg", 4, 16, 256, 10, 126, 128, "int", 101)
    codes, scales = synth.host_weights(wl)
    x = synth.host_tokens(wl)
    d = to_dev(codes, scales, x)
    ex = dsa.Experts(d[0], d[1])
    assert dsa.check_device_errors(library=D) == 0
    good_ids = torch.tensor([1, 2], dtype=torch.int32, device="cuda")
    good_offs = torch.tensor([0, 4, 10], dtype=torch.int32, device="cuda")
    dsa.moe_gemm_mxfp4(ex, d[2], good_ids, good_offs, 6, library=D)
    assert dsa.check_device_errors(library=D) == 0
    bad_ids = torch.tensor([1, 7], dtype=torch.int32, device="cuda")
    dsa.moe_gemm_mxfp4(ex, d[2], bad_ids, good_offs, 6, library=D)
    assert dsa.check_device_errors(library=D) == 7
    dsa.mxfp4_to_fp8(ex, bad_ids, library=D)
    assert dsa.check_device_errors(library=D) == 7
    bad_offs = torch.tensor([0, 4, 11], dtype=torch.int32, device="cuda")
    dsa.moe_gemm_mxfp4(ex, d[2], good_ids, bad_offs, 6, library=D)
    assert dsa.check_device_errors(library=D) == 7
    assert dsa.check_device_errors(library=D) == 0


@pytest.mark.parametrize("make", [synth.decode_layer, synth.prefill_layer])
def test_full_size_layer_sampled_experts(make):
    """The benchmark's layers (256 experts, N 4096, K 7168) run whole on the
    GPU in each path; sampled experts (the first, the largest, the last
    listed) are compared with the oracle on all their rows (prefill: their
    first 64 rows), within the fp32 accumulation bound."""
    wl = make()
    ids, offs, max_rows = synth.routing(wl)
    say(f"[moe full] {wl.name} n_act={len(ids)} max_rows={max_rows}")
    codes, scales = synth.device_weights(wl)
    x = synth.device_tokens(wl)
    d_ids, d_offs = to_dev(ids, offs)
    ex = dsa.Experts(codes, scales)
    y = dsa.moe_gemm_mxfp4(ex.tiled(), x, d_ids, d_offs, max_rows)
    y1 = dsa.moe_gemm_mxfp4(ex, x, d_ids, d_offs, max_rows)
    st = dsa.MoeStaged(wl.N, wl.K, 16)
    y2 = st(ex, x, d_ids, d_offs, max_rows)
    torch.cuda.synchronize()
    assert torch.equal(y, y1), "tiled weights differ from row-major weights"
    assert torch.equal(y, y2), "staged pipeline differs from the fused product"
    del y1, y2, st
    counts = np.diff(offs)
    for i in sorted({0, int(np.argmax(counts)), len(ids) - 1}):
        e = int(ids[i])
        r0, r1 = int(offs[i]), int(min(offs[i + 1], offs[i] + 64))
        c = codes[e:e + 1].cpu().numpy()
        s = scales[e:e + 1].cpu().numpy()
        xs = x[r0:r1].cpu().numpy()
        sub_offs = np.array([0, r1 - r0], np.int32)
        ref = oracle.moe_gemm(xs, sub_offs, np.array([0], np.int32), c, s, wl.N, wl.K)
        w8 = oracle.mxfp4_to_fp8(c, s, np.array([0], np.int32), wl.N, wl.K)
        bnd = accumulation_bound(xs, [w8[0]], [slice(0, r1 - r0)], wl.K)[0]
        g = y[r0:r1].cpu().numpy().astype(np.float64)
        err = np.abs(g - ref)
        assert (err <= bnd + 1e-30).all(), f"expert {e} rows {r0}..{r1}"
        say(f"   expert {e} rows {r1 - r0}: worst error / bound "
            f"{float((err / (bnd + 1e-30)).max()):.3f}")
