"""GPU parity of the int4 decode and the SwiGLU-prologue / identity GEMVs against the
fp64 oracle (through the C ABI, via the ctypes binding)."""
import numpy as np
import pytest
import torch

import memory_bound_decode_add_amd as F
import oracle as O
import synth
from helpers import assert_bits_equal, assert_close, say

pytestmark = pytest.mark.gpu
DEV = "cuda"


def to_dev(inp: synth.GemvInputs):
    return (F.from_bits(inp.g), F.from_bits(inp.u), F.W4Weight.from_numpy(inp.W.qweight, inp.W.scales),
            None if inp.residual is None else F.from_bits(inp.residual))


def run_gemv(inp, out_scale=None, residual=True, ws=None):
    g, u, W, res = to_dev(inp)
    s = None if out_scale is None else F.scalar(out_scale)
    y = F.swiglu_w4_gemv(g, u, W, s, res if residual else None, ws=ws)
    torch.cuda.synchronize()
    return F.to_bits(y)


# ---------------------------------------------------------------------------
# int4 decode: bit-exact
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("K,N", [(1024, 512), (9216, 2560), (256, 8)])
def test_unpack_and_dequant_bit_exact(K, N):
    say(f"[unpack/dequant] K={K} N={N}")
    W = synth.w4_weight(np.random.default_rng(K + N), K, N)
    Wd = F.W4Weight.from_numpy(W.qweight, W.scales)
    q = F.w4_unpack(Wd).cpu().numpy()
    w = F.w4_dequant(Wd).cpu().numpy()
    torch.cuda.synchronize()
    assert np.array_equal(q, O.w4_unpack(W.qweight))
    ref = O.w4_dequant(W.qweight, W.scales)
    assert np.array_equal(w.astype(np.float64), ref)


def test_unpack_every_code_in_every_position():
    say("[unpack] all codes")
    k, n = np.meshgrid(np.arange(128), np.arange(64), indexing="ij")
    q = (((k + n) % 16) - 8).astype(np.int8)          # every code at every nibble position
    words = synth.pack_int4(q)
    sc = np.full((1, 64), 0x3F80, dtype=np.uint16)
    Wd = F.W4Weight.from_numpy(words, sc)
    got = F.w4_unpack(Wd).cpu().numpy()
    assert np.array_equal(got, q)


# ---------------------------------------------------------------------------
# the SwiGLU GEMV
# ---------------------------------------------------------------------------
def test_swiglu_gemv_small_config():
    say("[gemv] M=1 K=1024 N=512 scale 0.5 seed 0")
    inp = synth.make("swiglu_w4_gemv_1x1024x512")
    y = run_gemv(inp, inp.out_scale)
    ref = O.swiglu_w4_gemv(inp.g, inp.u, inp.W.qweight, inp.W.scales, inp.out_scale)
    say("  worst err/bound", assert_close(y, ref, "C1"))


def test_swiglu_gemv_decode_shape_full():
    say("[gemv] M=1 K=9216 N=2560 scale 1.0 seed 0 (default split)")
    inp = synth.make("swiglu_w4_gemv_1x9216x2560")
    y = run_gemv(inp, inp.out_scale)
    ref = O.swiglu_w4_gemv(inp.g, inp.u, inp.W.qweight, inp.W.scales, inp.out_scale)
    say("  worst err/bound", assert_close(y, ref, "C2"))
    y2 = run_gemv(inp, inp.out_scale)
    assert_bits_equal(y, y2, "C2 repeat (determinism)")


@pytest.mark.parametrize("split", [1, 2, 5, 9, 18, 72])
def test_swiglu_gemv_every_split(split):
    say(f"[gemv] M=1 K=9216 N=2560 forced split {split}")
    inp = synth.make("swiglu_w4_gemv_1x9216x2560")
    ref = O.swiglu_w4_gemv(inp.g, inp.u, inp.W.qweight, inp.W.scales, 1.0)
    try:
        F.set_gemv_split(split)
        y = run_gemv(inp, 1.0)
        y2 = run_gemv(inp, 1.0)
    finally:
        F.set_gemv_split(0)
    assert_close(y, ref, f"split {split}")
    assert_bits_equal(y, y2, f"split {split} repeat")


@pytest.mark.parametrize("M,K,N", [(1, 128, 8), (3, 384, 520), (5, 1280, 136), (16, 2048, 1032),
                                   (2, 256, 4104), (8, 4096, 776), (16, 14336, 128),
                                   (1, 1920, 17928), (2, 1024, 20480)])
def test_swiglu_gemv_ragged_shapes_with_residual(M, K, N):
    say(f"[gemv] ragged M={M} K={K} N={N} with residual")
    inp = synth.swiglu_gemv_inputs(M, K, N, seed=M * 7 + K + N, out_scale=0.75, with_residual=True)
    y = run_gemv(inp, 0.75, residual=True)
    ref = O.swiglu_w4_gemv(inp.g, inp.u, inp.W.qweight, inp.W.scales, 0.75, inp.residual)
    assert_close(y, ref, f"M={M} K={K} N={N}")


@pytest.mark.parametrize("M,K,N", [(17, 1024, 520), (32, 9216, 2560), (40, 2048, 1032), (64, 4096, 776),
                                   (64, 14336, 264), (24, 128, 8)])
def test_swiglu_gemv_row_blocks_with_residual(M, K, N):
    # 17..64 rows: the matrix-core kernel with two or four 16-row blocks per weight load
    say(f"[gemv] row blocks M={M} K={K} N={N} with residual")
    inp = synth.swiglu_gemv_inputs(M, K, N, seed=M * 11 + K + N, out_scale=0.5, with_residual=True)
    g, u, W, res = to_dev(inp)
    s = F.scalar(0.5)
    y = F.to_bits(F.swiglu_w4_gemv(g, u, W, s, res))
    ref = O.swiglu_w4_gemv(inp.g, inp.u, inp.W.qweight, inp.W.scales, 0.5, inp.residual)
    assert_close(y, ref, f"M={M} K={K} N={N}")
    # the same call again, with a workspace full of garbage: identical bits
    ws = F.workspace(F.gemv_workspace_bytes(M, K, N))
    ws.fill_(0xFF)
    y2 = F.to_bits(F.swiglu_w4_gemv(g, u, W, s, res, ws=ws))
    assert_bits_equal(y, y2, "repeat")
    # a forced split-K (a 16-row VALU kernel) does not apply past 16 rows
    try:
        F.set_gemv_split(4)
        y3 = F.to_bits(F.swiglu_w4_gemv(g, u, W, s, res))
    finally:
        F.set_gemv_split(0)
    assert_bits_equal(y, y3, "forced split ignored")
    # in place: y is the residual
    F.swiglu_w4_gemv(g, u, W, s, res, out=res)
    torch.cuda.synchronize()
    assert_bits_equal(F.to_bits(res), y, "in place")


def test_swiglu_gemv_strided_rows_and_null_scale():
    say("[gemv] g, u as halves of one [M, 2K] buffer; out_scale NULL")
    M, K, N = 4, 1024, 264
    inp = synth.swiglu_gemv_inputs(M, K, N, seed=3)
    gu = np.concatenate([inp.g, inp.u], axis=1)
    t = F.from_bits(gu)
    W = F.W4Weight.from_numpy(inp.W.qweight, inp.W.scales)
    y = F.to_bits(F.swiglu_w4_gemv(t[:, :K], t[:, K:], W, None))
    ref = O.swiglu_w4_gemv(inp.g, inp.u, inp.W.qweight, inp.W.scales, 1.0)
    assert_close(y, ref, "strided")


def test_swiglu_gemv_output_scale_matrix():
    """The folded scale: a value changed in device memory is read at launch."""
    say("[gemv] output-scale matrix")
    inp = synth.swiglu_gemv_inputs(1, 2048, 512, seed=5)
    g, u, W, _ = to_dev(inp)
    s = F.scalar(1.0)
    for v in (0.0, 2.0**-3, 0.5, 1.0, 3.7):
        s.fill_(v)
        y = F.to_bits(F.swiglu_w4_gemv(g, u, W, s))
        ref = O.swiglu_w4_gemv(inp.g, inp.u, inp.W.qweight, inp.W.scales, v)
        if v == 0.0:
            assert np.all(O.bf16_to_f64(y) == 0)
        else:
            assert_close(y, ref, f"scale {v}")


def _exact_case(M, K, N, seed):
    """g in {0, 32}, u in {-1, 0, 1}, power-of-two scales: every partial sum is exact in
    fp32 (see the bound below), so the GPU must match exact rational arithmetic."""
    rng = np.random.default_rng(seed)
    g = rng.choice([0.0, 32.0], size=(M, K)).astype(np.float32)
    u = rng.integers(-1, 2, size=(M, K)).astype(np.float32)
    q = rng.integers(-8, 8, size=(K, N)).astype(np.int8)
    s = rng.choice([2.0**-6, 2.0**-7], size=(K // 128, N)).astype(np.float32)
    exact = (g.astype(np.float64) * u) @ (q.astype(np.float64) * np.repeat(s, 128, axis=0))
    # silu(32) = 32 and silu(0) = 0 exactly in fp32.  A group's largest |act| = 32 is stored
    # as 2^14 (scale 2^-9), so every per-lane dot is a multiple of 2^14 below 2^22, and every
    # scaled partial sum a multiple of 2^14 * 2^-7 * 2^-9 = 2^-2 bounded by
    # sum |act q s| <= 32 * 8 * 2^-6 * K = 4K.  fp32 holds all of them exactly if 4K / 2^-2 < 2^24.
    assert 16 * K < 2**24
    return (synth.f32_to_bf16_bits(g), synth.f32_to_bf16_bits(u), synth.pack_int4(q),
            synth.f32_to_bf16_bits(s), exact)


@pytest.mark.parametrize("M,K,N", [(1, 1024, 512), (1, 9216, 2560), (4, 2048, 256), (8, 1024, 136),
                                   (16, 2048, 264), (16, 14336, 520), (1, 1536, 17920), (2, 1024, 20488)])
def test_swiglu_gemv_exact_special_cases_bit_exact(M, K, N):
    say(f"[gemv] exact special case M={M} K={K} N={N}")
    gb, ub, qw, sb, exact = _exact_case(M, K, N, seed=K + N)
    W = F.W4Weight.from_numpy(qw, sb)
    for scale in (0.5, 1.0):
        y = F.to_bits(F.swiglu_w4_gemv(F.from_bits(gb), F.from_bits(ub), W, F.scalar(scale)))
        want = O.f64_to_bf16(exact * scale)     # exact value, one rounding
        assert_bits_equal(y, want, f"exact scale={scale}")


# ---------------------------------------------------------------------------
# the column kernel at every columns-per-wave variant (forced workgroup shapes)
# ---------------------------------------------------------------------------
def _column_plan_accepts(M, K, waves, cols):
    """The column planner's conditions for taking a forced (waves, cols) shape: at most
    the variant's columns per wave for this chunk count and row count, and staging waves
    (those the dot waves leave of 16) for every (row, 512-wide block) task."""
    nch = K // 32
    ni = -(-nch // 64)
    mr = 1 if M <= 1 else 2 if M <= 2 else 4
    if mr >= 4:
        cmax = 4 if ni <= 1 else 2 if ni <= 3 else 1
    else:
        cmax = 8 if ni <= 1 else 4 if ni <= 3 else 3 if ni <= 4 else 2 if ni <= 6 else 1
    ntask = mr * -(-K // 512)
    stagers = min(min(8, max(2, ntask)), 16 - waves)
    return -(-cols // waves) <= cmax and stagers * 8 >= ntask and stagers >= 1


# (M, K, dot waves, columns per workgroup): columns per wave 1, 2, 3, 4, 5 -> 6, 6, 7 -> 8
# and 8, at one to four rows, so the outputs per wave (rows x columns) run over 1..16 and
# fill the last group of four partly and wholly; N leaves a ragged last workgroup.
FORCED = [(1, 1024, 8, 8), (1, 9216, 8, 16), (1, 8192, 8, 24), (1, 1024, 10, 36), (1, 1024, 8, 40),
          (1, 1024, 8, 48), (1, 1024, 8, 56), (1, 1024, 8, 64), (2, 1024, 8, 64), (2, 6144, 8, 32),
          (3, 1024, 8, 32), (4, 1024, 8, 24), (4, 4096, 8, 16), (2, 9216, 8, 8)]


@pytest.mark.parametrize("M,K,waves,cols", FORCED)
@pytest.mark.parametrize("pro", ["swiglu", "identity"])
def test_column_kernel_forced_tilings(M, K, waves, cols, pro):
    assert _column_plan_accepts(M, K, waves, cols)
    N = -(-(3 * cols + 12) // 8) * 8
    say(f"[gemv forced tiling] {pro} M={M} K={K} N={N} waves={waves} cols={cols}")
    inp = synth.swiglu_gemv_inputs(M, K, N, seed=M * 7 + cols, out_scale=0.75, with_residual=True)
    F.set_gemv_tiling(waves, cols)
    try:
        if pro == "swiglu":
            y = run_gemv(inp, inp.out_scale)
            ref = O.swiglu_w4_gemv(inp.g, inp.u, inp.W.qweight, inp.W.scales, inp.out_scale, inp.residual)
        else:
            y = F.to_bits(F.w4_gemv(F.from_bits(inp.g), F.W4Weight.from_numpy(inp.W.qweight, inp.W.scales),
                                    F.scalar(inp.out_scale)))
            torch.cuda.synchronize()
            ref = O.w4_gemv(inp.g, inp.W.qweight, inp.W.scales, inp.out_scale)
    finally:
        F.set_gemv_tiling(0, 0)
    assert_close(y, ref, f"forced tiling {pro} M={M} K={K} waves={waves} cols={cols}")


# ---------------------------------------------------------------------------
# the identity-prologue GEMV (gate_up)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("M,K,N", [(1, 1536, 17920), (16, 4096, 28672), (3, 640, 392), (64, 1024, 2056),
                                   (21, 4096, 1024)])
def test_w4_gemv_identity(M, K, N):
    say(f"[gemv identity] M={M} K={K} N={N}")
    rng = np.random.default_rng(M + K + N)
    x = synth._normal_bf16(rng, (M, K))
    W = synth.w4_weight(rng, K, N)
    y = F.to_bits(F.w4_gemv(F.from_bits(x), F.W4Weight.from_numpy(W.qweight, W.scales)))
    torch.cuda.synchronize()
    ref = O.w4_gemv(x, W.qweight, W.scales)
    assert_close(y, ref, "identity")


def test_w4_gemv_identity_large_dynamic_range():
    """Activations far outside fp16's range still work (per-group power-of-two scaling)."""
    say("[gemv identity] large dynamic range")
    M, K, N = 2, 1024, 256
    rng = np.random.default_rng(11)
    xf = rng.standard_normal((M, K)).astype(np.float32)
    xf[0] *= 1e6          # beyond fp16's 65504
    xf[1] *= 1e-6         # deep in fp16's subnormal range
    x = synth.f32_to_bf16_bits(xf)
    W = synth.w4_weight(rng, K, N)
    y = F.to_bits(F.w4_gemv(F.from_bits(x), F.W4Weight.from_numpy(W.qweight, W.scales)))
    ref = O.w4_gemv(x, W.qweight, W.scales)
    for m in range(M):
        assert_close(y[m:m + 1], ref[m:m + 1], f"row {m}")


@pytest.mark.parametrize("M,K,N,split", [(16, 14336, 4096, 0), (8, 9216, 2560, 0), (5, 4096, 1000, 0),
                                         (1, 9216, 2560, 7), (3, 2048, 520, 4)])
def test_split_k_ignores_workspace_contents(M, K, N, split):
    """K-sliced GEMVs (the matrix-core kernel at 5..16 rows, the VALU split kernel when
    forced) write every partial they read back: a workspace full of NaN patterns, reused
    for two different inputs in a row, gives the oracle's result both times."""
    say(f"[split-K] M={M} K={K} N={N} forced split={split}: workspace filled with NaN patterns")
    if split:
        F.set_gemv_split(split)
    try:
        need = F.gemv_workspace_bytes(M, K, N)
        assert need > 0
        ws = torch.full((need,), 0xFF, dtype=torch.uint8, device=DEV)
        for seed in (1, 2):
            inp = synth.swiglu_gemv_inputs(M, K, N, seed=seed * 100 + M, out_scale=0.5, with_residual=True)
            got = run_gemv(inp, 0.5, True, ws=ws)
            ref = O.swiglu_w4_gemv(inp.g, inp.u, inp.W.qweight, inp.W.scales, 0.5, inp.residual)
            say(f"  seed {seed}: worst err/bound {assert_close(got, ref, 'y'):.3f}")
    finally:
        F.set_gemv_split(0)


@pytest.mark.parametrize("M,K,N", [(64, 9216, 2560), (16, 14336, 4096)])
def test_gemv_graph_replays_match_eager(M, K, N):
    # the split-K GEMV (main kernel + finish kernel) captured once and replayed several
    # times, with other eager work and synchronisations between the replays
    say(f"[gemv] graph replays M={M} K={K} N={N}")
    inp = synth.swiglu_gemv_inputs(M, K, N, seed=M + K + N, out_scale=0.5, with_residual=True)
    g, u, W, res = to_dev(inp)
    s = F.scalar(0.5)
    ws = F.workspace(F.gemv_workspace_bytes(M, K, N))
    ref = F.to_bits(F.swiglu_w4_gemv(g, u, W, s, res, ws=ws))
    y = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        F.swiglu_w4_gemv(g, u, W, s, res, out=y, ws=ws)          # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        F.swiglu_w4_gemv(g, u, W, s, res, out=y, ws=ws)
    for i in range(3):
        y.fill_(0)
        ws.fill_(0xFF)                                            # workspace contents must not matter
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert_bits_equal(F.to_bits(y), ref, f"replay {i}")
        F.swiglu_w4_gemv(g, u, W, s, res, ws=ws)                  # eager work between replays
        torch.cuda.synchronize()
    assert_close(ref, O.swiglu_w4_gemv(inp.g, inp.u, inp.W.qweight, inp.W.scales, 0.5, inp.residual), "eager vs oracle")


# ---------------------------------------------------------------------------
# the matrix-core kernel whose waves split K: every tile and groups-per-wave variant,
# forced (the built-in plan takes it with one group per wave and the SwiGLU prologue)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("pro", ["swiglu", "identity"])
@pytest.mark.parametrize("tiles,gw", [(8, 1), (8, 2), (4, 1), (4, 2), (8, 3), (4, 4)])
def test_kmfma_kernel_every_variant(pro, tiles, gw):
    if pro == "swiglu" and gw > 2:
        pytest.skip("the SwiGLU prologue takes at most 2 groups per wave")
    M, K, N = 12, 4224, 1000            # 33 groups: a ragged last slice; 1000 columns: a ragged tile
    say(f"[kmfma] {pro} tiles={tiles} groups/wave={gw} M={M} K={K} N={N}")
    inp = synth.swiglu_gemv_inputs(M, K, N, seed=tiles * 10 + gw, out_scale=0.5, with_residual=True)
    g, u, W, res = to_dev(inp)
    s = F.scalar(0.5)
    F.set_mfma_plan(2, tiles, gw)
    try:
        ws = torch.full((max(16, F.gemv_workspace_bytes(M, K, N)),), 0xFF, dtype=torch.uint8, device=DEV)
        if pro == "swiglu":
            y = F.to_bits(F.swiglu_w4_gemv(g, u, W, s, res, ws=ws))
            y2 = F.to_bits(F.swiglu_w4_gemv(g, u, W, s, res, ws=ws))
            ref = O.swiglu_w4_gemv(inp.g, inp.u, inp.W.qweight, inp.W.scales, 0.5, inp.residual)
        else:
            y = F.to_bits(F.w4_gemv(g, W, s, ws=ws))
            y2 = F.to_bits(F.w4_gemv(g, W, s, ws=ws))
            ref = O.w4_gemv(inp.g, inp.W.qweight, inp.W.scales, 0.5)
    finally:
        F.set_mfma_plan(0)
    say("  worst err/bound", assert_close(y, ref, "y"))
    assert_bits_equal(y, y2, "repeat")


@pytest.mark.parametrize("waves", [6, 7, 8])
@pytest.mark.parametrize("tiles,gw", [(8, 1), (4, 2)])
def test_kmfma_kernel_wave_counts(waves, tiles, gw):
    # fewer waves than 8 tiles: some waves sum and store two tiles
    M, K, N = 16, 4224, 1000
    say(f"[kmfma] SwiGLU waves={waves} tiles={tiles} groups/wave={gw} M={M} K={K} N={N}")
    inp = synth.swiglu_gemv_inputs(M, K, N, seed=waves * 100 + tiles * 10 + gw, out_scale=0.5, with_residual=True)
    g, u, W, res = to_dev(inp)
    s = F.scalar(0.5)
    F.set_mfma_plan(2, tiles, gw)
    F.set_kmfma_waves(waves)
    try:
        ws = torch.full((max(16, F.gemv_workspace_bytes(M, K, N)),), 0xFF, dtype=torch.uint8, device=DEV)
        y = F.to_bits(F.swiglu_w4_gemv(g, u, W, s, res, ws=ws))
        y2 = F.to_bits(F.swiglu_w4_gemv(g, u, W, s, res, ws=ws))
        xi = F.to_bits(F.w4_gemv(g, W, s, ws=ws))
    finally:
        F.set_kmfma_waves(0)
        F.set_mfma_plan(0)
    say("  worst err/bound", assert_close(y, O.swiglu_w4_gemv(inp.g, inp.u, inp.W.qweight, inp.W.scales, 0.5,
                                                               inp.residual), "y"))
    assert_bits_equal(y, y2, "repeat")
    say("  identity worst err/bound", assert_close(xi, O.w4_gemv(inp.g, inp.W.qweight, inp.W.scales, 0.5), "x"))


# ---------------------------------------------------------------------------
# outputs that should be exactly zero: the kernels keep a known offset in every decoded
# weight (1032 + q or 1152 + 16 q in fp16) and remove it once per chunk or group, so a
# zero weight column leaves the rounding of those offset sums.  The offsets are summed
# from the same fp16 activation values the dot uses, so what is left is bounded by fp32
# rounding of sums of about 1152 * |a| per k: below 2^-10 of sum_k |act| * scale.
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("M,K,N,split", [(1, 9216, 2560, 0), (3, 4096, 520, 0), (8, 9216, 2560, 0),
                                         (16, 14336, 4096, 0), (32, 2048, 776, 0), (1, 4096, 520, 4)])
def test_zero_weight_columns_give_zero(M, K, N, split):
    say(f"[zero columns] M={M} K={K} N={N} forced split={split}")
    inp = synth.swiglu_gemv_inputs(M, K, N, seed=M + K + N, out_scale=1.0, with_residual=True)
    q = O.w4_unpack(inp.W.qweight).astype(np.int64)
    zero_cols = np.arange(0, N, 7)
    q[:, zero_cols] = 0
    qw = synth.pack_int4(q)
    W = F.W4Weight.from_numpy(qw, inp.W.scales)
    g, u, res = F.from_bits(inp.g), F.from_bits(inp.u), F.from_bits(inp.residual)
    if split:
        F.set_gemv_split(split)
    try:
        ws = F.workspace(F.gemv_workspace_bytes(M, K, N))
        y = F.to_bits(F.swiglu_w4_gemv(g, u, W, F.scalar(1.0), None, ws=ws))
        yr = F.to_bits(F.swiglu_w4_gemv(g, u, W, F.scalar(1.0), res, ws=ws))
    finally:
        F.set_gemv_split(0)
    act = np.abs(O.silu_mul(O.bf16_to_f64(inp.g), O.bf16_to_f64(inp.u)))
    smax = O.bf16_to_f64(inp.W.scales).max()
    bound = 2.0 ** -10 * act.sum(axis=1, keepdims=True) * smax           # per row
    z = O.bf16_to_f64(y)[:, zero_cols]
    assert np.all(np.abs(z) <= bound), f"worst |y| / bound = {np.max(np.abs(z) / bound):.3f}"
    say(f"  largest |y| on a zero column: {np.abs(z).max():.3e} (bound {bound.min():.3e} .. {bound.max():.3e})")
    # with the residual in the epilogue, y is the residual to within that bound plus one rounding
    r = O.bf16_to_f64(inp.residual)[:, zero_cols]
    zr = O.bf16_to_f64(yr)[:, zero_cols]
    assert np.all(np.abs(zr - r) <= bound + np.abs(r) * 2.0 ** -8)
    # the other columns are unaffected
    ref = O.swiglu_w4_gemv(inp.g, inp.u, qw, inp.W.scales, 1.0)
    assert_close(y, ref, "y")
