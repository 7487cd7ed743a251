"""The algorithmic byte models against the figures the pages print (tests/golden)."""
import json
import os

from memory_bound_decode_add_amd import traffic as T

FIG = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_figures.json")))


def test_add_rmsnorm_bytes_per_element_and_times():
    f = FIG["add_rmsnorm_bytes"]
    M, H = f["rows"], f["cols"]
    fused = T.add_rmsnorm_bytes(M, H)
    eager = T.add_rmsnorm_eager_bytes(M, H)
    assert (fused - 2 * H) // (M * H) == f["fused_bytes_per_elem"] == 8
    assert round(eager / (M * H)) == f["eager_bytes_per_elem"] == 42
    # the page's times follow from bytes / 226 GB/s
    assert round(eager / (f["mixed_rw_gbps"] * 1e9) * 1e3, 1) == f["eager_ms"]
    assert round(fused / (f["mixed_rw_gbps"] * 1e9) * 1e3, 2) == f["fused_ms"]
    # 42/8 = 5.25 by bytes; the page's 5.2x is the ratio of its rounded times
    assert abs(eager / fused - f["speedup"]) < 0.1
    assert round(f["eager_ms"] / f["fused_ms"], 1) == f["speedup"]


def test_swiglu_bytes_per_element():
    f = FIG["swiglu_bytes"]
    M, K, N = 1, 4096, 4096
    unfused = T.unfused_act_gemv_bytes(M, K, N)
    gemv_on_act = M * K * 2 + T.w4_weight_bytes(K, N) + M * N * 2     # reads act, writes z
    scale = 2 * M * N * 2 + 4                                          # separate scale launch
    eager_swiglu = unfused - gemv_on_act - scale
    assert eager_swiglu == f["eager_bytes_per_elem"] * M * K           # silu + mul: 10 B/elem
    # one standalone fused SwiGLU kernel reads g, u and writes act: 6 B/elem; the fused
    # prologue does not even write act, reading only g and u
    assert 3 * 2 == f["fused_bytes_per_elem"]
    assert (T.swiglu_w4_gemv_bytes(M, K, N) - T.w4_weight_bytes(K, N) - M * N * 2 - 4) == 4 * M * K
    assert abs(f["flops_per_elem"] / f["fused_bytes_per_elem"] - f["flops_per_byte"]) < 0.05
    assert abs(1 - f["fused_bytes_per_elem"] / f["eager_bytes_per_elem"] - f["time_saving_fraction"]) < 1e-9


def test_silu_output_bytes_llama3_8b():
    f = FIG["silu_output_llama3_8b"]
    per_layer = f["width"] * f["bytes_per_elem"]
    assert round(per_layer / 1024) == f["approx_kilobytes_per_token_per_layer"]
    assert round(2 * per_layer / 1024) == f["fused_saving_kilobytes_per_token_per_layer"]
    assert round(2 * per_layer * f["layers"] / 1e6, 1) == f["approx_megabytes_per_token"]


def test_product_bytes():
    f = FIG["product_buffer"]
    assert T.product_bytes(f["M"], f["K"], f["N"]) == 94_371_840
    # unfused product path: the product is written and read back
    assert T.unfused_product_gemv_bytes(9216, 2560) == 200_961_028


def test_config_byte_totals():
    assert T.swiglu_w4_gemv_bytes(1, 1024, 512) == 275_460
    assert T.swiglu_w4_gemv_bytes(1, 9216, 2560) == 12_207_108
    assert T.add_rmsnorm_bytes(8192, 4096) == 268_443_648
    assert T.mlp_layer_bytes(16, 4096, 14336, True) == 93_593_604
    assert T.mlp_layer_bytes(1, 1536, 8960, False) == 21_382_148
    assert 28 * T.mlp_layer_bytes(1, 1536, 8960, False) == 598_700_144
    # two-kernel layer, by hand: kernel 1 = x, r (6,144) + norm weight (3,072) + gate_up
    # (13,762,560 + 430,080) + h (3,072) + act (17,920); kernel 2 = act (17,920) + down
    # (6,881,280 + 215,040) + out (3,072) + scale (4) + h -> residual (6,144)
    assert T.mlp2_layer_bytes(1, 1536, 8960, False) == 14_222_848 + 7_123_460


def test_fp4_gemv_bytes():
    # E2M1 codes (K*N/2) + one E4M3 byte per 16 weights + g, u in + y out + the scalar
    assert T.fp4_weight_bytes(9216, 2560) == 11_796_480 + 1_474_560
    assert T.swiglu_fp4_gemv_bytes(1, 9216, 2560) == 11_796_480 + 1_474_560 + 36_864 + 5_120 + 4
    assert T.swiglu_fp4_gemv_bytes(1, 9216, 2560) - T.swiglu_w4_gemv_bytes(1, 9216, 2560) == 1_474_560 - 368_640


def test_swiglu_epilogue_layer_bytes():
    # the form with SwiGLU as the gate_up epilogue writes act [M, I] where the three-kernel
    # form writes the gate/up pair [M, 2I] and reads it back: 2 * M * I * 2 bytes fewer
    M, H, I = 16, 4096, 14336
    assert T.mlp_layer_bytes(M, H, I, True) - T.mlp2_layer_bytes(M, H, I, True) == 2 * M * I * 2
    assert T.w4_gemv_swiglu_bytes(M, H, I) == H * 2 * I // 2 + (H // 128) * 2 * I * 2 + M * H * 2 + M * I * 2
