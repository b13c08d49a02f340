"""The benchmark's algorithmic byte and flop counts (host logic, no GPU).

The roofline figures divide these counts by measured time, so they are pinned here against
the values that follow from the packed format (0.5 B of codes, one fp16 scale and half a
zero byte per 128 weights) and the Llama-2 shapes.
"""

import bench


def test_packed_bytes_per_weight():
    N, K = 4096, 4096
    assert bench.packed_bytes(N, K) == N * K // 2 + N * (K // 128) * 2 + N * (K // 128) // 2
    assert bench.packed_bytes(N, K) / (N * K) == 0.51953125
    # 8-bit codes: one byte per weight and one zero byte per group; 3-bit: 3/8 B
    assert bench.packed_bytes(N, K, w_bit=8) == N * K + N * 32 * 2 + N * 32
    assert bench.packed_bytes(N, K, w_bit=3) == N * K * 3 // 8 + N * 32 * 2 + N * 16


def test_7b_decode_bytes():
    # the 7 matrices of one layer at M = 1: 105.30 MB
    layer = sum(bench.linear_bytes(1, N, K) for _, _, _, N, K in bench.MATRICES)
    assert abs(layer / 1e6 - 105.30) < 0.01
    # the fused sweep: q|k|v, o, gate|up (its output N/2 wide), down; mean bytes per launch
    fused = [bench.linear_bytes(1, N, K, g in bench.GATED) for g, (N, K) in bench.SEARCH_GROUPS.items()]
    assert sum(fused) // 4 == 26312448
    # the gated launch writes SiLU(g) * u: N/2 outputs
    assert bench.linear_bytes(1, 22016, 4096, True) == bench.linear_bytes(1, 22016, 4096) - 2 * 11008


def test_70b_resident_bytes():
    # 80 Llama-2-70B layers pack to 35.56 GB
    total = 80 * sum(bench.packed_bytes(N, K) for N, K in bench.GROUPS_70B.values())
    assert abs(total / 1e9 - 35.5625) < 0.001


def test_gemm_and_search_flops():
    gemm = sum(2 * bench.PREFILL_M * N * K for N, K in bench.SEARCH_GROUPS.values())
    assert abs(gemm / 1e12 - 0.8289) < 0.0001
    search = sum(2 * bench.CALIB_T * N * K * 20 for N, K in bench.SEARCH_GROUPS.values())
    assert abs(search / 1e12 - 4.145) < 0.001
