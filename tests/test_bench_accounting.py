"""The bench's accounting, on the CPU: the algorithmic bytes behind
roofline.achieved, the prefill's matrix-core flops, and the cold-cache rotation.
Each expected figure is counted here item by item from the data the step must
move (or the products the chunked form executes), not through the bench's own
formula."""
import bench

MiB = 1 << 20


def _row_bytes_08b(tokens=1):
    """One real row of the 0.8B-like layer (16 value heads of 128 x 128 fp32,
    6144 bf16 channels, conv width 4), counted item by item."""
    state = 16 * 128 * 128 * 4            # one slot's state, read once and written once
    window = 3 * 6144 * 2                 # one slot's conv window, read once and written once
    x = tokens * 6144 * 2                 # the row's pre-conv activations
    out = tokens * 16 * 128 * 2           # bf16 read-out
    gates = tokens * 16 * 4 * 2           # g and beta
    return 2 * state + 2 * window + x + out + gates


def test_decode_bytes_at_64_rows_twin():
    # 2,097,152 state + 73,728 window + 12,288 x + 4,096 out + 128 gates = 2,187,392 a row, plus slot indices:
    # the read and write slot, and the swapped pair the fused commit writes (4 x 4 B)
    assert _row_bytes_08b() == 2_187_392
    weights = 6144 * 4 * 2
    want = 64 * (2_187_392 + 16) + weights
    assert want == 140_043_264
    assert bench.algorithmic_bytes(64, 0, 1, 16, 128, 128, 6144, 4, "twin") == want


def test_decode_bytes_in_place_with_tokens_and_padding():
    # 46 real rows of 4 tokens in place (one read slot each), 82 padding rows that
    # read their slot index and write a zero read-out of 4 tokens
    real = _row_bytes_08b(tokens=4) + 4
    pad = 4 + 4 * 16 * 128 * 2
    want = 46 * real + 82 * pad + 6144 * 4 * 2
    assert bench.algorithmic_bytes(46, 82, 4, 16, 128, 128, 6144, 4, "inplace") == want


def test_decode_bytes_with_a_state_per_token():
    # 3 tokens: one read of the read slot's state and window, a write of both per
    # token; the read slot and three token slots are read
    state, window = 16 * 128 * 128 * 4, 3 * 6144 * 2
    row = 4 * (state + window) + 3 * (6144 * 2 + 16 * 128 * 2 + 16 * 4 * 2) + 4 * 4
    assert bench.algorithmic_bytes(64, 0, 3, 16, 128, 128, 6144, 4, "tokens") == 64 * row + 6144 * 4 * 2


def test_prefill_flops_per_token_at_the_08b_shapes():
    # per chunk of 32 tokens and value head: W S0, Q~ S0 and K~^T U (32 x 128 x 128
    # each), K K^T and Q K^T (32 x 32 x 128 each), P U (32 x 32 x 128); 2 flops a
    # multiply-add; 16 value heads
    per_chunk = 3 * (2 * 32 * 128 * 128) + 2 * (2 * 32 * 32 * 128) + 2 * 32 * 32 * 128
    assert per_chunk == 3_932_160
    assert bench.prefill_flops_per_token(16, 128, 128) == 16 * per_chunk / 32 == 1_966_080


def test_cold_rotation_row_sets():
    # 64 twin rows write 64 MiB a step: 12 more sets must pass before a set comes
    # back for 768 MiB to be written in between, and a set takes 128 slots
    assert bench.row_sets("twin", 64, 1, MiB, hot=False) == (13, 128)
    assert bench.row_sets("inplace", 64, 1, MiB, hot=False) == (13, 64)
    # at least four sets even when a step writes more than 768 MiB
    assert bench.row_sets("twin", 256, 1, 4 * MiB, hot=False) == (4, 512)
    assert bench.row_sets("tokens", 16, 4, MiB, hot=False) == (13, 80)
    assert bench.row_sets("twin", 64, 1, MiB, hot=True) == (1, 128)


def test_kernel_code_hash_reads_the_built_library():
    """The measured-traffic gate hashes the kernels' gfx950 machine code from the
    built library: found for the kernels the bench times, different for
    different kernels, None for a kernel that is not there."""
    import os
    if not os.path.exists(os.path.join(bench.ROOT, "gated_deltanet_recurrent_decode_amd", "libgdn.so")):
        import pytest
        pytest.skip("libgdn.so is not built")
    a = bench.kernel_code_sha256(bench.STEP_KERNELS_64_TWIN)
    b = bench.kernel_code_sha256(bench.PREFILL_KERNELS)
    assert a is not None and b is not None and a != b
    assert bench.kernel_code_sha256(("_ZN3gdn_no_such_kernel",)) is None
    assert bench.kernel_code_sha256(bench.STEP_KERNELS_64_TWIN) == a  # deterministic


def test_ceiling_is_the_fastest_copy_design():
    cal = {"read_only": {"GBps": 7000.0, "us_mean": 9.0},
           "copy_slots_tile1": {"GBps": 5000.0, "us_mean": 26.8},
           "copy_slots_tile2": {"GBps": 5300.0, "us_mean": 25.3},
           "copy_contiguous_chunk256x8": {"GBps": 5700.0, "us_mean": 23.5},
           "copy_slots_tile1_hold0.9": {"GBps": 5600.0, "us_mean": 24.0}}
    c = bench.ceiling_of(cal, 140_000_000, 5200.0)
    assert c["design"] == "copy_contiguous_chunk256x8"
    assert c["on_the_steps_slots"]["design"] == "copy_slots_tile1_hold0.9"
    assert c["without_hold"]["design"] == "copy_contiguous_chunk256x8"
    cal["copy_contiguous_chunk256x8"]["GBps"] = 5500.0
    c2 = bench.ceiling_of(cal, 140_000_000, 5200.0)
    assert c2["design"] == "copy_slots_tile1_hold0.9"
    assert c2["without_hold"]["design"] == "copy_contiguous_chunk256x8"
    assert abs(c2["without_hold"]["step_fraction"] - 5200.0 / 5500.0) < 1e-12
    cal["copy_contiguous_chunk256x8"]["GBps"] = 5700.0
    assert abs(c["us_at_step_bytes"] - 140_000_000 / 5.7e12 * 1e6) < 1e-9
    assert abs(c["step_fraction"] - 5200.0 / 5700.0) < 1e-12


def test_step_kernel_label_follows_the_routing():
    lab = bench.step_kernel_label
    assert lab(True, 64, 1, 16, 16, 128, 128, False) == "gdn_step_tile_kernel"
    # past one round of four-tile workgroups: consecutive row parts of one round each
    assert lab(True, 128, 1, 16, 16, 128, 128, False) == "gdn_step_tile_kernel (2 launches over consecutive rows)"
    assert lab(True, 64, 1, 16, 32, 128, 128, False) == "gdn_step_tile_kernel (2 launches over consecutive rows)"
    assert lab(True, 256, 1, 16, 16, 128, 128, False) == "gdn_step_tile_kernel (4 launches over consecutive rows)"
    assert lab(True, 80, 1, 16, 16, 128, 128, False) == "gdn_step_tile_kernel"   # halves of 2.5 heads a CU
    assert lab(True, 128, 1, 16, 16, 64, 64, False) == "gdn_step_tile_kernel"    # d = 64: no four-tile path
    assert lab(False, 64, 1, 16, 16, 128, 128, False) == "gdn_step_kernel (4 key heads a workgroup)"
    assert lab(False, 64, 1, 8, 16, 128, 128, False) == "gdn_step_kernel (2 key heads a workgroup)"
    assert lab(False, 16, 1, 16, 16, 128, 128, False) == "gdn_step_tile_kernel"     # 256 heads: one a CU
    assert lab(False, 128, 1, 16, 16, 128, 128, False) == "gdn_step_tile_kernel"    # 2048 heads: past 4 a CU
    assert lab(False, 64, 1, 4, 16, 128, 128, False) == "gdn_step_kernel"           # G = 4
    assert lab(False, 64, 4, 16, 16, 128, 128, False) == "gdn_step_kernel"          # a token walk
    assert lab(False, 64, 1, 16, 16, 64, 64, False) == "gdn_step_tile_kernel"       # d = 64: no grouping
    assert lab(False, 16, 4, 16, 16, 128, 128, True) == "gdn_step_kernel"           # per-token states
