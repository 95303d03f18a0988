"""The randomized differential tests' draws (host logic, CPU): every entry
point, and every launch choice of the GEMM over wide matrices, is reached."""

from test_gpu_random import CASES, ENTRIES, WIDE_CASES, draw, draw_wide, route_wide


def test_draw_covers_every_entry_point():
    seen = {draw(i)[0] for i in range(CASES)}
    assert seen == set(ENTRIES)


def test_draw_reaches_both_gated_paths():
    gated = [draw(i)[2] for i in range(CASES) if draw(i)[0] == "ffn_gate_up_q4_0"]
    assert any(m <= 4 for m in gated) and any(m > 8 for m in gated) and any(4 < m <= 8 for m in gated)


def test_draw_wide_reaches_every_route():
    # 256 x 256 tiles need at least 192 of them (M >= 1536 at these N): the
    # fixed prefill shapes cover those
    seen = {route_wide(*draw_wide(i)[2:4]) for i in range(WIDE_CASES)}
    assert seen == {"mid_1x1", "mid_2x1", "mid_1x2", "mid_2x2", "mid_2x2_4waves", "tiles_128"}, seen


def test_route_wide_matches_measured_choices():
    # the launch table's choices at shapes it was measured on
    assert route_wide(16, 8192) == "mid_1x1"
    assert route_wide(64, 8192) == "mid_1x2"
    assert route_wide(128, 8192) == "mid_2x2"
    assert route_wide(80, 4096) == "mid_2x1"
    assert route_wide(128, 16384) == "mid_2x2_4waves"
    assert route_wide(256, 8192) == "mid_2x2_4waves"
    assert route_wide(384, 8192) == "tiles_128"
    assert route_wide(2048, 8192) == "tiles_256"
