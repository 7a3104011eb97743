"""Host logic of V-Smooth across denoising steps (no GPU)."""
import pytest

from bit_attention_video_amd.schedule import VSmoothSchedule


def test_first_quarter_then_off():
    s = VSmoothSchedule(n_steps=8)
    assert [s.action(i) for i in range(8)] == ["cold", "warm", "off", "off", "off", "off", "off", "off"]


def test_reuse_after_window_and_refresh():
    s = VSmoothSchedule(n_steps=10, vsmooth_frac=0.6, after="reuse", refresh=3)
    assert [s.action(i) for i in range(10)] == ["cold", "warm", "warm", "cold", "warm", "warm",
                                               "reuse", "reuse", "reuse", "reuse"]


def test_edges():
    assert [VSmoothSchedule(3, vsmooth_frac=0.0, after="reuse").action(i) for i in range(3)] == ["off"] * 3
    assert [VSmoothSchedule(3, vsmooth_frac=1.0).action(i) for i in range(3)] == ["cold", "warm", "warm"]
    assert VSmoothSchedule(1).action(0) == "cold"
    with pytest.raises(ValueError):
        VSmoothSchedule(4).action(4)
    for bad in (dict(n_steps=0), dict(n_steps=4, vsmooth_frac=1.5), dict(n_steps=4, after="x"),
                dict(n_steps=4, warm_iters=0)):
        with pytest.raises(ValueError):
            VSmoothSchedule(**bad)
