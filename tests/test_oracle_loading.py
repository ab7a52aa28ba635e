"""Pins for the loading controller ([CB] section 位置恢复、KV 存储与加载流水线)
and the same function in the C ABI (cb_loading_ratio; host only, no GPU)."""
import json
import os

import pytest

from oracle.loading import load_seconds, loading_ratio

HERE = os.path.dirname(os.path.abspath(__file__))


def _golden():
    return json.load(open(os.path.join(HERE, "golden", "loading_controller.json")))


def test_worked_examples_of_the_page():
    g = _golden()
    floor = g["floor"]
    for c in g["cases"]:
        # per layer: T_prefill = T_recompute(15%) / 15%; T_load as printed (1 token of 1 byte per ms)
        t_prefill = c["recompute_ms_at_floor"] / floor
        r = loading_ratio(c["load_ms"], 1.0, 1.0, t_prefill, floor)
        if c["load_hides_recompute"]:
            # the load is the longer one: the controller recomputes more, exactly until the two match
            assert r > floor
            assert r * t_prefill == pytest.approx(c["load_ms"])
        else:
            # recompute already exceeds the load: stay at the quality floor
            assert r == floor
            assert floor * t_prefill > c["load_ms"]
    # the two printed cases give 80% and the 15% floor
    r7 = loading_ratio(16.0, 1.0, 1.0, 3.0 / 0.15, 0.15)
    r70 = loading_ratio(4.0, 1.0, 1.0, 7.0 / 0.15, 0.15)
    assert r7 == pytest.approx(0.8) and r70 == 0.15


def test_closed_forms_and_limits():
    # 128 KiB per token (8B shape, bf16), 4096 tokens over 4.8 GB/s (the pages' NVMe) -> 0.112 s
    assert load_seconds(131072, 4096, 4.8e9) == pytest.approx(131072 * 4096 / 4.8e9)
    assert loading_ratio(1.0, 10.0, 1.0, 1.0) == 1.0                       # capped
    assert loading_ratio(0.0, 10.0, 1.0, 1.0) == 0.15                      # free load -> floor
    assert loading_ratio(1.0, 1.0, 1.0, 4.0, r_min=0.0) == pytest.approx(0.25)
    lo, hi = loading_ratio(1.0, 100.0, 2e3, 1.0, 0.0), loading_ratio(1.0, 100.0, 1e3, 1.0, 0.0)
    assert hi == pytest.approx(2 * lo)                                     # half the bandwidth, twice the share
    with pytest.raises(ValueError):
        loading_ratio(1.0, 1.0, 0.0, 1.0)


def test_library_matches_the_oracle():
    from cacheblend_selective_recompute_amd import _abi
    if not os.path.exists(_abi.LIB_PATH):
        pytest.skip("library not built")
    lib = _abi.load()
    for args in [(131072, 4096, 4.8e9, 0.5, 0.15), (163840, 4096, 4.8e9, 2.0, 0.15), (1.0, 10.0, 1.0, 1.0, 0.15),
                 (0.0, 1.0, 1.0, 1.0, 0.15), (16.0, 1.0, 1.0, 20.0, 0.15), (4.0, 1.0, 1.0, 46.0, 0.15)]:
        assert lib.cb_loading_ratio(*map(float, args)) == pytest.approx(loading_ratio(*args), rel=1e-12)
    assert lib.cb_loading_ratio(1.0, 1.0, 0.0, 1.0, 0.15) == -1.0
    assert lib.cb_loading_ratio(1.0, 1.0, 1.0, 0.0, 0.15) == -1.0
