"""Plain oracle of the CacheBlend loading controller (TEST INFRASTRUCTURE ONLY).

[CB] "CacheBlend 完全拆解" (pinghaoyang.com.cn), section 位置恢复、KV 存储与加载
流水线, the loading-controller paragraphs: recomputing a share r of the tokens
costs T_recompute(r) = r * T_prefill; loading the cache costs
T_load = PerTokenKVSize * (context tokens) / Throughput(device); the controller
takes the r at which the two are equal and then the larger of that and the
quality floor r* = 15%.  The garbled formula on the page is read as that
quotient (bytes per token times tokens, over bytes per second).  A share above
100% is meaningless, so the result is capped at 1.

Parity: pinned by tests/test_oracle_loading.py against the pages' two worked
examples (tests/golden/loading_controller.json) and closed-form properties.
"""
from __future__ import annotations


def load_seconds(kv_bytes_per_token: float, n_tokens: float, load_bytes_per_s: float) -> float:
    """T_load: PerTokenKVSize x tokens / Throughput(device)."""
    return float(kv_bytes_per_token) * float(n_tokens) / float(load_bytes_per_s)


def loading_ratio(kv_bytes_per_token: float, n_tokens: float, load_bytes_per_s: float, prefill_seconds: float,
                  r_min: float = 0.15) -> float:
    """The controller's recompute share: max(r*, T_load / T_prefill), at most 1."""
    if prefill_seconds <= 0 or load_bytes_per_s <= 0:
        raise ValueError("prefill time and load bandwidth must be positive")
    r_match = load_seconds(kv_bytes_per_token, n_tokens, load_bytes_per_s) / float(prefill_seconds)
    return max(float(r_min), min(1.0, r_match))
