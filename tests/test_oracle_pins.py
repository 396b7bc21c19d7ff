"""The CPU oracle against its pins (hand-worked cases, brute force, closed forms,
invariants, independent library routines).  See tests/pins.py."""
import pytest

import pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=[p.__name__ for p in pins.ALL_PINS])
def test_oracle_pin(oracle_lib, pin):
    fails = pin(oracle_lib)
    assert not fails, fails[:5]


def test_oracle_rejects_bad_k(oracle_lib):
    import numpy as np

    with pytest.raises(ValueError):
        oracle_lib.route(np.zeros((2, 4), np.float32), 5)


@pytest.mark.parametrize("name", ["tiny", "decode", "skewed"])
def test_oracle_properties_on_workloads(oracle_lib, name):
    """Selection/weight/map properties hold on the real workload inputs."""
    from moe_glue_amd import inputs as I

    cfg = I.CONFIGS[name]
    logits, bias = I.make_logits(cfg, 0)
    r = oracle_lib.route(logits, cfg.k, bias)
    assert not pins.check_route_properties(logits, cfg.k, bias, r)
    assert not pins.check_maps(r["topk_ids"], cfg.E, r)


def test_skewed_routing_is_skewed(oracle_lib):
    """The log-Zipf offsets send most rows to a few experts and the injected
    ties reach the selection boundary."""
    import numpy as np
    from moe_glue_amd import inputs as I

    cfg = I.CONFIGS["skewed"]
    logits, bias = I.make_logits(cfg, 0)
    r = oracle_lib.route(logits, cfg.k, bias)
    counts = np.sort(r["expert_counts"])[::-1]
    assert counts[:8].sum() > 0.5 * cfg.R
    assert (counts == 0).sum() >= 1 or counts[-1] < cfg.T // 100
    # every even-positioned tie row has an exact tie between the k-th and (k+1)-th keys
    rows = I.tie_rows(cfg, 0)
    assert len(rows) == 10
    for i, t in enumerate(rows):
        s = np.sort(logits[t])[::-1]
        if i % 2 == 0:
            assert s[cfg.k - 1] == s[cfg.k]
        else:
            assert s[0] == s[1]
