"""The workload presets against what the pages state about these networks
(tests/golden/page_facts.txt holds each fact with its source)."""
import math
import os

import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _facts():
    out = {}
    with open(os.path.join(GOLDEN, "page_facts.txt")) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                k, v, _src = [p.strip() for p in line.split(";")]
                out[k] = v
    return out


F = _facts()
WL = workloads.WORKLOADS


def _fc_params(layers):
    return sum(math.prod(s) for s in layers if len(s) == 2)


def test_param_counts():
    assert WL["tiny"].P == 29354
    assert WL["nin"].P == 7595176 and len(WL["nin"].layers) == 24
    assert WL["googlenet"].P == 6998552 and len(WL["googlenet"].layers) == 116
    assert WL["alexnet16"].P == WL["alexnet128_sparse"].P == 60965224


def test_nin_about_8x_fewer_params_than_alexnet():
    ratio = WL["alexnet16"].P / WL["nin"].P
    assert abs(ratio - float(F["nin_vs_alexnet_param_ratio"])) < 0.5


def test_alexnet_fc_bytes_exceed_150mb():
    assert _fc_params(WL["alexnet16"].layers) * int(F["bytes_per_weight"]) > int(F["alexnet_fc_bytes_min"])


def test_nin_has_no_fc_and_googlenet_fc_is_small():
    assert _fc_params(WL["nin"].layers) == int(F["nin_fc_layers"])
    g = _fc_params(WL["googlenet"].layers) * int(F["bytes_per_weight"])
    assert g < int(F["alexnet_fc_bytes_min"]) / 10


def test_googlenet_conv_count():
    convs = [s for s in WL["googlenet"].layers if len(s) == 4]
    assert len(convs) == 57
    chans = {s[0] for s in convs}
    assert min(chans) == 16 and max(chans) == 384


def test_tree_serial_steps():
    """2*log2(p) serialized steps for the binary tree at p = 128."""
    assert 2 * int(math.log2(128)) == int(F["tree_serial_steps_p128"])
