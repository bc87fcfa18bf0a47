"""Skip selectors: the page examples (tests/golden/selector_examples.txt, vLLM-Omni
"Quantized KV Cache", "Parameters"/"Configuration") and the readings for the cases the
page leaves open."""
import os

import pytest

from fp8_dynamic_scaled_amd import parse_selector, skip_fp8
from workloads import WORKLOADS, dit_schedule

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "selector_examples.txt")


def test_page_examples():
    n = 0
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        spec, want = [x.strip() for x in line.split("|")]
        assert parse_selector(spec) == {int(x) for x in want.split()}
        n += 1
    assert n == 4


@pytest.mark.parametrize("spec,want", [(None, set()), ("", set()), ("  ", set()),
                                       (" 3 , 5-6 ", {3, 5, 6}), ("7-7", {7}), ("2,2", {2})])
def test_readings(spec, want):
    assert parse_selector(spec) == want


@pytest.mark.parametrize("spec", ["1,,2", "3-1", "-1", "a", "1-", "1-2-3", "1.5", "0x3"])
def test_malformed(spec):
    with pytest.raises(ValueError):
        parse_selector(spec)


def test_dit_workload_routing():
    w = WORKLOADS["dit"]
    steps, layers = parse_selector(w.skip_steps), parse_selector(w.skip_layers)
    sched = dit_schedule(w, steps, layers)
    assert len(sched) == 32
    bf16 = [s for s in sched if s[3]]
    fp8 = [s for s in sched if not s[3]]
    assert len(bf16) == 22 and len(fp8) == 10
    assert all(st >= 2 and ly >= 3 for (_, st, ly, _) in fp8)
    assert skip_fp8(0, 7, steps, layers) and skip_fp8(3, 2, steps, layers)
    assert not skip_fp8(2, 3, steps, layers)
