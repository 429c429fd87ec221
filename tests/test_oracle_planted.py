"""Each plausible mistake planted in a copy of the oracle is caught by a pin.

The planted copies are built from the oracle's own source with -DORA_PLANT=n
(see the comment at ORA_PLANT in oracle/kvq_oracle.c); the oracle proper is
built with 0.  A mistake that no pin caught would mean the pins cannot tell a
wrong oracle from the right one.
"""
import pytest

import oracle
import oracle_pins

PLANTS = {
    1: "boosted channels quantized with 2 bits",
    2: "ties in the channel ranking go to the higher channel",
    3: "hi and lo planes swapped",
    4: "Value zero point dropped on dequantization",
    5: "codes truncated instead of rounded",
    6: "Key metadata read from the wrong token group",
    7: "query heads mapped to KV heads with a stride",
    8: "softmax scale dropped",
    9: "newest residual token dropped",
    10: "channels ranked by minimum magnitude",
    11: "Value groups taken along tokens",
    13: "scale divided by L + 1",
    14: "query-aware score ignores the relevance",
    15: "query-aware difficulty = largest group range instead of their sum",
    16: "relevance = largest |q| of the group's heads instead of the sum",
    17: "prefill attention without the causal mask",
    18: "cumulative scores summed before the softmax normalization",
    19: "token selection ties to the higher position",
    20: "recent window one position short",
    21: "prefill rows without the diagonal key",
    22: "batched quantizer ignores the level count",
}


@pytest.mark.parametrize("n", sorted(PLANTS), ids=lambda n: f"plant{n}")
def test_planted_mistake_is_caught(n):
    lib = oracle.planted(n)
    caught = []
    for pin in oracle_pins.PINS:
        try:
            pin(lib)
        except AssertionError:
            caught.append(pin.__name__)
            break
    assert caught, f"no pin caught planted mistake {n}: {PLANTS[n]}"
