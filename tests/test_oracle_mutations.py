"""Each planted mistake in the oracle (a dropped term, a wrong sign, index or operand) must
make at least one pin fail.  The mutants are separate builds of the same C file; the oracle
itself is built with no mutation.  CPU only."""
import pytest

import oracle
import pins

MUTATIONS = {
    1: "softmax without the extra zero logit",
    2: "stick-breaking keeps p instead of 1-p",
    3: "ties broken toward the higher chunk index",
    4: "causal limit admits the token's own chunk",
    5: "pooling drops the chunk's last row",
    6: "stick-breaking backward drops the later-slot term",
    7: "value gradient ignores the chunk weight",
    8: "selection-query gradient uses Qs instead of the chunk key",
    9: "query head mapped to group h % Hkv",
    10: "logit scale dropped",
    11: "softmax-weight backward drops the weighted mean of dw",
    12: "a NaN selection score is not ranked as -inf",
}


@pytest.mark.parametrize("m", sorted(MUTATIONS), ids=lambda m: MUTATIONS[m])
def test_mutation_is_caught(m):
    orc = oracle.build_mutant(m)
    caught = []
    for pin in pins.ALL_PINS:
        try:
            pin(orc)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"mutation {m} ({MUTATIONS[m]}) passed every pin"
