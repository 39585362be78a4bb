"""The seeded inputs of the measured workloads are fixed: every generated
array must hash to the SHA-256 recorded in tests/golden/input_manifest.json
(written by tests/golden/make_input_manifest.py from the generators alone).
A silent change to a generator, a seed or a reading of the input recipe would
otherwise move every float parity result and benchmark number unnoticed."""
import json
import os

import pytest

from tests.golden.make_input_manifest import OUT, workload_digests
from workloads import ALL

MANIFEST = json.load(open(OUT))


def test_manifest_covers_every_workload():
    assert sorted(MANIFEST) == sorted(ALL)


@pytest.mark.slow
@pytest.mark.parametrize("name", sorted(ALL))
def test_generated_inputs_match_the_manifest(name):
    assert workload_digests(name) == MANIFEST[name]
