"""Host-side rules of the library that fix results, checked on the CPU
against their statement in the oracle: the default FP32 reduction order of
the DFP contractions is a function of the shape alone (reading U35), so the
library's choice must equal the oracle's rule on every shape."""
import itertools

import pytest

import oracle
from integer_only_nn_amd import ops

ROLES = {"fwd": 0, "dgrad": 1, "wgrad": 2}


def test_default_fp32_split_rule_matches_oracle():
    dims = (1, 63, 64, 65, 127, 128, 129, 256, 511, 1000, 1024, 4096, 25088)
    for (M, K, N), role in itertools.product(itertools.product(dims, repeat=3), ROLES):
        assert ops.dfp16_f32_splits(M, K, N, ROLES[role]) == oracle.dfp16_default_splits(M, K, N, role), \
            (M, K, N, role)
