"""GPU: ionn_bias_grad_noalloc (the offset gradient for callers that cannot
allocate; its row-range sums live in the library's device scratch) against
ionn_bias_grad with a caller workspace, bit for bit, on two calls in a row
(the second with a smaller input, so stale scratch entries of the first
would show), and against the oracle's column sums."""
import numpy as np
import pytest
import torch

import oracle
from integer_only_nn_amd import ops
from gpu_helpers import dev, host, say, to_dev

pytestmark = pytest.mark.gpu


def _one(M, C, seed):
    rng = np.random.default_rng(seed)
    d = rng.integers(-128, 128, (M, C)).astype(np.int8)
    dd = to_dev(d)
    want = torch.empty(C, dtype=torch.int32, device=dev())
    ws = torch.empty(max(ops.ionn_bias_grad_workspace_bytes(M, C), 4), dtype=torch.uint8, device=dev())
    ops.ionn_bias_grad(dd, want, ws)
    got = torch.full((C,), -7, dtype=torch.int32, device=dev())
    ops.ionn_bias_grad_noalloc(dd, got)
    say("noalloc bias grad", M, C)
    np.testing.assert_array_equal(host(got), host(want), err_msg=f"M={M} C={C}")
    np.testing.assert_array_equal(host(got), oracle.bias_grad(d), err_msg=f"M={M} C={C} vs oracle")


def test_noalloc_matches_workspace_call_twice():
    # the workload's offset gradient (8192 error rows x 4096 channels), then
    # a smaller, ragged one on the one-column-per-lane path
    _one(8192, 4096, 1)
    _one(1000, 100, 2)


def test_noalloc_more_shapes():
    for M, C, seed in ((1, 16, 3), (65, 1040, 4), (401408 // 8, 64, 5), (3, 7, 6), (0, 33, 7)):
        if M == 0:
            got = torch.full((C,), 5, dtype=torch.int32, device=dev())
            ops.ionn_bias_grad_noalloc(torch.empty(0, C, dtype=torch.int8, device=dev()), got)
            assert (host(got) == 0).all()
        else:
            _one(M, C, seed)
