"""The binding rejects tensors whose shape or dtype the C ABI would misread (CPU only: the checks
run before any device pointer is taken)."""
import re

import pytest
import torch

from lossless_speculative_sampling_amd import capi


def _inputs(B=3, K=2, V=64, dt=torch.int16):
    return (torch.zeros((B, K, V), dtype=dt), torch.zeros((B, K + 1, V), dtype=dt),
            torch.zeros((B, 3), dtype=torch.int32), torch.zeros((B, K), dtype=torch.int32))


@pytest.mark.parametrize("case,msg", [
    ("target_rows", "K + 1"),
    ("dtype_mismatch", "same dtype"),
    ("draft_vocab", "does not match"),
    ("tokens_dtype", "tokens must be int32"),
    ("tokens_shape", "tokens must have shape"),
    ("params_shape", "params must have shape"),
    ("no_draft", "draft logits are required"),
])
def test_spec_verify_argument_checks(case, msg):
    d, t, p, tok = _inputs()
    K = 2
    if case == "target_rows":
        t = torch.zeros((3, K + 2, 64), dtype=torch.int16)
    elif case == "dtype_mismatch":
        d = torch.zeros((3, K, 64), dtype=torch.float32)
    elif case == "draft_vocab":
        d = torch.zeros((3, K, 63), dtype=torch.int16)
    elif case == "tokens_dtype":
        tok = tok.to(torch.int64)
    elif case == "tokens_shape":
        tok = torch.zeros((3, K + 1), dtype=torch.int32)
    elif case == "params_shape":
        p = torch.zeros((2, 3), dtype=torch.int32)
    elif case == "no_draft":
        d = None
    with pytest.raises(ValueError, match=re.escape(msg)):
        capi.spec_verify(d, t, K, p, tok)


def test_verify_cache_needs_the_cache_row():
    d, t, p, tok = _inputs()
    with pytest.raises(ValueError, match="rows"):
        capi.saguaro_verify_cache(d, t, 2, p, tok, 8, 0.7, 1.0)


def test_cache_lookup_checks_the_fanout_and_shapes():
    cache = torch.zeros((4, 10), dtype=torch.int32)
    k = torch.zeros(4, dtype=torch.int32)
    with pytest.raises(ValueError, match="fan-out entries"):
        capi.saguaro_cache_lookup(0, cache, [3, 3], 3, 4, k, k)
    with pytest.raises(ValueError, match="fan-out needs"):
        capi.saguaro_cache_lookup(0, cache, [3, 3, 3, 3], 3, 4, k, k)
    with pytest.raises(ValueError, match="kappa"):
        capi.saguaro_cache_lookup(1, cache, [2, 5, 1], 0, 4, k, k)
    with pytest.raises(ValueError, match="tstar"):
        capi.saguaro_cache_lookup(0, cache, [3, 3, 3, 1], 3, 4, k, k.to(torch.int64))
    # branch mode: k and t* per chain (kappa per request), branches B * kappa * gamma
    br = torch.zeros((8, 5), dtype=torch.int32)
    with pytest.raises(ValueError, match="k must hold 8"):
        capi.saguaro_cache_lookup(1, br, [2, 5], 0, 4, k, k)
