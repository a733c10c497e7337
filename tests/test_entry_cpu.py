"""The code comparison that smoke() runs on the GPU's quantizer output,
exercised on the CPU with the oracle's output on both sides."""
import numpy as np
import pytest

import __graft_entry__ as entry
import oracle
import testkit


def test_smoke_code_comparison():
    cfg = testkit.CONFIGS[1]
    q, k, v = testkit.make_inputs(cfg, Nq=300, Nkv=300)
    want = oracle.quantize(q, k, v)
    got = {n: (x.copy() if isinstance(x, np.ndarray) else x) for n, x in want.items()}
    entry.assert_codes_equal(got, want)
    got["k8"].reshape(-1)[7] ^= 1
    with pytest.raises(AssertionError, match="k8"):
        entry.assert_codes_equal(got, want)
    got["k8"].reshape(-1)[7] ^= 1
    got["qk_format"] = "fp8"
    with pytest.raises(AssertionError, match="qk_format"):
        entry.assert_codes_equal(got, want)
