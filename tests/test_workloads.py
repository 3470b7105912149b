"""The seeded input generators: deterministic, the stated shapes and the stated slopes."""
import numpy as np
import torch

import workloads


def test_inputs_are_deterministic_and_bf16_rounded():
    a = workloads.make_inputs(2, 3, 17, 64, "bf16", seed=5, with_dout=True)
    b = workloads.make_inputs(2, 3, 17, 64, "bf16", seed=5, with_dout=True)
    for nm in ("q", "k", "v", "dout"):
        assert a[nm].dtype == torch.bfloat16 and a[nm].shape == (2, 17, 3, 64)
        assert torch.equal(a[nm], b[nm])
    # bf16 values are the RNE rounding of the float32 draws in order q, k, v, dout
    g = torch.Generator().manual_seed(5)
    q32 = torch.randn((2, 17, 3, 64), generator=g)
    assert torch.equal(a["q"], q32.to(torch.bfloat16))


def test_alibi_slopes_formula():
    s = workloads.alibi_slopes(32)
    assert s.dtype == torch.float32
    assert abs(float(s[0]) - 2 ** -0.25) < 1e-7 and abs(float(s[31]) - 2 ** -8) < 1e-9


def test_workload_table():
    w = workloads.WORKLOADS
    assert (w[3].B, w[3].H, w[3].N, w[3].d, w[3].causal) == (4, 32, 8192, 128, True)
    assert w[5].window == (4096, 0) and w[5].alibi and w[5].backward
    assert w[1].dtype == "f32" and not w[1].causal


def test_row_sampling():
    r = workloads.sample_query_rows(4, 32, 8192, 256, seed=1003)
    assert r.shape == (256, 3) and len({tuple(x) for x in r}) == 256
    assert r[:, 0].max() < 4 and r[:, 1].max() < 32 and r[:, 2].max() < 8192
    kr = workloads.sample_key_rows(1, 32, 16384, 256, max_heads=4, seed=1005)
    assert len({(b, h) for b, h, _ in kr}) <= 4 and len(kr) == 256
    assert np.array_equal(r, workloads.sample_query_rows(4, 32, 8192, 256, seed=1003))
