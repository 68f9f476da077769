"""The prefill tolerance is a bound on the kernel's rounding, checked on the
CPU: a model of that rounding (fp32 scores and exponentials, probabilities
rounded to bf16 for the value product, an fp32 normaliser of the unrounded
probabilities, bf16 output) stays within u * (A + |out|) of the fp64 oracle
row, A = the softmax-weighted mean of |V|, u = 2^-8, over random rows and
the stress value distributions; and the bound is not vacuous (the model's
error reaches a sizeable fraction of it)."""
import numpy as np
import pytest
import torch

import oracle.attention as att

U = 2.0 ** -8


def _bf16(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).float().numpy()


def _kernel_rounding_row(q, k, v, scale):
    """One query head: fp32 scores, bf16 probabilities in the product."""
    x = (k.astype(np.float32) @ q.astype(np.float32)) * np.float32(scale)
    p = np.exp(x - x.max()).astype(np.float32)
    num = (_bf16(p).astype(np.float64) @ v.astype(np.float64))
    return _bf16(num / np.float64(p.sum(dtype=np.float32)))


@pytest.mark.parametrize("qscale,kscale", [(1, 1), (64, 1), (512, 1), (512, 32)])
def test_rounding_model_stays_within_bound(qscale, kscale):
    rng = np.random.default_rng(qscale + kscale)
    d = 128
    worst = 0.0
    for n in (1, 2, 6, 33, 300, 2000):
        for _ in range(4):
            k = _bf16(rng.standard_normal((n, d)) / np.sqrt(d) * kscale)
            v = _bf16(rng.standard_normal((n, d)) / np.sqrt(d))
            q = _bf16(rng.standard_normal(d) / np.sqrt(d) * qscale)
            scale = 1 / np.sqrt(d)
            ref = att.dense_attention(q[None].astype(np.float64), k[:, None].astype(np.float64),
                                      v[:, None].astype(np.float64), scale)[0]
            A = att.dense_attention(q[None].astype(np.float64), k[:, None].astype(np.float64),
                                    np.abs(v[:, None]).astype(np.float64), scale)[0]
            got = _kernel_rounding_row(q, k, v, scale)
            ratio = np.abs(got - ref) / (U * (A + np.abs(ref)) + 1e-5 * A + 1e-7)
            worst = max(worst, float(ratio.max()))
    assert worst <= 1.0
    assert worst > 0.05  # the bound is within a small factor of what rounding does
