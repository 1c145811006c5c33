"""The device arithmetic the kernels rely on, against fp64 host references.

* The exponential variate of the samplers, -log2(U) for every one of the 2^23
  possible U = (2k + 1) 2^-24 (Philox word k << 9), is within 1 ulp: near
  ties of the Gumbel keys the GPU's winner then differs from the oracle's only
  where the keys lie within rounding, which the parity bar exempts.
* The native exp2 used for the softmax statistics is within 1 ulp over the
  range its arguments take (z c - R from the fp32 normal limit up to 64: the
  reference R may lie up to 64 below a row's largest z c) on a dense sample
  of fp32 inputs, and underflows to [0, 2^-126] below it.
* The native log2 the bonus keys apply to those variates stays within 2 ulp
  of the result, or 2^-22 absolute where the result is near 0.
"""
import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _ulp(x):
    """Spacing of fp32 at |x| (fp64 values), floored at the smallest normal's spacing."""
    e = np.floor(np.log2(np.maximum(np.abs(x), 2.0 ** -126)))
    return np.exp2(e - 23)


def _run(fn, *args):
    import torch
    import rejection_sampling_verify_17_amd as S
    st = fn(*args, torch.cuda.current_stream().cuda_stream)
    assert st == S.SV_OK
    torch.cuda.synchronize()


def test_exponential_variate_every_U():
    import torch
    import rejection_sampling_verify_17_amd as S
    n = 1 << 23
    out = torch.empty(n, dtype=torch.float32, device="cuda")
    _run(S.lib().sv_probe_variates, 0, n, out.data_ptr())
    got = out.cpu().numpy().astype(np.float64)
    U = (2.0 * np.arange(n, dtype=np.float64) + 1.0) * 2.0 ** -24
    ref = -np.log2(U)
    err = np.abs(got - ref) / _ulp(ref)
    worst = int(np.argmax(err))
    _say(f"-log2(U) over all 2^23 U: max {err[worst]:.3f} ulp at U = {U[worst]!r}; "
         f"mean {err.mean():.3f} ulp; U -> 1: {got[-1]!r} vs {ref[-1]!r}")
    assert np.all(got > 0.0)
    assert err.max() <= 1.0


def test_native_exp2_on_statistics_range():
    import torch
    import rejection_sampling_verify_17_amd as S
    # every 64th fp32 bit pattern from -0 down to -150 and from +0 up to 64
    # (the arguments of the statistics are z c - R <= 64)
    lo, hi = np.float32(-0.0).view(np.uint32), np.float32(-150.0).view(np.uint32)
    neg = np.arange(lo, hi, 64, dtype=np.uint64).astype(np.uint32)
    pos = np.arange(np.float32(0.0).view(np.uint32), np.float32(64.0).view(np.uint32) + 1, 64,
                    dtype=np.uint64).astype(np.uint32)
    bits = np.concatenate([neg, pos])
    x = bits.view(np.float32)
    xt = torch.from_numpy(x).cuda()
    out = torch.empty_like(xt)
    _run(S.lib().sv_probe_math, xt.data_ptr(), x.size, 0, out.data_ptr())
    got = out.cpu().numpy().astype(np.float64)
    ref = np.exp2(x.astype(np.float64))
    normal = x >= -126.0
    err = np.abs(got[normal] - ref[normal]) / _ulp(ref[normal])
    _say(f"exp2 on {normal.sum()} inputs in [-126, 64]: max {err.max():.3f} ulp, mean {err.mean():.3f}")
    assert err.max() <= 1.0
    tail = got[~normal]
    assert np.all(tail >= 0.0) and np.all(tail <= 2.0 ** -126)


def test_native_log2_of_the_variates():
    import torch
    import rejection_sampling_verify_17_amd as S
    n = 1 << 23
    e2 = torch.empty(n, dtype=torch.float32, device="cuda")
    _run(S.lib().sv_probe_variates, 0, n, e2.data_ptr())
    out = torch.empty_like(e2)
    _run(S.lib().sv_probe_math, e2.data_ptr(), n, 1, out.data_ptr())
    x = e2.cpu().numpy().astype(np.float64)
    got = out.cpu().numpy().astype(np.float64)
    ref = np.log2(x)
    aerr = np.abs(got - ref)
    uerr = aerr / _ulp(ref)
    near0 = np.abs(ref) < 2.0 ** -6
    _say(f"log2 of the 2^23 variates: max {uerr[~near0].max():.3f} ulp away from 0, "
         f"max abs {aerr[near0].max() if near0.any() else 0.0:.3e} near 0")
    assert uerr[~near0].max() <= 2.0
    if near0.any():
        assert aerr[near0].max() <= 2.0 ** -22
