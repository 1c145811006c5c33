"""sv_verify_noalloc, the entry point that allocates nothing (its workspace is
a fixed buffer inside the library, one per GPU): through the C ABI its
outputs equal sv_verify's on the same arguments, call after call, the second
call smaller than the first (the buffer keeps the first call's contents),
and a shape whose workspace exceeds the buffer is refused before launch."""
import ctypes
import sys

import numpy as np
import pytest

import parity as PT
from workloads import synth as I

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _noalloc(L, tgt, drf, tok, w, seed, out, n):
    import torch
    dt = 1 if w.is_bf16 else 0
    return L.sv_verify_noalloc(tgt.data_ptr(), drf.data_ptr(), tok.data_ptr(), w.B, w.gamma, w.V, dt,
                               ctypes.c_float(w.temperature), w.top_k, ctypes.c_float(w.top_p), seed, 0,
                               out.data_ptr(), n.data_ptr(), torch.cuda.current_stream().cuda_stream)


# each call smaller than the one before, across the dense, top-k and arg-max layouts
SEQUENCE = [("c4b", 512, 4101), ("c2", 8, 4102), ("c3", 32, 4103), ("g4b", 64, 4104), ("c1", 4, 4105)]


def test_noalloc_equals_sv_verify_call_after_call():
    import torch
    import rejection_sampling_verify_17_amd as S
    L = S.lib()
    for name, B, seed in SEQUENCE:
        w = I.make(name, B=B)
        dt = S.SV_BF16 if w.is_bf16 else S.SV_F32
        assert S.workspace_bytes(w.B, w.gamma, w.V, w.top_k, dt) <= S.NOALLOC_WORKSPACE_BYTES
        _say(f"case noalloc {name} B={w.B} gamma={w.gamma} V={w.V} T={w.temperature} K={w.top_k}")
        tgt, drf, tok = PT.to_device(w)
        out = torch.full((w.B, w.gamma + 1), -7, dtype=torch.int32, device="cuda")
        n = torch.full((w.B,), -7, dtype=torch.int32, device="cuda")
        assert _noalloc(L, tgt, drf, tok, w, seed, out, n) == S.SV_OK
        ref_out, ref_n = S.verify(tgt, drf, tok, w.temperature, w.top_k, seed=seed, top_p=w.top_p)
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy(), ref_out.cpu().numpy()), name
        assert np.array_equal(n.cpu().numpy(), ref_n.cpu().numpy()), name
        # and both meet the oracle bar
        rep = PT.compare(w, seed, PT.GpuResult(out.cpu().numpy(), n.cpu().numpy()), check_probs=False)
        _say(name, rep.summary())
        assert rep.ok() and rep.mismatches == 0


def test_noalloc_refuses_shapes_beyond_its_buffer():
    import torch
    import rejection_sampling_verify_17_amd as S
    L = S.lib()
    # top-k lists of K = 1024 at B = 256, gamma = 8: 256 * 16 * 1024 * 8 bytes > 32 MiB
    need = S.workspace_bytes(256, 8, 152064, 1024, S.SV_BF16)
    assert need > S.NOALLOC_WORKSPACE_BYTES
    x = torch.zeros(16, dtype=torch.int32, device="cuda")
    st = L.sv_verify_noalloc(x.data_ptr(), x.data_ptr(), x.data_ptr(), 256, 8, 152064, S.SV_BF16,
                             ctypes.c_float(0.8), 1024, ctypes.c_float(1.0), 1, 0, x.data_ptr(), x.data_ptr(),
                             torch.cuda.current_stream().cuda_stream)
    assert st == S.SV_EINVAL
