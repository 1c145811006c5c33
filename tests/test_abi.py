"""The C ABI on the host (no GPU needed): the library loads, exports every
symbol the header declares, sizes workspaces, and rejects bad arguments with
SV_EINVAL before anything is enqueued."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "specverify.h")


@pytest.fixture(scope="module")
def L():
    import rejection_sampling_verify_17_amd as S
    return S.lib()


def declared_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"SV_API\s+[\w\s\*]+?\b(sv_\w+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_symbols()
    for required in ("sv_verify", "sv_workspace_bytes", "sv_verify_debug", "sv_status_string", "sv_draft_sample",
                     "sv_accept_histogram"):
        assert required in names


def test_library_exports_every_declared_symbol(L):
    for name in declared_symbols():
        assert hasattr(L, name), f"{name} declared in include/specverify.h but not exported"


def test_status_strings_and_version(L):
    import rejection_sampling_verify_17_amd as S
    assert S.status_string(0) == "ok"
    assert "invalid" in S.status_string(1)
    assert "gfx950" in S.version()


def test_workspace_bytes(L):
    import rejection_sampling_verify_17_amd as S
    assert S.workspace_bytes(0, 4, 256, 0, 0) == 0          # B < 1
    assert S.workspace_bytes(1, 0, 256, 0, 0) == 0          # gamma < 1
    assert S.workspace_bytes(1, 65, 256, 0, 0) == 0         # gamma > 64
    assert S.workspace_bytes(1, 4, 1, 0, 0) == 0            # V < 2
    assert S.workspace_bytes(1, 4, 256, 0, 7) == 0          # dtype
    a = S.workspace_bytes(64, 5, 128256, 0, 1)
    b = S.workspace_bytes(256, 8, 152064, 50, 1)
    assert a > 0 and b > 0 and a % 256 == 0 and b % 256 == 0
    # top-k lists: B * 2 gamma * K * 8 bytes at least
    assert b >= 256 * 16 * 50 * 8
    # top-k off when K <= 0 or K >= V
    assert S.workspace_bytes(8, 3, 32000, 0, 0) == S.workspace_bytes(8, 3, 32000, 32000, 0)
    # the arg-max mode's chunk keys fit: B * (gamma + 1) * 8 bytes at least
    assert S.workspace_bytes(4096, 64, 2, 50, 0) >= 4096 * 65 * 8


def test_launch_names(L):
    import rejection_sampling_verify_17_amd as S
    # top-p without top-k (or K > 1024) cuts every row by mass: the rows go
    # through the top-k path's windows
    assert S.launch_names(64, 5, 128256, 1, 0, 0.7, 0.9) == ["k_topk_step"] * 4    # [0,1) [1,3) [3,5)
    assert S.launch_names(64, 5, 128256, 1, 3000, 0.7, 0.9) == ["k_topk_step"] * 4
    assert S.launch_names(64, 5, 128256, 1, 0, 0.0, 0.9) == ["k_greedy_step"] * 4  # arg-max ignores top-p
    assert S.launch_names(64, 5, 128256, 1, 0, 0.7, 1.0) == ["k_rows", "k_rows"]
    # small inputs: statistics of every row, then the judgement (in every
    # block) and the sampling
    assert S.launch_names(64, 5, 128256, 1, 0) == ["k_rows", "k_rows"]
    # large inputs: statistics of position 0 and its judgement, then one launch
    # per further position (each judges its position in place) and one to sample
    assert S.launch_names(1024, 4, 50257, 0, 0) == ["k_rows", "k_judge"] + ["k_rows"] * 4
    # the top-k path: windows [0,1), [1,3), [3,7), ... of the sequences still
    # alive (one that would leave a single position over runs to gamma), then
    # the judgement of the last window and the draw
    assert S.launch_names(256, 8, 152064, 1, 50) == ["k_topk_step"] * 4   # [0,1) [1,3) [3,8)
    assert S.launch_names(16, 1, 152064, 1, 50) == ["k_topk_step"] * 2   # [0,1)
    assert S.launch_names(4, 3, 152064, 1, 300) == ["k_topk_step"] * 3   # [0,1) [1,3)
    assert S.launch_names(4, 4, 152064, 1, 300) == ["k_topk_step"] * 3   # [0,1) [1,4)
    assert S.launch_names(4, 5, 152064, 1, 300) == ["k_topk_step"] * 4   # [0,1) [1,3) [3,5)
    # [0,1) [1,3) [3,7) [7,15) [15,31) [31,64)
    assert S.launch_names(2, 64, 2048, 0, 16) == ["k_topk_step"] * 7
    # the arg-max mode (T = 0): the same windows over target rows 0..gamma
    # ([0,1), [1,3), [3,5) at gamma = 4), then the judgement of the last
    # window; top-k changes nothing
    assert S.launch_names(1024, 4, 50257, 0, 0, 0.0) == ["k_greedy_step"] * 4
    assert S.launch_names(1024, 4, 50257, 0, 50, 0.0) == ["k_greedy_step"] * 4
    # [0,1) [1,3) [3,7) [7,15) [15,31) [31,63) [63,65)
    assert S.launch_names(3, 64, 100, 1, 0, 0.0) == ["k_greedy_step"] * 8
    assert S.launch_names(3, 1, 100, 1, 0, 0.0) == ["k_greedy_step"] * 3


def _call(L, **over):
    """sv_verify with fake, well-aligned device addresses; some argument is
    always invalid so nothing is ever launched."""
    args = dict(target=0x100000, draft=0x200000, tokens=0x300000, B=4, gamma=3, V=1000, dtype=0,
                T=1.0, K=0, P=1.0, seed=1, off=0, out=0x400000, n=0x500000, ws=0x600000, wsb=1 << 30, stream=None)
    args.update(over)
    return L.sv_verify(args["target"], args["draft"], args["tokens"], args["B"], args["gamma"], args["V"],
                       args["dtype"], args["T"], args["K"], args["P"], args["seed"], args["off"], args["out"],
                       args["n"], args["ws"], args["wsb"], args["stream"])


@pytest.mark.parametrize("over", [
    dict(target=None), dict(draft=None), dict(tokens=None), dict(out=None), dict(n=None), dict(ws=None),
    dict(B=0), dict(B=-3), dict(gamma=0), dict(gamma=65), dict(V=1), dict(V=(1 << 28) + 1),
    dict(dtype=2), dict(T=-1e-30), dict(T=-1.0), dict(T=float("nan")), dict(T=float("inf")),
    dict(wsb=16), dict(target=0x100002), dict(dtype=1, draft=0x200001), dict(tokens=0x300002),
    dict(ws=0x600010), dict(P=float("nan")),
    dict(P=0.9, K=50, ws=None),
    # grids that would not fit 32 bits: top-k (B * 2 gamma blocks), arg-max
    # (B * (gamma + 1) * chunks); the workspace size is made to pass
    dict(B=1 << 25, gamma=64, K=50, wsb=1 << 62), dict(B=1 << 25, gamma=64, T=0.0, wsb=1 << 62),
], ids=lambda d: ",".join(f"{k}={v}" for k, v in d.items()))
def test_invalid_arguments_rejected_before_launch(L, over):
    assert _call(L, **over) == 1  # SV_EINVAL


def test_product_path_does_not_touch_the_oracle():
    """The package never imports or loads the oracle."""
    pkg = os.path.join(ROOT, "rejection_sampling_verify_17_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f)).read()
                for needle in ("from oracle", "import oracle", "sv_oracle", "svo_"):
                    assert needle not in text, f"{f} mentions {needle}"


@pytest.mark.parametrize("over", [
    dict(draft=None), dict(out=None), dict(B=0), dict(gamma=0), dict(gamma=65), dict(V=1), dict(dtype=3),
    dict(T=-1.0), dict(T=float("nan")), dict(T=float("inf")), dict(draft=0x200002), dict(out=0x400002),
    dict(dtype=1, draft=0x200001), dict(P=float("nan")),
], ids=lambda d: ",".join(f"{k}={v}" for k, v in d.items()))
def test_draft_sample_invalid_arguments(L, over):
    args = dict(draft=0x200000, B=4, gamma=3, V=1000, dtype=0, T=1.0, K=0, P=1.0, seed=1, off=0, out=0x400000,
                stream=None)
    args.update(over)
    assert L.sv_draft_sample(args["draft"], args["B"], args["gamma"], args["V"], args["dtype"], args["T"],
                             args["K"], args["P"], args["seed"], args["off"], args["out"], args["stream"]) == 1


@pytest.mark.parametrize("over", [dict(n=None), dict(h=None), dict(B=0), dict(gamma=0), dict(gamma=65),
                                  dict(n=0x100002), dict(h=0x200002)],
                         ids=lambda d: ",".join(f"{k}={v}" for k, v in d.items()))
def test_accept_histogram_invalid_arguments(L, over):
    args = dict(n=0x100000, B=8, gamma=4, h=0x200000, stream=None)
    args.update(over)
    assert L.sv_accept_histogram(args["n"], args["B"], args["gamma"], args["h"], args["stream"]) == 1
