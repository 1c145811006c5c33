"""specverify: batched speculative-sampling verification on one MI355X.

The C ABI (include/specverify.h) is implemented by libspecverify.so, built
from csrc/ with hipcc for gfx950; this package is its thin torch binding
(`verify`, `verify_debug`, `verify_timed`, `draft_sample`,
`accept_histogram`).  Seeded synthetic workloads for tests and the benchmark
live outside the package, in `workloads/synth.py`.
"""
from ._binding import (NOALLOC_WORKSPACE_BYTES, SV_BF16, SV_EHIP, SV_EINVAL, SV_F32, SV_OK, SpecVerifyError, accept_histogram,
                       draft_sample, launch_names, lib, status_string, verify, verify_debug, verify_noalloc, verify_timed,
                       version,
                       workspace_bytes)

__all__ = ["verify", "verify_noalloc", "verify_debug", "verify_timed", "draft_sample", "accept_histogram", "workspace_bytes", "launch_names", "lib", "version",
           "status_string", "SpecVerifyError", "SV_F32", "SV_BF16", "SV_OK", "SV_EINVAL", "SV_EHIP"]
