"""MI355X-native verify-and-resample step of speculative sampling.

The computation lives in libspecverify.so (HIP kernels for gfx950 behind a C ABI declared in
include/spec_verify.h); this package is its thin Python binding.
"""

from ._lib import (SpecVerifyError, expected_tokens, ops_factor, optimal_gamma,  # noqa: F401
                   release_workspaces, sample_summary, spec_acceptance_rate, spec_build_tree,
                   spec_philox_uniform, spec_sample, spec_verify, spec_verify_noalloc,
                   spec_verify_tree, status_string, walltime_speedup)

__all__ = ["spec_verify", "spec_verify_noalloc", "spec_sample", "spec_verify_tree",
           "spec_build_tree", "spec_philox_uniform", "spec_acceptance_rate", "expected_tokens",
           "walltime_speedup", "ops_factor", "optimal_gamma", "SpecVerifyError", "status_string",
           "sample_summary", "release_workspaces"]
