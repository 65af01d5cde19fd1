"""MI355X-native verify-and-resample step of speculative sampling.

The computation lives in libspecverify.so (HIP kernels for gfx950 behind a C ABI declared in
include/spec_verify.h); this package is its thin Python binding.
"""

from ._lib import (SpecVerifyError, spec_build_tree, spec_philox_uniform,  # noqa: F401
                   spec_sample, spec_verify, spec_verify_tree, status_string)

__all__ = ["spec_verify", "spec_sample", "spec_verify_tree", "spec_build_tree",
           "spec_philox_uniform", "SpecVerifyError", "status_string"]
