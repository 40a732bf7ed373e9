"""MI355X-native joint prefix/suffix attention for diffusion transformers.

The product is the C-ABI library libjpa (include/jpa.h) built from csrc/ for
gfx950; ``jpa`` is its Python binding.
"""

from .jpa import (  # noqa: F401
    JpaArgumentError,
    JpaError,
    jpa_abi_version,
    jpa_forward,
    jpa_plan,
    jpa_status_str,
    jpa_validate,
    library_path,
    load_library,
)
