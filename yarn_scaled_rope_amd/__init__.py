"""YaRN-scaled RoPE causal attention for AMD Instinct MI355X (gfx950).

The compute lives in ``libyarnattn.so`` (hand-written HIP kernels behind a C
ABI, declared in ``include/yarnattn.h``).  ``yarn_scaled_rope_amd.ops`` is a
thin ctypes binding with the same entry-point names; it loads the library on
first use and raises if it is missing.  ``workloads`` draws seeded synthetic
inputs and counts algorithmic work.
"""

from . import workloads  # noqa: F401

__all__ = ["workloads"]
