"""ReplaySSM decode hot path for MI355X (gfx950).

The compute lives in ``libreplayssm.so`` -- hand-written HIP kernels behind a
C ABI declared in ``include/replayssm.h``.  ``hybrid_model_ssm_amd.replayssm``
is the thin ctypes binding (argument marshalling only; PyTorch supplies device
memory and streams).  ``hybrid_model_ssm_amd.synth`` draws the seeded
synthetic inputs.  Nothing here imports the CPU oracle.

Importing this package loads nothing; the library is loaded on first use and
a missing build raises ``ReplaySSMLibraryMissing``.
"""

__all__ = ["replayssm", "synth", "build"]
