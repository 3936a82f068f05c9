"""The hyper-connection read on AMD Instinct MI355X (gfx950).

The compute lives in libhc.so (HIP kernels behind the C ABI of include/hc.h);
`binding` marshals torch tensors to it.  `workloads` draws the seeded synthetic
inputs.  Binding names are loaded on first use so that importing the package
does not need the built library.
"""
_BINDING_NAMES = ("hc_read", "hc_read_commit", "hc_read_bf16_lo", "hc_short_window_on", "hc_status_string", "hc_last_hip_error", "hc_dims",
                  "hc_timeouts", "hc_release", "read", "library", "HCError")

__all__ = list(_BINDING_NAMES)


def __getattr__(name):
    if name in _BINDING_NAMES:
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)
