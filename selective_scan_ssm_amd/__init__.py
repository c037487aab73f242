"""MI355X (gfx950) selective scan: hand-written HIP kernels behind a C ABI
(include/ssm_scan.h, libssmscan.so) with thin torch wrappers.

    from selective_scan_ssm_amd import scan_fwd, sm1_scan_fwd, state_update

The wrappers are imported lazily so that `selective_scan_ssm_amd.inputs`
(seeded synthetic inputs) can be used without torch or the built library.
"""

__all__ = ["scan_fwd", "sm1_scan_fwd", "state_update"]


def __getattr__(name):
    if name in __all__:
        from . import ops
        return getattr(ops, name)
    raise AttributeError(name)
