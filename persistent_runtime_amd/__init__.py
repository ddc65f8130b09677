"""MI355X-native decode-step megakernel: a persistent HIP kernel that runs one
transformer decode step from a host-built task list with HBM event counters.

Importing this package loads nothing; `persistent_runtime_amd.mk` loads the
compiled library (libmk.so) and raises if it is missing.
"""
__all__ = ["sol"]
