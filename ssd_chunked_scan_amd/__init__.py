"""MI355X-native chunked SSD (Mamba-2) forward pass.

``ssd_chunked_scan_amd.ssd`` is the binding to the HIP library (``libssd.so``,
built from ``csrc/``); ``ssd_chunked_scan_amd.workloads`` draws seeded inputs.
Importing the package itself loads nothing: the binding loads the library the
first time it is used and raises if it is missing.
"""

__all__ = ["ssd", "workloads"]
