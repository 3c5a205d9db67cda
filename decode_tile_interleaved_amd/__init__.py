"""Lattice-rANS weight compression with fused gfx950 tile decoding.

The C ABI (include/ep.h, libep.so) holds the whole path; ``ep`` is its thin
ctypes binding and ``workloads`` draws the seeded synthetic inputs.
"""
