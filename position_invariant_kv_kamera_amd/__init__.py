"""Kamera KV reuse operator for AMD MI355X (gfx950): HIP kernels behind a C ABI.

``workloads`` draws seeded synthetic inputs; the binding to ``libkamera.so`` is added by the
GPU path.
"""
