"""Kamera KV reuse operator for AMD MI355X (gfx950): HIP kernels behind a C ABI.

    binding    ctypes binding of libkamera.so (include/kamera.h), same function names
    workloads  seeded synthetic inputs shaped like the GQA / MLA / MHA backbones
    build      hipcc build of libkamera.so

The operator (technical summary of "Kamera: Unified Position-Invariant Multimodal KV Cache for
Training-Free Reuse", §2): KV^(B|A) = R(delta) KV(B|empty) + U_m V_m^T, written through a
page table into a KV cache.
"""
