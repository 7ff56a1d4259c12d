"""MI355X-native W8A8 quantized linear for quantized RL rollout (QuRL).

The compute path is the HIP library ``libqurl_w8a8.so`` (C ABI declared in
``include/qurl_w8a8.h``); ``w8a8_gemm_rl_amd.binding`` is a thin ctypes layer
over it. Submodules are imported on demand so that importing the package (for
example for the seeded inputs in ``w8a8_gemm_rl_amd.inputs``) neither loads the
shared library nor initialises a GPU.
"""

__all__ = ["binding", "inputs"]
