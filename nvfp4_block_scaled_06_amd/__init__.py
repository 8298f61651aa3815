"""MI355X-native NVFP4 dense-MoE router: runtime NVFP4 activation quantization,
block-scaled gate projection and the fused sigmoid/bias/top-k epilogue.

The compute lives in the HIP library ``libnvfp4_router.so`` (C ABI declared in
``include/nvfp4_router.h``); :mod:`.router` is the thin ctypes binding and
:mod:`.workloads` the seeded synthetic inputs. Importing the package loads
nothing; the binding loads the library on first use and fails loudly if it
is missing.
"""
