"""MI355X-native persistent megakernel for one MoE-transformer decode step.

The package is a thin Python layer over ``libmk.so`` (C ABI declared in
``include/mk.h``): ``mk`` holds the ctypes binding, ``synth`` the seeded
synthetic inputs, ``configs`` the model shapes and ``sol`` the closed-form
byte count used for speed-of-light figures. Importing the package loads
nothing; ``mk.load()`` opens the library (after torch, so both share one HIP
runtime).
"""
