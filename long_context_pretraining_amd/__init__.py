"""MI355X-native Lighthouse Attention layer (forward and backward).

The compute lives in the HIP library built from csrc/ (see build.py); the
Python side is `lighthouse` (ctypes binding, same names as include/lighthouse.h)
and `inputs` (seeded synthetic tensors).
"""
