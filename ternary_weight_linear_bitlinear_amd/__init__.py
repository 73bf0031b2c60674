"""MI355X-native BitNet b1.58 BitLinear forward pass (HIP kernels for gfx950).

The compute path lives in ``libbitlinear.so`` (C ABI: include/bitlinear.h);
``bitlinear`` is its thin torch binding. ``synth`` builds seeded synthetic
inputs. Importing ``bitlinear`` requires the built library (there is no
fallback).
"""
