"""Q4_0-weight x Q8_0-activation quantized matrix product for MI355X (gfx950).

The work is done by hand-written HIP kernels in ``libq4bq.so`` (built from
``csrc/``) behind a C ABI declared in ``include/q4bq.h``; ``binding`` marshals
torch device tensors into that ABI.  The library is loaded on first use and a
missing or unloadable library raises -- there is no CPU fallback.
"""
