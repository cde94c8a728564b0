"""Affine-Q4 mixture-of-experts feed-forward for AMD MI355X (gfx950).

The compute path is the HIP library ``libq4moe.so`` behind a C ABI
(``include/q4moe.h``); :mod:`.binding` marshals torch tensors into it.
:mod:`.synth` draws the seeded synthetic inputs.  Importing this package does
not load the library; the first call into :mod:`.binding` does, and it raises
if the library is missing.
"""
