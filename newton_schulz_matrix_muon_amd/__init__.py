"""MI355X-native Newton-Schulz orthogonalization (standard and Gram) and the fused Muon step.

The compute lives in ``libmuon_ns.so`` (hand-written HIP for gfx950 behind a C ABI,
declared in ``include/muon_ns.h``). ``newton_schulz_matrix_muon_amd.ops`` is the thin
ctypes binding; importing this package does not load the library.
"""
__all__ = ["flops", "ops"]
