"""Seeded synthetic inputs shared by the tests, the bench and the smoke check.

This package builds inputs only (random orthonormal factors, spectra, noise,
weights). It holds none of the Newton-Schulz or Muon arithmetic, and it imports
neither the oracle nor the HIP library.
"""
from .generators import *  # noqa: F401,F403
