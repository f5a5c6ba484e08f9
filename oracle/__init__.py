"""CPU fp64 oracle for Newton-Schulz orthogonalization and the Muon step.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package. The HIP library and
its Python binding never import, call or link anything here, and nothing here
imports them.
"""
from .ns import (  # noqa: F401
    QUINTIC,
    CUBIC,
    default_coeffs,
    orient,
    frobenius_normalize,
    ns_standard,
    ns_gram,
    ns_svd_closed_form,
    ns_closed_form_entries,
    scalar_ns_map,
    muon_step,
)
from .adamw import adamw_step  # noqa: F401
