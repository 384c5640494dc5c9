"""Plain fp64 CPU oracle for the Muon / MONA optimizer step.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import this
package: only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline``
leg of ``bench.py`` use it.  It shares no code, headers, tables or helpers with
the HIP implementation under ``newton_schulz_matrix_momentum_amd/``.
"""
from .muon_oracle import (  # noqa: F401
    CUBIC,
    QUINTIC,
    coefficient_table,
    restart_due,
    mona_acceleration,
    mona_lite_acceleration,
    round_bf16,
    momentum_update,
    frobenius_normalize,
    newton_schulz_direct,
    newton_schulz_gram,
    newton_schulz,
    limuon_orthogonalize,
    decoupled_update,
    muon_step_matrix,
    muon_step,
    adamw_step,
)
