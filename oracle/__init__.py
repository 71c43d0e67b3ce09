"""The oracle: plain fp64 CPU reference of the Mamba-2 mixer hot path.

TEST INFRASTRUCTURE ONLY -- imported by ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py``; never by the library.  The
arithmetic lives in ``ssd_oracle.c`` (plain C, fp64, token by token); this
module only marshals numpy arrays into it.

Parity pins (see ``tests/test_oracle_pins.py``): brute-force semiseparable
form, the d_state=1 closed form, ``torch.nn.functional.conv1d``, and the
invariants dt=0, reset, prefill-then-decode, split prefill, group
equivalence, linearity and zero-B/C.  The packed-batch (varlen) and
state-pool forms run those routines per sequence; their indexing is pinned by
``tests/test_oracle_varlen.py``.
"""
from .oracle import Oracle, load  # noqa: F401
