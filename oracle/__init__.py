"""CPU oracle for the KLA forward path (float64).

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import, call, link or execute anything
under ``oracle/``. The library ``delta_rule_recurrence_kla_amd`` never touches
it, and the two share no code.

  kla_ref.py   plain NumPy token-by-token recurrence (the definition)
  kla_ref.c    the same recurrence in plain C, OpenMP over heads
  psd_lift.py  the rank-one PSD lift psi(u) = vec(u u^T) of queries and keys
               (features rounded to bf16) in front of kla_ref.forward
  loglinear.py log-linear KLA: Fenwick-bucketed states with per-level output weights,
               as a token-pair definition and as the recurrent (bucket-merge) form
  kla_bwd.py   reverse-mode gradients of the token loop (dq, dk, dv, dlog_alpha, deta, dS0)
               for a loss with given dO and dS_T
  cref.py      ctypes loader for the C build
  build.py     gcc build of kla_ref.c into oracle/libkla_ref.so
"""
from . import kla_ref  # noqa: F401
from . import psd_lift  # noqa: F401
from . import loglinear  # noqa: F401
from . import kla_bwd  # noqa: F401
