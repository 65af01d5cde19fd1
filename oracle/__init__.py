"""CPU oracle for speculative-sampling verification.

Test infrastructure only: imported by ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py``.  The product path never imports it.
"""
from .spec_verify_oracle import *  # noqa: F401,F403
