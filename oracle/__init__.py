"""Plain fp64 CPU oracle of PARK retrieval + block-sparse attention.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg
of ``bench.py`` may import it. It shares no code with the HIP library and imports nothing from it.

Source: "PARK: Accurate Block Retrieval for Sparse Attention in Video Diffusion Transformers"
(abstract on both PARK pages; Figure 1, Figure 2 caption and Tables 1, 4, 5 on the
thelatestinai.com page); the block sampling with inclusion-probability weighting follows the SIP
paragraph of the AB-Attention page. Each function names the passage it follows. Where the pages leave a step
open, the function states the reading it takes.

Parity status:
  * every step of the hot path is pinned by the ``-m "not gpu"`` tests (library routines,
    closed forms, brute force on tiny inputs, hand-worked fixtures under ``tests/golden``);
  * ``centered_log_mass_error`` is **parity unpinned**: the pages name the quantity (Figure 4) but
    do not define it.
"""
from .park import *  # noqa: F401,F403
from .park import __all__  # noqa: F401
