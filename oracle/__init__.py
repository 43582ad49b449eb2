"""CPU oracle for regularized direct (single-side-band) ptychography.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or run anything in this
package.  The HIP library never calls it, shares no code with it, and fails
loudly when its own extension is missing.

``dsp_oracle`` holds the plain FP64 definition of every hot-path result;
``simulate`` holds the physical forward models (first-order weak-object model
and a brute-force wave-optics simulation) that the oracle's own pins use.
"""
from . import dsp_oracle, simulate  # noqa: F401
