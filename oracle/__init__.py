"""Float64 CPU oracles of the KDA forward recurrence.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import, call, link or run anything
under ``oracle/``. The library (gated_delta_rule_channel_amd) never does and
shares no code with it.

* ``kda_oracle`` -- numpy, token by token (the definition written out);
* ``native``     -- the same definition in plain C with OpenMP, for the
                    workloads too large for numpy;
* ``chunked_mirror`` -- a float64 numpy evaluation of the chunkwise (UT/WY)
                    form, used only to pin that the chunk algebra reaches the
                    token-by-token result.
"""
from .kda_oracle import kda_decode, kda_forward, kda_step  # noqa: F401
