"""Plain CPU oracle of the routed-expert MoE layer over a device-resident slot cache.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything in this
package. The product path (``expert_offload_routed_amd``) never does, and the
two share no code: only the seeded input generator
(``expert_offload_routed_amd.workloads``) feeds both.

Everything here is written from the definitions on the source pages, in
float64 unless a float decides an integer (expert selection, int8 activation
codes); those decisions are taken in float32, the precision of the kernels.
"""
from .moe_oracle import *  # noqa: F401,F403
