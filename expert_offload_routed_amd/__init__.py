"""Routed-expert MoE layer over a device-resident expert slot cache, for MI355X (gfx950).

The compute path is the C-ABI library ``libmoe_offload.so`` (hand-written HIP);
``expert_offload_routed_amd.binding`` is its thin ctypes binding. Importing the
package loads nothing; ``binding.lib()`` loads the library and raises if it has
not been built.
"""
