"""Fused Mixture-of-Experts layer forward for AMD MI355X (gfx950).

The compute path is a HIP library with a C ABI (``include/moe.h``); this
package is its thin Python binding plus the seeded synthetic workloads.
"""
