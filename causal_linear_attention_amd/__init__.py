"""Lightning Attention-2 tiled causal linear attention on MI355X (gfx950).

The HIP library is loaded on first use of the binding; ``inputs`` (seeded
synthetic workloads) imports without it.
"""
