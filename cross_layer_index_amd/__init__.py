"""IndexCache sparse attention on MI355X (gfx950).

The compute path is the C-ABI library ``libic.so`` built from ``csrc/``;
``cross_layer_index_amd.ic`` binds it. Importing this package does not load the
library, so the input generator (``workloads``) is usable on machines without
a GPU.
"""
__all__ = ["workloads", "ic"]
