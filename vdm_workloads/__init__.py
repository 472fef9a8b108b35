"""Seeded synthetic inputs for the vecset SDF decoder.

This module builds *data*: decoder weights, latent vecsets, analytic shape
primitives and query point sets, for the five workloads (tiny fp32 dense,
dense 129^3 grid, hierarchical 75->150->300, hierarchical with KV
selection, 40,960-token x 200K-query dense) and for the local KNN decoder
(AVS-Conv of the MSVS-VAE page) at that 200K x 40,960 shape. It holds none of the decoder's
arithmetic: no embedding of queries, no projection, no attention, no MLP,
no SDF evaluation and no voxel selection. Both the oracle (``oracle/``) and
the GPU path consume what it returns; neither is imported here.

The pages (FlashVDM summary, "Unleashing Vecset Diffusion Model for Fast
Shape Generation", sections 4.1 and 6) evaluate on Hunyuan3D-2
reconstructions and a 200K-query batch (MSVS-VAE page, section 3.3); those
datasets and trained weights are not available, so these seeded synthetic
inputs stand in for them with the same shapes and sizes.
"""

from .gen import (  # noqa: F401
    Workload,
    Prim,
    make,
    CONFIG_NAMES,
    round_bf16_values,
    with_unseen_key,
    make_local,
    small_local,
    LocalWorkload,
)
