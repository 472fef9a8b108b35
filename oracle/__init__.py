"""Oracle for the vecset SDF decoder: TEST INFRASTRUCTURE ONLY.

A plain, slow CPU implementation (numpy, float64) of what the decoder and
its two accelerations compute, written from the pages:

* FlashVDM summary ("Unleashing Vecset Diffusion Model for Fast Shape
  Generation", aipaper.cc), section 3 (the vecset decoder cross-attends
  query points against the latent set to give an SDF value) and section 4.1
  (Lightning Vecset Decoder: Hierarchical Volume Decoding, Adaptive KV
  Selection, efficient decoder design);
* the techwalker article on FlashVDM, parts 2 and 5 (sign test between
  neighbouring voxels, truncated-SDF band, dilation; probe queries per
  sub-volume);
* the MSVS-VAE page (kwkr.cn), sections 1.1 and 3.3 (a local decoder: each
  query fuses the features of its K nearest supports with offset-dependent
  weights and a mean-pool residual).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package. The GPU library shares no code with it.

Modules:
  bf16     round-to-nearest-even emulation of bfloat16 (pinned against torch)
  decoder  grid coordinates, Fourier embedding, projections, attention, MLP,
           SDF head, analytic prior, full decode
  hvd      hierarchical volume decoding: cell test, dilation, child marking,
           nearest-ancestor fill, blocked-order lists, the level loop
  akvs     adaptive KV selection: corner probes, head-mean scores, top-k,
           union and cap
  brute    pure-Python loop versions of all of the above for tiny inputs
  surface  marching cubes at SDF = 0 on the decoded volume (the surface
           extraction stage that follows decoding)
  local    the local KNN decoder (AVS-Conv): float32 neighbour decision,
           offset MLP, weighted sum with mean residual, head

Parity status: every function is pinned by a CPU test (closed forms,
invariants, library routines or brute force on tiny inputs); see the
``tests/test_oracle_*.py`` files. Absolute decoder outputs on the synthetic
weights have no printed values on the pages; they are pinned through the
brute-force loops and the closed-form special cases.
"""

from . import bf16, decoder, hvd, akvs, brute, surface, local  # noqa: F401
