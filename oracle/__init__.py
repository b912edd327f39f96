"""Plain fp64 CPU oracle of the TurboQuant KV-cache path.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the package smoke check and
the CPU-baseline leg of the benchmark may import or run anything in this
directory.  The HIP library never calls it, never links it and shares no code
with it: the oracle has its own random-stream generator, rotation builder,
Lloyd-Max solver, bit packing, estimator and softmax.  Every step is written
out in float64 numpy (or plain Python) in the order the source pages give
it, with library primitives (a matrix product, a QR factorisation) used as
single steps and no blocking, fusion or reordering beyond that.

Sources cited in the docstrings (titles of the pages the method comes from):
  [Mobilint]  "TurboQuant explained: near-optimal KV cache compression and why
              the theory breaks down in practice", Mobilint blog.
  [cuTile]    function listing of DevTechJr/turboquant_cutile (codehub.bot).
  [tq-kv]     docs.rs page of the tq-kv crate.
  [ginkgoq]   "Limits And Assumptions", ginkgoq TurboQuant docs.

Parity status of each function (what pins it, other than itself) is listed in
the test module tests/test_oracle_pins.py.  The random-stream definition, the
bit layouts and the GQA/causal conventions are not fixed by the pages: those
readings are pinned only by hand-worked examples in tests/golden/ and are
marked "parity unpinned by the pages" where they are defined.
"""

from . import rng, transforms, codebook, codec, attention  # noqa: F401
