"""CPU oracle for TurboQuant KV-cache compression and decode attention.

TEST INFRASTRUCTURE ONLY.  Only the test suite, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import this package.  The
product path (the HIP library and its Python binding) never imports, links or
executes anything here, and nothing here imports the product path.

Everything is plain numpy / scipy in float64, written step by step from what
the three source pages state (their titles are cited per function):

* "lightning-mlx plan.md" -- a feasibility study for TurboQuant at 256k
  context (memory arithmetic, bandwidth-bound decode, the three decompression
  steps: unpack + Lloyd-Max lookup, denormalise, inverse rotation).
* "omlx turboquant_kv.py" -- the continuous-batching TurboQuant KV cache
  (state types, packed width ceil(head_dim*bits/32), deterministic codec
  rebuild from (head_dim, bits, seed), K seed s and V seed s+1, append at the
  written end, causal mask for new tokens).
* "turboquant validate_moe_phase2.py" -- the synthetic validation of
  TurboQuantProd keys (MSE + 1-bit QJL) and group-quantised values at
  head_dim 256 (Tests 1-5 and the commit note).

Where the pages are silent the module docstrings state the reading taken.
Modules:

* :mod:`oracle.prng`      counter-based SplitMix64 + Box-Muller normals
* :mod:`oracle.codec`     rotation, Lloyd-Max codebook, QJL sketch
* :mod:`oracle.packing`   the packed index layout
* :mod:`oracle.quant`     MSE / Prod / group quantisers and dequantisers
* :mod:`oracle.attention` decode attention over a compressed cache
"""
