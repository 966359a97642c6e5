"""fp64 CPU oracle for weight-absorbed MLA / TPLA decode over a latent KV cache.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the test suite, the smoke check in
``__graft_entry__.py`` and the CPU-baseline leg of ``bench.py`` may import this
package.  The HIP library and its Python binding never import it, and it shares
no code with them (no helpers, constants or tables).  See ``tpla_oracle.py`` for
the definitions and their sources, and ``tests/test_oracle_pins.py`` for what
pins each function to something other than itself.
"""

from .tpla_oracle import (  # noqa: F401
    bf16_rne,
    hadamard,
    gather_sequence,
    latent_cache_append,
    tpla_decode_sharded,
    mla_decode_absorbed,
    mla_prefill_absorbed,
    mla_unabsorbed_bruteforce,
    value_up_projection,
    merge_context_parts,
    rms_normalize,
)
