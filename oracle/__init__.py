"""CPU oracle for the paged KV-cache hot path.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import or run anything in this
package.  The product path (the HIP library and its Python binding) never
imports it, and this package never imports the product path.

``ref``   numpy fp64 definitions of the three operations (store, decode,
          varlen causal prefill over the cache) and of the split-K partials
          and merge, plus varlen causal prefill over contiguous k/v.
``brute`` pure-Python loop versions of decode, prefill and contiguous
          prefill for tiny inputs, written independently of ``ref`` to pin
          it.
``prefix_plan`` the shared-prefix decode plan (which sequences' leading
          splits are computed once for a group), in plain Python.
``block_manager`` the host block manager's allocation algorithms.

Parity status: every function here is pinned by CPU tests (brute force,
library SDPA on contiguous tensors, closed forms, invariants and the worked
address-translation example printed on the pages); none is "parity unpinned".
"""
