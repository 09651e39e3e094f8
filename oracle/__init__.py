"""CPU float64 oracle for the sparse-MLA writer and attention.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports this package:
only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg use it.
It shares no code with the HIP library (no kernels, headers, helpers, tables
or constants); both sides are fed from the seeded generators in `workloads`.

Modules:
  e4m3      - OCP E4M3 ("fn") encode (round to nearest even, saturate to
              finite) and decode, from the format definition.
  writer    - packing of a bf16 latent (+ RoPE) row into the 656-byte
              fp8_ds_mla row, dropping writes aimed at the reserved slot 0.
  attention - exact softmax attention over the valid top-k entries of the
              dequantised cache, and the faulty clamp-to-slot-0 reader that
              the pages describe (kept only as a negative control).
  merge     - log-sum-exp merge of partial (output, lse) results of disjoint
              shares of a row's top-k entries.
  gather    - listed cache rows dequantised into 576-wide bf16 rows.
  pages     - re-paging of touched 256-token pages into a 64-token scratch.
"""
from . import e4m3, writer, attention, merge, gather, pages  # noqa: F401
