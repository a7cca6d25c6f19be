"""CPU oracle for the FlashLoop loop-attention hot path.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls or links
this package: only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline
leg of ``bench.py`` use it.  It shares no code with the HIP library or its
binding; the two meet only through the seeded inputs of ``workloads``.

The oracle is plain and slow on purpose: numpy, float64 for every attention
quantity, and the exact fp32 operation sequence for the quantizer so that codes
can be compared bit for bit.  Each function cites the passage of the FlashLoop
pages it follows (paperlayer.ai abstract page: "p1", with its section; the
flozi-tech guide: "guide", with its section or cell).

Modules
  quant      base (int8) and residual (4/2-bit) group quantizers, fp16 directed
             rounding, reconstruction chains
  records    byte layout of the packed base and residual records (pack/unpack)
  prefill    loop-1 dense attention, column mass, top-K, cached mass and reused
             part, sparse loop-r update; whole-slice driver
  decode     one decode step per loop over a packed cache
  brute      full-matrix bookkeeping form of the loop recurrences (tiny sizes)
  active     the next loop's active-token set (relative hidden-state change,
             top-k, nested)
  paper_format the paper's own cache format (INT4 asymmetric, group 64,
             per-channel keys, per-token values, bf16 tail)

Pins (see tests/test_oracle_*.py): brute-force code search, the half-step
reconstruction bound, special groups, a hand-worked packing example, a library
sort and exhaustive subset search for top-K, the textbook causal softmax (via
torch's CPU attention) when nothing is sparse or quantized, invariants of the
recurrences, the full-matrix brute force, decode == prefill row, and the byte
counts printed on the guide's Cell 1.  The paper-level quality claims (for
example 10% of columns recovering over 90% of the output, p1 §3.2) need trained
models and are parity unpinned.
"""
