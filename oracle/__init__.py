"""CPU oracle for one rank's ZeRO-1/2 optimizer step.

TEST INFRASTRUCTURE: imported only by tests/, the package smoke check and the
benchmark's CPU-baseline leg.  It shares no code with the HIP library.

Parity pins (all in tests marked "not gpu"):
  layout  - brute-force per-element ownership, single-bucket = plain
            reduce-scatter chunking, partition/alignment/cap invariants.
  step    - W=1 against torch.optim.AdamW / Adam (library), first-step closed
            form, beta1=beta2=0 closed form at every t, lr=0, float64
            evaluation of the same formula, reassembly of all ranks' shards
            against the full-array mean (all-reduce = reduce-scatter +
            all-gather).
  bf16    - against torch's float->bfloat16 conversion on every high half.
  pack    - brute-force per-element placement.
  accounting - the printed memory and fit tables of the pages.
"""
