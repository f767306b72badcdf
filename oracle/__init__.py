"""Float64 CPU oracle for multi-row speculative-verification decode attention.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute anything in this package: only the tests, the smoke check and the
benchmark's CPU-baseline leg use it.  It shares no code, table or helper with
the HIP library and imports neither it nor its Python binding.

Where it comes from (the three pages on the subject):

* IQuestRT technical report, section "Read only the KV tiles needed by the
  current positions": eight query rows times the six query heads that share
  one KV head; the read is bounded by the current query positions with a
  causal mask at the boundary; a learned attention sink with zero value adds
  only to the softmax denominator; the work is split along the sequence and a
  separate combine merges the splits; sliding-window layers keep a ring of the
  4,096-position window plus one 64-slot tile, and the rows written before the
  read never evict history an earlier row needs.
* IQuestRT report, section "Expose more parallelism in attention": the split
  partials are merged through their log-sum-exp values and the combine applies
  the sink.
* IQuestRT report, section "Let correctness checks change the design": the
  ring state is checked with independent position labels and visible-position
  sets.
* "Qwen3.8-27B on one RTX 4090", section "More tokens per round: verify
  trees": a 16-node draft tree verified in one pass under a tree mask; section
  "A cheaper cache and state": FP8 keys after a Hadamard rotation, INT8 values.

Modules:
  masks   -- visibility sets, tree ancestry, union extent, split rule, ring replay
  attn    -- the definition (brute force), the split form and the LSE combine
  codec   -- e4m3fn bit-field decode / saturating RNE encode, Sylvester WHT,
             int8 values with a per-(token, head) scale

Parity status: every function here is pinned by a CPU test against something
other than itself (closed forms, brute force, library routines, a hand-worked
fixture).  Values at the configurations' random N(0,1) inputs have no printed
counterpart on the pages; for those the oracle is the definition itself.
"""

from . import masks, attn, codec  # noqa: F401
