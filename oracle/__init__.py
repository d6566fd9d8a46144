"""CPU oracle for the KVpop future-attention target path.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the bench's
CPU-baseline leg may import this package.  It is a plain, slow, fp64
implementation written from the KVpop pages and shares no code with the HIP
library (it imports nothing from `attention_target_amd`).

Sources cited in this package:
  [P] "KVpop -- Key-Value Cache Compression with Predictive Online Pruning",
      paper text (papers.paperslantern.ai page): Section 3 (method overview and
      per-head budget), Section 3.1 (future-attention target, Eqs. 2-4),
      Section 3.2 (transposed-attention target computation, Eq. 8; running
      top-k sparse attention), Section 4 (setup: packing, S = 16384).
  [G] "KVpop -- predictive online pruning" Korean technical summary
      (gist.science page): Section 2.1 (budget B = s + w + k, first tokens are
      sinks), Section 2.2 (target over queries d >= t + w), Section 2.4
      (running threshold with a Fenwick tree).

Modules:
  dense   -- dense causal attention with LSE, column sums of the attention
             matrix (future mass), the transposed (Eq. 8) formulation, and the
             target epilogue (SUM / MAX / NONE aggregation over query heads).
  budget  -- static ranks, the Fenwick-tree running cutoff, mask rows, a
             per-row brute-force top-k selection, masked attention.
  brute   -- pure-Python triple loops with math.fsum for tiny inputs.

Conventions (readings of the pages, see each function):
  * softmax scale sigma = 1/sqrt(D) unless given;
  * all logs are natural logs;
  * query head g uses KV head g // G (G = Hq / Hkv);
  * packed sequences: attention never crosses a document boundary;
  * the protected window of query d is (d-w, d]; the eligible set is
    E_d = [s, d-w] (inclusive); the target of key t sums over d >= t + w.

Every function is pinned by tests under tests/test_oracle_*.py against brute
force, closed forms, invariants or library routines; none is "parity
unpinned" except the heavy-hitter input recipe, which is input generation, not
oracle arithmetic.
"""
from . import dense, budget, brute  # noqa: F401

__all__ = ["dense", "budget", "brute"]
