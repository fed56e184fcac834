"""CPU oracle for the sparse masked-diffusion sampling step (test infrastructure).

This package is TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import it.  The HIP library and
its Python binding never import, call or link anything here, and nothing here
imports them: the only code both sides share is the seeded input generator
package ``mdm_inputs``, which holds none of the method's arithmetic.

It is a plain, slow NumPy implementation in float64 of what one sampling step of
Sparse-LaViDa computes, written from the pages' statement of the method:

* sparse representation of a partially masked sequence (page 1, key design 1;
  page 3, section 3.1 and Figure 4)                              -> sparse_repr
* register tokens after the sequence end (page 1, key design 2)  -> step
* step-causal attention, inference form (page 1, worked example =
  paper Figure 3; page 3, Figure 3) and training form (page 1,
  key design 3; page 3, sections 3.3 and 7.3)                    -> masks
* attention over explicit sparse position ids (RoPE)              -> rope, attention
* logits only for the decoded subset, max-probability confidence
  and argmax (page 1, key design 1; page 3, section 3.2)         -> logits
* unmasking: pre-generated order (images) or confidence within a
  semi-autoregressive block (text) (page 3, section 3.2)         -> select
* the incremental loop with KV cache (page 3, section 3.2)        -> step
* from-scratch recompute under the training-form block mask       -> dense

Every function cites the passage it follows.  Pins against values the pages
print, closed forms and independent library routines live in
``tests/test_oracle_*.py``.  Parity of decoded tokens on the synthetic
workloads is pinned only by this oracle plus those invariants (the pages print
no token values for them).
"""
