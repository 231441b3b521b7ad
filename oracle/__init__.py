"""CPU fp64 oracle for the fused scaled-dot-product attention forward pass.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or load
this package: only ``tests/``, ``__graft_entry__.smoke()`` and the oracle
leg of ``bench.py`` (``cpu_baseline``, ``cpu_baseline_by_workload`` and the
``max_abs_err`` comparison, all skipped with ``--no-cpu-baseline``) use it.  It shares no code with the HIP
library in ``attention_forward_06_amd/`` and imports nothing from it.

Contents
  attention.py  plain definition (full masked score rows, standard softmax) and
                the pages' online recurrence written out in fp64
  brute.py      pure-Python loops (math.exp / math.fsum) for L <= 16
  fp_formats.py round-to-nearest-even into narrow float formats (OCP e5m2,
                bfloat16, IEEE binary16) written from the format definitions

Sources (web pages; cited by title and section):
  [TLX]   "TLX Block Attention" -- block-diagonal sparse attention in Triton
  [TCA]   "Triton-CUDA Attention" -- online softmax core + full FlashAttention example
  [FA-A]  "Fused Attention" (Triton-Ascend example 04) -- causal two-stage kernel,
          fp8 V, head_dim 256

Parity status: every function here is pinned by tests/test_oracle.py against
brute force, a library routine, closed forms or invariants, except where its
docstring says "parity unpinned".
"""
from .attention import (MODES, visible_mask, attn_weights, attn_ref, attn_online_ref, attn_lse_ref,
                        visible_pairs, attn_flops)
from .brute import attn_brute, lse_brute
from .fp_formats import (round_e5m2, round_bf16, round_f16, e5m2_decode, e5m2_encode,
                         round_to_format)

__all__ = ["MODES", "visible_mask", "attn_weights", "attn_ref", "attn_online_ref", "attn_lse_ref",
           "visible_pairs", "attn_flops", "attn_brute", "lse_brute", "round_e5m2", "round_bf16",
           "round_f16", "e5m2_decode", "e5m2_encode", "round_to_format"]
