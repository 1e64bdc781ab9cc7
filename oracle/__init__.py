"""Plain fp64 CPU oracle for the TiDAR decode-step hot path.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or
execute anything in this package: only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it. It shares no code with the
HIP library or its Python binding, and neither side imports the other; inputs
come from the separate ``tidar_synth`` generators.

Contents (every function cites the passage it follows):

* ``attention.attn_step``   - hybrid-mask attention by its plain definition,
  per query row over an explicit list of visible keys.
* ``attention.attn_rows``   - the same definition at chosen (b, r, h)
  triples (the checker of sampled outputs at full sizes).
* ``dense.attn_dense``      - independent brute force: a literal 0/1 mask
  matrix built from the region rules, then masked softmax. Used to pin
  ``attn_step`` and ``attn_rows``.
* ``reject.reject_sample``  - AR rejection sampling of the diffusion drafts
  with residual / bonus resampling by inverse CDF; ``trust_ar`` mixes the
  AR and diffusion logits of the targets (``reject.target_logits``).
* ``commit.kv_commit``      - exact-KV append of accepted drafts.
* ``likelihood.token_logprobs`` - AR log-likelihood of each next token from
  the logits of the causal (likelihood-mode) forward.
* ``loop``                  - the step loop around the path: rows and
  positions of a step, and how verification picks the next step's inputs.

All floating point is fp64. Pins live in ``tests/test_oracle_*.py``; no part
is "parity unpinned".
"""
from .attention import attn_step, attn_rows, local_keys, visible_local_count
from .dense import attn_dense, hybrid_mask_matrix
from .reject import reject_sample, expected_accept_len, invcdf, softmax_t, SampleResult, selected_block_rows, target_logits
from .commit import kv_commit
from .likelihood import token_logprobs, sequence_loglik, log_normaliser
from . import loop

__all__ = [
    "attn_step", "attn_rows", "local_keys", "visible_local_count", "attn_dense",
    "hybrid_mask_matrix", "reject_sample", "expected_accept_len", "invcdf", "softmax_t",
    "SampleResult", "selected_block_rows", "target_logits", "kv_commit",
    "token_logprobs", "sequence_loglik", "log_normaliser", "loop",
]
