"""CPU oracle for the fused top-K KD loss and its teacher cache.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the bench's
CPU-baseline leg may import this package.  The product path (the HIP
library and its Python binding) never imports, links or calls it, and the
two share no code.

Everything here is plain float64 numpy: the dense definitions written out,
with no blocking, fusion or reordering beyond splitting the token axis into
blocks so the [T, V] logits of large inputs need not exist at once.

Sources (cited by title and section, figure or equation):

* "The Gradient That Top-k Distillation Never Computes" (Khanbayov, Kurban):
  abstract and Figures 1-3 define the renormalized top-k objective L_S, the
  tail masses m_q / m_p, the truncated-gradient decomposition, and the
  twelve-token worked example (Figure 2).
* "Tail-Aware Top-k On-Policy Distillation" (Huang, Wei), abstract: the
  top-k bins plus one tail bin carrying the tail probability, in the forward
  (TAIL) and in the paper's own reverse (TAIL_REVERSE) direction.
* "Unbiased Top-k Estimation for On-Policy Distillation" (Meng et al.),
  abstract and Table 2: reverse KL between the normalized top-k
  distributions, with the student's own top-16 as the support; abstract and
  Figure 1: the top-k reverse-KL gradient plus a sampled-token tail
  correction under a stop-gradient (REVERSE_TT).
* "Efficient Knowledge Distillation for LLMs: Offline Top-K Logits and a
  Fused Chunked KL Loss", section 3.2, Eq. (2) and Eq. (3): the partial-mass
  forward KL against an unrenormalized top-K teacher and its closed-form
  logit gradient M*softmax(z) minus the sparse teacher term.
* "Sparse Teacher Support Cuts LLM Distillation Cost Without Losing
  Accuracy", definition of k_rho: the smallest k whose top-k teacher mass
  reaches rho.
* "The Gradient That Top-k Distillation Never Computes", Figure 3 (bottom):
  the hidden-state teacher cache, whose head reconstruction gives the exact
  full-vocabulary KL.
* "The Gradient That Top-k Distillation Never Computes", abstract and
  Table 1: the teacher is recoverable from k >= d + 1 cached log-probs.
* The hard-label cross-entropy term that "The Gradient That Top-k
  Distillation Never Computes" (abstract) trains with or without, added
  with a weight to any of the four distillation losses.

Every function is pinned by a CPU test (tests/test_oracle.py) against
printed values, closed forms, library routines, finite differences or
brute force; none is "parity unpinned".
"""
from .kd_oracle import (  # noqa: F401
    RENORM, TAIL, FULL, REVERSE, TAIL_REVERSE, REVERSE_TT, MODES, MODE_NAMES,
    logsumexp, student_logits, loss_rows_from_logits, loss_fwd_bwd,
    topk_row, cache_from_logits, cache_build, teacher_logp, adaptive_k_row, kl_hidden_fwd_bwd,
    quantize_hidden_int8, recover_teacher_hidden,
)
