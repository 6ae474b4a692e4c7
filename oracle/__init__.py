"""fp64 CPU oracle for the linear-attention state-composition path.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import, call or run anything in this
package.  It shares no code with the device path (no kernels, headers, helpers
or constants) and never imports it; the product library never imports it.

Everything here is a plain token-by-token loop in float64 over the same rounded
inputs the device reads (bf16 or fp32 values promoted to float64), written from
the HYPIC pages and the published gated delta rule:

* per-token transition A_t = alpha_t (I - beta_t k_t k_t^T) and write
  beta_t k_t v_t^T (gated delta rule, Yang, Kautz & Hatamizadeh, ICLR 2025);
  the diagonal (GLA) and scalar (RetNet/Mamba2) decay families named in the
  HYPIC news article's linear-layer paragraph, and the per-channel gated delta
  rule A_t = diag(alpha_t)(I - beta_t k_t k_t^T) of the KDA family it also names;
* the segment transition T_C (ordered product of the A_t) and zero-start end
  state S(C|0), composed by S(C1.C2) = T(C2) S(C1) + S(C2) (same paragraph);
* naive addition S(C1) + S(C2), the straw-man the same paragraph rejects;
* the seam window (HYPIC news article, seam-window paragraph; README, "PIC modes");
* the depthwise causal convolution with carried state (conv-state warm-up,
  linear-layer paragraph);
* LPT list scheduling (segment-parallelism paragraph; Graham 1969);
* RoPE state re-rotation of a cached element moved to a new offset (linear-layer
  paragraph; README, "PIC modes", transition_rope).

Parity pins for every function are in tests/test_oracle.py.
"""

from .reference import (  # noqa: F401
    affine_compose,
    apply_T,
    causal_conv,
    compose_fold,
    compose_T,
    dense_recurrence,
    diag_recurrence,
    kda_recurrence,
    l2_normalise,
    lpt_schedule,
    naive_add,
    opt_makespan_bruteforce,
    rel_err,
    rel_err_T,
    rerotate,
    rope_matrix,
    rope_pairs,
    rope_rotate,
    rr_schedule,
    scalar_recurrence,
    seam_advance,
    T_value,
    warm_chain_reference,
)
