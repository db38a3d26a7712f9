"""Plain fp64 CPU oracle for the joint video+text attention hot path.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The product path
(``rope_joint_attention_amd`` and its HIP library) never calls it, and it never
calls the product path: the two share no code.  Inputs come from ``hvinputs``,
which holds no arithmetic of the method.

Each function restates, in NumPy float64, what the HunyuanVideo notes page
("HunyuanVideo 模型结构与数学原理", note.shouss.top) says is computed:

* ``token_grid``      section 4 (Causal 3D VAE) latent-size and token-count formulas;
* ``apply_rope3d``    section 5.5 (3D RoPE), a direct sum of three 1-D rotary
                      embeddings over channel blocks (16, 56, 56);
* ``joint_attention`` section 5.2 (double-stream block) joint softmax attention
                      over the video-then-text sequence, scale 1/sqrt(128),
                      with padded text keys left out (section 3.1 keeps at
                      most 256 prompt tokens; section 5.2 names the valid
                      text length);
* ``rms_norm_heads``  section 5.4, per-head RMSNorm of Q and K;
* ``qk_norm_rope3d``  RMSNorm (video / text gamma, section 5.2) followed by the
                      3D RoPE of section 5.5;
* ``attention_lse``   attention of query rows against a separate K/V block,
                      with the log-sum-exp of each row (section 9.2, Ring
                      Attention keeps query rows and passes K/V blocks);
* ``merge_partials``  the exact combination of attention over disjoint key
                      blocks from their outputs and log-sum-exps;
* ``varlen_attention`` attention over packed segments (section 9.1, the
                      variable-length FlashAttention call);
* ``joint_attention_bwd`` gradients dQ, dK, dV of the joint attention (the
                      report summary page's training-side attention cost),
                      by the chain rule through the softmax
                      (``joint_attention_bwd_dq_rows``: dQ of selected rows;
                      ``joint_attention_bwd_by_rows``: all three for long
                      sequences, the key gradients summed over chunks of
                      query rows; ``varlen_attention_bwd``: the same over
                      packed segments);
* ``hot_path``        token grid, RoPE and attention in sequence.

Nothing here is blocked, fused or reordered beyond the formulas: the matrix
products use NumPy's matmul as a library primitive, and query rows are
processed in independent chunks only to bound memory.

Pins (tests/test_oracle_*.py): printed token counts, closed-form rotation
angles, norm and relative-position invariants, the complex-number form of
RoPE, uniform/one-key/two-key closed forms, permutation and shift
invariance, masking with poisoned values, a pure-Python brute force, and for
the RMSNorm unit output RMS, scale invariance, an epsilon closed form, head and
channel isolation and the per-pair magnitudes that fix its order against RoPE;
for the log-sum-exp, merge and packed forms closed forms on one and repeated
keys, the union identity, brute force, and agreement of the packed form with
separate per-clip calls; for the gradients central finite differences of the
oracle's own forward, and the shift and sum identities they obey.
"""
from .hv_oracle import (  # noqa: F401
    HEADS,
    HEAD_DIM,
    ROPE_AXES,
    OracleGrid,
    token_grid,
    rope_frequencies,
    video_coordinates,
    apply_rope3d,
    rms_norm_heads,
    qk_norm_rope3d,
    joint_attention,
    attention_lse,
    merge_partials,
    varlen_attention,
    joint_attention_bwd,
    joint_attention_bwd_dq_rows,
    joint_attention_bwd_by_rows,
    varlen_attention_bwd,
    hot_path,
)
