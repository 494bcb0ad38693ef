"""Oracle for block-causal / teacher-forcing masked attention forward + JVP.

TEST INFRASTRUCTURE ONLY.  Plain, slow, float64 CPU code that states what
the fused GPU operator must compute.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py``
may import it; the product path never does.  It shares no code, headers,
tables or helpers with the HIP library, and it never reads anything the
HIP library produced.

Sources (Causal-rCM, arXiv 2606.25473):

* section 2.3 and section 3.1.1 (eq. 8): the teacher-forcing (TF) packed
  sequence [clean | noisy] and its mask; the Table 2 legend (TF = clean and
  noisy frames concatenated under a special causal mask, DF = plain
  block-causal mask);
* section 4 "Experiments": frame-wise (c1-1) and chunk-wise (c3-3) chunking,
  with the same chunk pattern for every packed mask;
* Appendix B, eqs. (42)-(45): masked attention, the score tangent, the
  attention tangent with the mask held fixed, and its online form;
* section 3.1.2 (teacher-forcing sCM, after eq. 17): the clean context
  carries zero tangent, only the noisy tokens move;
* section 3.2.1 (FlashAttention-2 based kernel with custom masks): the
  backward of the same masked attention, for training the student;
* Appendix B, "sparse custom mask representation": masks as query groups
  (contiguous query intervals) with lists of allowed key intervals
  (``RangeMask``); section 4 (cA-B chunk patterns with an initial chunk of
  another size, ``ChunkListDesc``) and section 4.2.2 / Figure 9 (an
  understanding / generation layout) give the range masks exercised.

Parity pins (see ``tests/test_oracle_*.py``): hand-written golden masks,
closed-form pair counts, finite differences, ``torch.func.jvp`` on dense
masked attention, closed forms (uniform scores, two-key rows, single-key
rows), and the invariants of softmax and its tangent.  Every function here
has at least one pin.
"""
from .masked_attention import (  # noqa: F401
    MaskDesc,
    ChunkListDesc,
    RangeMask,
    allowed,
    allowed_row,
    mask_dense,
    pair_count,
    row_groups,
    query_blocks,
    key_tiles,
    tile_classes,
    masked_attention_jvp_slice,
    masked_attention_jvp,
    masked_attention_jvp_rows,
    masked_attention_jvp_scalar,
    zero_clean_tangents,
    masked_attention_jvp_slice_ctz,
    pair_counts_by_class,
    useful_flops,
    masked_attention_bwd_slice,
    masked_attention_bwd,
    masked_attention_bwd_rows,
    backward_useful_flops,
)
