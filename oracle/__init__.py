"""CPU oracle for single-query GQA decode attention (TEST INFRASTRUCTURE).

This package is the correctness reference the GPU path is checked against.  It
is a plain, slow, float64 implementation of what the method computes, written
from the pages' definitions and sharing no code with the HIP library.  Only the
test suite, the entry file's ``smoke()`` and the bench's ``cpu_baseline`` leg
may import it; the product path never does.

Pages cited throughout:
  * decode-long page -- "GQA fused-attention decode kernel -- long context"
    (kernbench2, ``_gqa_attention_decode_long.py``): the local tile sweep,
    ``_merge_running``, the final normalise.
  * kernel-map page -- ``muh_kernel_map.py``, ``VLLM_KERNEL_MAP`` entries
    ``paged_attention_v1`` / ``paged_attention_v2``: tensor layouts, fp32
    score/exp_sum/max_logits, single pass vs split + merge.
  * policy page -- ``muh_cc_dispatch.py``, ``AttentionConfig`` and
    ``select_attention_config``: partition size 512, v1/v2 threshold 8192.

Modules:
  oracle.reference  float64 definition, partial triples, merge, split decode.
  oracle.brute      40-digit Decimal brute force for tiny shapes.
"""
