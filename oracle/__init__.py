"""Plain, slow, float64 CPU oracle for PACE-style periodic-rounding GDN decode.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call, link
or execute anything in this package: only the tests, the smoke check and the
CPU-baseline leg of the benchmark use it.  It shares no code, header, table or
helper with the HIP library; the only thing both sides consume in common is the
seeded input generator, which holds none of the method's arithmetic.

What it computes, in the order of the pages:

* ``gdn``   - the gated delta-rule recurrence, token by token, in float64
              (the gate sets the forgetting rate, the delta rule makes each write
              an online-learning step against the current state:
              '低比特量化新突破：GGA+PW让线性注意力长文本生成更准更短', section
              '为什么低比特状态量化会“越写越错”').
* ``quant`` - symmetric round-to-nearest-even quantization with one scale per
              state column ('PACE: A New 4-Bit Recurrent State Quantization
              Method ...', section 'Channel-Aligned Encoding').
* ``pace``  - periodic rounding: decode the stored state, apply the period's
              tokens in high precision, re-encode once per period
              ('PACE: four-bit recurrent state by rounding less often', TL;DR
              point (1) and the flowchart 'Fewer roundings, less compounded
              error').
* ``chunk`` - the chunked (WY/UT) form of one period, used only to pin that
              chunked and sequential updates agree; chunked kernels are the
              pages' motivation for periodic rounding (same page, TL;DR (1)).

Parity status per function is listed in each module header.
"""
from . import chunk, gdn, pace, quant  # noqa: F401
