"""Plain CPU oracle for the tiered decode-attention path (TEST INFRASTRUCTURE).

This package is the slow, obviously-correct definition that the HIP path is
checked against.  Only the test-suite, the smoke entry point and the
benchmark's CPU-baseline leg may import it; the product path never does.  It
shares no code with the HIP library: every formula here is written from the
pages, in numpy, in float64 for attention and score arithmetic, with float32 /
float16 only where a quantization step fixes that precision.

Modules and the passages they follow:

* ``numerics``  -- bfloat16 / float16 roundings used by the codecs.
* ``codec``     -- the uniform (affine, zero = min) quantizer of the HqeKV
                   notes section 2.3 Eq.(2), grouped KIVI-style (keys per
                   channel, values per token; KV-cache evolution page section 5),
                   the normalized quantizer of Eq.(3)-(4), canonical packing.
* ``attention`` -- scaled-dot-product single-query attention, QEvict notes
                   section 4.1 Eq.(attention); H2O page section 1.1.
* ``rank``      -- the total order used by every router (score desc, position
                   desc) and multi-tier assignment by counts.
* ``qevict``    -- QEvict accumulated window score Eq.(1), capacities Eq.(3),
                   candidate pool / tiering Eq.(4)-(6), Algorithm 1 (pack once,
                   reuse codes, dequantize on promotion).
* ``h2o``       -- H2O cumulative score, budget split, update order and
                   victim choice (H2O page sections 1.2, 2.1, 3.3).
* ``hqekv``     -- HqeKV joint metric, ratio tiers and downgrade-only
                   re-quantization (HqeKV notes sections 3.2-3.5, 3.7).
* ``budget``    -- capacity and payload arithmetic (QEvict section 4.3/4.5;
                   KV-cache evolution page sections 2, 5, 10).
* ``diagnostics`` -- future missed mass, mass by tier, selection churn and
                   long-term importance recovery against full-cache attention
                   (QEvict notes section 3).

Readings of silent or ambiguous passages are stated where they are used.
"""
