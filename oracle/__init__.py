"""CPU oracle for the NVFP4 mixture-of-experts expert layer.

TEST INFRASTRUCTURE, NOT PRODUCT. Only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import anything from here. The
HIP library never calls into this package and this package never calls into
the HIP library: the two share no code, tables, constants or helpers.

What it computes, and where the pages fix it (page titles as in the source
pages; sections named there):

* ``formats``   bf16, OCP E4M3FN and E2M1 decode tables and round-to-nearest-
                even encoders, written from the format definitions.
                E2M1 is sign-magnitude with bit 3 the sign and bits 2:0 an index
                into {0, 0.5, 1, 1.5, 2, 3, 4, 6} (src commit log, quantizer
                fix). E4M3 scale bytes are bit patterns that are reinterpreted,
                never value-converted (src commit log, `.view` vs `.to` fix).
* ``quantize``  the two-level NVFP4 quantization of a tensor: global scale
                amax/(6*448), one E4M3 scale per 16 elements equal to
                block_amax/(6*global), nearest E2M1 value, two nibbles per byte
                with the even element in the low nibble (NVFP4 MegaMoE Debug Log, Hypothesis 6
                "vLLM weight loader" steps 1-5; Hypothesis 5 packing; later
                revision, "input_scale red herring" and code-review item 1).
* ``gemm``      dequantization and the block-scaled GEMM with the per-expert
                fp32 alpha applied outside the E4M3 scales (NVFP4 MegaMoE Debug Log,
                Hypothesis 3 and "NVFP4 MoE Pipeline"), accumulated in fp64.
* ``moe``       the five-stage expert layer of the NVFP4 MegaMoE Debug Log "NVFP4 MoE Pipeline".
* ``loops``     an independent pure-Python twin (exact rational arithmetic)
                used only on tiny shapes to pin the vectorized code.

Parity status per function is listed in each module's header.
"""
