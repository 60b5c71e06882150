"""fp64 CPU oracle of the quantized routed-MoE layer.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call,
link or execute anything in this package: only tests/, the smoke check in
__graft_entry__.py and the cpu_baseline leg of bench.py use it.  It shares
no code, header, table or constant generator with the HIP library under
bit_quantized_moe_02_amd/; the two meet only through arrays and bytes in
the tests.

What it computes comes from the ds4 pages (routed experts quantized to 2-bit,
up/gate in a codebook format and down in a K-quant format; shared expert and
router kept in high precision -- ds4 digest "Model weights" section and the
upppp.jp article's "asymmetric 2-bit quantization" section) and from the
format definitions that include/qmoe.h documents (CB2, K2, K4, BF16 tiles).
See qmoe_oracle.py for the functions and their readings of the pages.
"""
from .qmoe_oracle import *  # noqa: F401,F403
