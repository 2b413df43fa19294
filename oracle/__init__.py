"""CPU oracle for Ozaki scheme II DGEMM/ZGEMM -- test infrastructure only.

Imported only by tests/, __graft_entry__.smoke() and bench.py's cpu_baseline
leg; see oz2_oracle.py for what it computes and how it is pinned, and
rescale_be.py for the persistent tensor-chain method (OzII-RescaleBE).
"""
from .oz2_oracle import *  # noqa: F401,F403
from .oz2_oracle import (  # noqa: F401
    max_product_moduli, moduli_product, log2_M, n_limbs, scaling_width, moduli_for_bits,
    sym, sym_byte, crt_weights, crt_reconstruct, frexp_exponent, exact_dot,
    fraction_to_double, gemm_entries, chat_residues, encode_vectors, hat_to_int,
    i256_to_int, max_threads,
)
from . import rescale_be  # noqa: F401,E402
