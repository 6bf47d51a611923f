"""fp64 CPU oracle (test infrastructure only; see ``oracle.nq_oracle``)."""
from .nq_oracle import (bits_per_weight, compression_ratio, linear_dense, linear_factored,
                        rank_for_bits, stored_bytes, reconstruct_weight)

__all__ = ["bits_per_weight", "compression_ratio", "linear_dense", "linear_factored",
           "rank_for_bits", "reconstruct_weight", "stored_bytes"]
