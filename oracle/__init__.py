"""CPU oracle for the MBOK linear layer (test infrastructure only; see
mbok_oracle's header for who may import it)."""
from .mbok_oracle import *  # noqa: F401,F403
from .mbok_oracle import (GROUP, ROW_BLOCK, bound, dequantize, max_error_ratio,  # noqa: F401
                          pack, packed_nbytes, product, product_fraction,
                          residual_binarize, round_alpha, unpack)
