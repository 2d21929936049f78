"""CPU reference oracle (test infrastructure only; see bsa_oracle)."""
from .bsa_oracle import (PlanRef, attention_dense_masked, attention_live_tiles, plan,  # noqa: F401
                         token_mask, topk_attention)
