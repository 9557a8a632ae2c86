"""Float64 CPU oracle (test infrastructure only; never imported by the product path)."""
from .dcp_oracle import (attention, merge, owner_rank, rank_tokens, rank_length,  # noqa: F401
                         mla_inputs, gqa_inputs, request_inputs, rank_partial, full_attention,
                         causal_limits, causal_attention, mtp_query, mtp_rank_partial,
                         mtp_full_attention)
