"""CPU oracle for the FAD-KV encoder (test infrastructure; see fadkv_oracle's header)."""
from .fadkv_oracle import *  # noqa: F401,F403
from .fadkv_oracle import (OracleParams, Codes, VectorCode, encode, encode_vector, adapt,  # noqa: F401
                           adapt_dictionary, reconstruct, replay_support, round_to_storage,
                           screening_scores, candidate_pool, gm_support, pl_support,
                           ridge_system, ridge_coefficients, relative_residual,
                           append, append_dictionary, pool_recall)
