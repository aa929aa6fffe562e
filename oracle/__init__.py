"""CPU oracle for SparK (test infrastructure only; see spark_oracle's header)."""
from .spark_oracle import *  # noqa: F401,F403
from .spark_oracle import (num_kept, chan_energy, saliency_keys, select_top_t, mask_words,  # noqa: F401
                           mask_from_words, pack_kept, prune, stats, expand_keys, decode_attn,
                           dense_attn, window_scores, snapkv_evict, window_rows, philox4x32_10,
                           uniform01, recovery_samples, expand_keys_sampled, decode_attn_sampled,
                           value_keys, prune_v, decode_attn_kv, value_block_keys, prune_v_blocks, channel_groups,
                           grouped_num_kept, select_grouped, prune_grouped, tree_sum32,
                           select_top_p, prune_topp, append_tokens, grow_cache)
