"""MI355X-native (gfx950) hot path of one native-MTP speculative decoding cycle.

The kernels live in libmtp.so behind the C ABI declared in include/mtp.h; ``mtp`` is the
thin Python binding with the same entry-point names.
"""
from .mtp import *  # noqa: F401,F403
from .mtp import (EXPORTED, LIB_PATH, Head, MtpError, load_library, mtp_accept_sample,  # noqa: F401
                  mtp_commit_state, mtp_draft_head, mtp_verify_logits, mtp_verify_logits_noalloc, row_stats_empty,
                  row_stats_fields,
                  mtp_pack_head, mtp_tiled_bytes, sampling, tiled_head, workspace, workspace_bytes)
