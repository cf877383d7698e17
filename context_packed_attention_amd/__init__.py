"""MI355X-native context-parallel packed-THD ring attention: one rank's share.

The compute lives in libcpattn.so (HIP, gfx950); :mod:`.api` is its Python
binding and :mod:`.synth` draws seeded synthetic inputs.
"""
from . import api, synth  # noqa: F401
from .api import (  # noqa: F401
    CpAttnError, Meta, cp_attn_bwd, cp_attn_fwd, cp_attn_last_error, cp_attn_meta_export, cp_attn_rank_metadata,
    cp_attn_rank_metadata_host,
    cp_attn_shard_gather, cp_attn_workspace_bytes,
)
