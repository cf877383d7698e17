"""The Python binding's layout checks (the C ABI sees only pointers, so the
binding refuses tensors that are too small, of the wrong element type,
non-contiguous, on the host, or a shard list of the wrong length) before any
launch; the library is not called."""
import math

import pytest

from context_packed_attention_amd import api, synth
from tests import gpu_harness as H

pytestmark = pytest.mark.gpu


def test_binding_refuses_bad_tensors():
    import torch
    bt = synth.make_batch("binding", 5, [96, 32], [96, 32], 4, 2, 64)
    db = H.DeviceBatch(bt)
    meta, loc = H.local_inputs(db, 2, 0)
    scale = 1.0 / math.sqrt(bt.d)
    ta = loc["t_alloc"]
    out = torch.empty((ta, bt.hq, bt.d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((bt.hq, ta), dtype=torch.float32, device="cuda")
    ws = torch.empty(api.cp_attn_workspace_bytes(meta, bt.hq, bt.hkv, bt.d, 0), dtype=torch.uint8, device="cuda")
    q, ks, vs = loc["q"], loc["k"], loc["v"]

    def fwd(**kw):
        a = dict(q=q, k_shards=ks, v_shards=vs, out=out, lse=lse)
        a.update(kw)
        api.cp_attn_fwd(meta, a["q"], a["k_shards"], a["v_shards"], bt.hq, bt.hkv, bt.d, scale, 1, a["out"],
                        a["lse"], ws)

    cases = {
        "short q": dict(q=q[:-1]),
        "float32 out": dict(out=out.float()),
        "non-contiguous out": dict(out=out.transpose(1, 2)),
        "host lse": dict(lse=lse.cpu()),
        "one shard missing": dict(k_shards=ks[:1]),
        "short shard": dict(v_shards=[vs[0], vs[1][:-1]]),
    }
    for name, kw in cases.items():
        with pytest.raises(ValueError):
            fwd(**kw)
        H.log(f"[binding] {name}: refused")
    fwd()  # the well-formed call still runs
    torch.cuda.synchronize()
    meta.close()
