"""Move seeded workload inputs onto the GPU and describe the workload's mods
to the binding.  Plumbing only: no attention arithmetic."""
from __future__ import annotations

import numpy as np
import torch

from . import Workload


def to_device(w: Workload, inputs: dict, device="cuda"):
    """q, k, v device tensors (float32 or bfloat16, exactly the generated values) and doc_id."""
    dev = torch.device(device)
    out = []
    for name in ("q", "k", "v"):
        if w.dtype == "bf16":
            bits = np.ascontiguousarray(inputs[name + "_bits"]).view(np.int16)
            out.append(torch.from_numpy(bits).to(dev).view(torch.bfloat16))
        else:
            out.append(torch.from_numpy(np.ascontiguousarray(inputs[name], dtype=np.float32)).to(dev))
    doc = None
    if inputs.get("doc_id") is not None:
        doc = torch.from_numpy(np.ascontiguousarray(inputs["doc_id"], dtype=np.int32)).to(dev)
    return out[0], out[1], out[2], doc


def specs(w: Workload, doc_id=None):
    """(MaskSpec, ScoreSpec) of the binding for this workload."""
    from programmable_block_sparse_amd import MaskSpec, ScoreSpec
    mask = MaskSpec(kind=w.mask, window=w.window, sinks=w.sinks, q_offset=w.q_offset, doc_id=doc_id,
                    clauses=w.clauses)
    score = ScoreSpec(kind=w.score, cap=w.cap, alibi_m=w.alibi_m)
    return mask, score

