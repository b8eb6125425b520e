"""Upload a generated workload to device memory (plumbing only: copies, no arithmetic)."""

from __future__ import annotations

import numpy as np
import torch


def upload(w, device="cuda") -> dict:
    """Device tensors of a :class:`gen.Workload`: bf16 data as torch.bfloat16 views of the bits."""
    def bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(torch.bfloat16)

    def i32(a):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(device)

    out = {
        "q": bf16(w.q),
        "k_pages": bf16(w.k_pages),
        "v_pages": bf16(w.v_pages),
        "page_table": i32(w.page_table),
        "seq_lens": i32(w.seq_lens),
    }
    if getattr(w, "csize", None) is not None:
        out["centroids"] = bf16(w.centroids)
        out["csize"] = i32(w.csize)
        out["coff"] = i32(w.coff)
    return out
