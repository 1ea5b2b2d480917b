"""Copy host weight arrays to the device and wrap them in descriptors.

Pure marshalling: numpy arrays (storage layout, see include/sfnn.h) become
torch device tensors and sfnn descriptors.  No arithmetic on the values.
"""
from __future__ import annotations

from typing import Optional

import numpy as np
import torch

from ._lib import FFN, Pred, SFNN_RELU, SFNN_REGLU


def to_dev(a: Optional[np.ndarray], device="cuda") -> Optional[torch.Tensor]:
    if a is None:
        return None
    return torch.from_numpy(np.ascontiguousarray(a)).to(device, non_blocking=False)


def upload_layer(lay, device="cuda", predictor: bool = True):
    """(Pred | None, FFN) on ``device`` from an object holding the storage arrays
    (w1_t, w2_t, tau, w_up/q_up, w_gate/q_gate, w_down_t/q_down_t, s_*, b_*)."""
    act = SFNN_REGLU if getattr(getattr(lay, "spec", None), "act", "relu") == "reglu" else SFNN_RELU
    pred = None
    if predictor and getattr(lay, "w1_t", None) is not None:
        pred = Pred(to_dev(lay.w1_t, device), to_dev(lay.w2_t, device), to_dev(lay.tau, device))
    q = getattr(lay, "q_up", None)
    if q is not None:
        ffn = FFN(to_dev(lay.q_up, device), to_dev(lay.q_down_t, device), act=act,
                  w_gate=to_dev(getattr(lay, "q_gate", None), device),
                  s_up=to_dev(lay.s_up, device), s_gate=to_dev(getattr(lay, "s_gate", None), device),
                  s_down_t=to_dev(lay.s_down_t, device),
                  b_up=to_dev(lay.b_up, device), b_gate=to_dev(getattr(lay, "b_gate", None), device),
                  b_down=to_dev(lay.b_down, device))
    else:
        ffn = FFN(to_dev(lay.w_up, device), to_dev(lay.w_down_t, device), act=act,
                  w_gate=to_dev(getattr(lay, "w_gate", None), device),
                  b_up=to_dev(lay.b_up, device), b_gate=to_dev(getattr(lay, "b_gate", None), device),
                  b_down=to_dev(lay.b_down, device))
    return pred, ffn


def workspace(pred, ffn, batch: int, device="cuda") -> torch.Tensor:
    from ._lib import sfnn_workspace_bytes
    n = sfnn_workspace_bytes(pred, ffn, batch)
    if n == 0:
        raise ValueError("invalid layer shape or batch for the workspace query")
    return torch.empty(n, dtype=torch.uint8, device=device)
