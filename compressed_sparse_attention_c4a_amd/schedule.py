"""Attention type of every layer of DeepSeek-V4-Pro.

"图解DeepSeek V4：详细计算流程解析" section 1 (整体架构): the model has 61 layers;
the first three pair hash-MoE with the attention types HCA, HCA, CSA; in the
remaining 58 layers HCA and CSA alternate, and the last layer is SWA
(sliding-window attention).  The page defers the exact table to a config it
does not reproduce, so two points are readings: the alternation continues
from the first three (layer 3 is HCA, layer 4 CSA, ...), and the SWA layer is
the 61st layer itself.  That gives 31 HCA, 29 CSA and 1 SWA layers.
"""
from __future__ import annotations

N_LAYERS = 61
HCA, CSA, SWA = "hca", "csa", "swa"


def attention_kinds(n_layers: int = N_LAYERS) -> list:
    """The attention type of layers 0 .. n_layers-1 (n_layers >= 4): HCA,
    HCA, CSA, then HCA/CSA alternating, and SWA for the last layer."""
    if n_layers < 4:
        raise ValueError("the schedule needs at least 4 layers (3 leading layers and the SWA layer)")
    kinds = [HCA, HCA, CSA]
    for layer in range(3, n_layers - 1):
        kinds.append(HCA if layer % 2 == 1 else CSA)
    kinds.append(SWA)
    return kinds
