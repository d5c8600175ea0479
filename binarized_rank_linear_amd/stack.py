"""Stacks of independent LittleBit linears run as one group.

A stack holds L layers of the same linear shapes (for example the seven
linears of a decoder layer).  Every layer reads the same inputs (one x per
input width) and writes its own outputs.  The factors of each layer come from a
caller-supplied function, are packed on the GPU and the float copies dropped.
"""
from __future__ import annotations

from typing import Callable, Dict, List, Sequence, Tuple

from . import PackedLinear, Group, rank_for_budget, LB_PATH_AUTO


class LayerStack:
    def __init__(self, shapes: Sequence[Tuple[str, int, int]], layers: int, b_num: int, b_den: int,
                 residual: bool, make_factors: Callable, device="cuda"):
        """shapes: (name, d_in, d_out) per linear of one layer.
        make_factors(layer, index, d_in, d_out, r_path, paths) -> (U, V, h, g, l)
        GPU tensors as PackedLinear.from_factors takes them."""
        import torch
        self.shapes = list(shapes)
        self.layers = layers
        self.residual = residual
        self.P = 2 if residual else 1
        self.ranks = [rank_for_budget(di, do, b_num, b_den, residual) for (_, di, do) in shapes]
        self.linears: List[List[PackedLinear]] = []
        for L in range(layers):
            row = []
            for i, ((name, di, do), (r, rp)) in enumerate(zip(self.shapes, self.ranks)):
                U, V, h, g, l = make_factors(L, i, di, do, rp, self.P)
                row.append(PackedLinear.from_factors(U, V, h, g, l))
                del U, V
            self.linears.append(row)
        torch.cuda.synchronize()

    def bind(self, T: int, x_by_width: Dict[int, "object"], out_dtype, flags: int = LB_PATH_AUTO):
        """Allocate outputs and build the group for T tokens.  x_by_width maps
        d_in -> x tensor [T][d_in]."""
        import torch
        items = []
        self.outputs = []
        for L in range(self.layers):
            outs = []
            for lin in self.linears[L]:
                y = torch.empty((T, lin.d_out), dtype=out_dtype, device=x_by_width[lin.d_in].device)
                outs.append(y)
                items.append((x_by_width[lin.d_in], y, lin))
            self.outputs.append(outs)
        x0 = next(iter(x_by_width.values()))
        self.group = Group(items, T, x0.dtype, out_dtype, flags)
        return self.group

    def tight_sign_bytes(self) -> int:
        return sum(lin.tight_sign_bytes() for row in self.linears for lin in row)

    def scale_bytes(self) -> int:
        return sum(lin.scale_bytes() for row in self.linears for lin in row)

    def packed_bytes(self) -> int:
        return sum(lin.packed_bytes() for row in self.linears for lin in row)


class DecoderStack:
    """L decoder layers chained at decode time (lb_decoder_layer_forward):
    each layer's output is the next one's input.  The factors come from
    make_factors(layer, index, d_in, d_out, r_path, paths) for the seven
    linears q, k, v, o, gate, up, down in that order."""

    NAMES = ("q", "k", "v", "o", "gate", "up", "down")

    def __init__(self, d_model: int, d_ff: int, n_heads: int, n_kv_heads: int, layers: int, b_num: int,
                 b_den: int, residual: bool, make_factors: Callable, eps: float = 1e-6):
        import torch
        from . import DecoderLayer
        dkv = d_model // n_heads * n_kv_heads
        shapes = dict(q=(d_model, d_model), k=(d_model, dkv), v=(d_model, dkv), o=(d_model, d_model),
                      gate=(d_model, d_ff), up=(d_model, d_ff), down=(d_ff, d_model))
        self.d_model = d_model
        self.P = 2 if residual else 1
        self.layers: List[DecoderLayer] = []
        for L in range(layers):
            lins = []
            for i, name in enumerate(self.NAMES):
                di, do = shapes[name]
                r, rp = rank_for_budget(di, do, b_num, b_den, residual)
                U, V, h, g, l = make_factors(L, i, di, do, rp, self.P)
                lins.append(PackedLinear.from_factors(U, V, h, g, l))
                del U, V
            self.layers.append(DecoderLayer(*lins, n_heads=n_heads, n_kv_heads=n_kv_heads, eps=eps))
        torch.cuda.synchronize()

    def linears(self):
        return [lin for layer in self.layers for lin in layer.lin.values()]

    def workspace_bytes(self, T: int) -> int:
        return max(layer.workspace_bytes(T) for layer in self.layers)

    def forward(self, x, bufs, ws, stream=None):
        """Runs every layer; bufs is a pair of [T][d_model] bf16 tensors the
        activations alternate between (neither may be x).  Returns the one
        holding the output."""
        cur = x
        for i, layer in enumerate(self.layers):
            out = bufs[i & 1]
            layer.forward(cur, out=out, ws=ws, stream=stream)
            cur = out
        return cur
