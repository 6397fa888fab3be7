"""Full prefill weight pass on the A8 route: every projection of a 64-layer
dense decoder applied to an M-token prompt chunk, back to back on one stream.

For large prompt steps the pages' A8 artifact quantizes activations per token
and per 64 channels to int8 and contracts them with the groupwise 4-bit
weights on int8 matrix units (page 5, "Qwen3.8-27B on RTX 4090: 5,000 tok/s
Prefill Reproduced", section "Why the A8 artifact matters"; the pp2048 figure
in its reproduction section is a 2048-token prompt).  Layer widths as in the
decode pass: per layer qkv 5120 -> 7168, out 5120 -> 5120, gate and up
5120 -> 17408, down 17408 -> 5120.

Each layer quantizes its three distinct inputs once (the layer input, shared by
qkv, gate and up; the attention output, read by out; the FFN activation, read by
down) and runs five A8 GEMMs.  Inputs are synthetic and the same for every
layer, but every layer quantizes them again, as a model's would change; the
projections do not feed each other, so the pass measures the A8 route alone.
Outputs go to one buffer per projection, overwritten layer after layer.
"""

from . import binding, synthetic

# index of each projection's input among the three per-layer inputs
_INPUT_OF = {"qkv": 0, "out": 1, "gate": 0, "up": 0, "down": 2}


class PrefillPass:
    """Packed weights of all layers (or a DecodeStep's, shared), the three
    activation inputs, their A8 workspaces and one output per projection."""

    def __init__(self, m, layers=synthetic.N_LAYERS, device="cuda", weights=None, keep_rows=None):
        """weights: optional per-layer [(codes, scales)] in LAYER_PROJECTIONS
        order (e.g. a DecodeStep's ``layers``); else generated here.
        keep_rows: as for DecodeStep, {(layer, proj_index): row indices} whose
        fp32 weight rows are copied to the host for spot checks."""
        import torch
        self.m = m
        self.kept = {}
        if weights is None:
            weights = []
            for layer in range(layers):
                projs = []
                for pi, (_, k, n) in enumerate(synthetic.LAYER_PROJECTIONS):
                    w = synthetic.weights_device(n, k, synthetic.layer_weight_seed(layer, pi), device=device)
                    if keep_rows and (layer, pi) in keep_rows:
                        idx = torch.as_tensor(keep_rows[(layer, pi)], device=device)
                        self.kept[(layer, pi)] = w.index_select(0, idx).cpu().numpy()
                    projs.append(binding.pack(w))
                    del w
                weights.append(projs)
        self.layers = weights[:layers]
        ks = {}
        for name, k, _ in synthetic.LAYER_PROJECTIONS:
            ks[_INPUT_OF[name]] = k
        self.xs = [synthetic.activations_device(m, ks[i], synthetic.ACT_SEED + 10 + i, device=device)
                   for i in range(3)]
        self.ws = [torch.empty(max(binding.a8w4_ws_bytes(m, ks[i]), 1), dtype=torch.uint8, device=device)
                   for i in range(3)]
        self.ys = [torch.empty((m, n), dtype=torch.float16, device=device)
                   for (_, _, n) in synthetic.LAYER_PROJECTIONS]
        self.int_ops = 2 * m * len(self.layers) * sum(k * n for _, k, n in synthetic.LAYER_PROJECTIONS)

    def run(self, layers=None):
        """Enqueue the pass (or the given layer indices) on the current stream."""
        names = [p[0] for p in synthetic.LAYER_PROJECTIONS]
        for layer in (range(len(self.layers)) if layers is None else layers):
            done = set()
            for pi, name in enumerate(names):
                i = _INPUT_OF[name]
                if i not in done:           # quantize this layer's input once
                    binding.a8w4_prepare(self.xs[i], self.ws[i])
                    done.add(i)
                codes, scales = self.layers[layer][pi]
                _, k, _ = synthetic.LAYER_PROJECTIONS[pi]
                binding.a8w4_gemm_prepared(self.ws[i], self.m, k, codes, scales, self.ys[pi])
