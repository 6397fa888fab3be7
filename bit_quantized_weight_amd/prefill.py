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
down) and runs the A8 GEMMs.  Gate and up read the same input, so when their
packed weights sit back to back in memory (as this class packs them) they run
as one GEMM over both: y = [gate | up] in one [M, 2 x 17408] output, of which
the per-projection outputs are views.  Inputs are synthetic and the same for
every layer, but every layer quantizes them again, as a model's would change;
the projections do not feed each other, so the pass measures the A8 route
alone.  Outputs are overwritten layer after layer.
"""

from . import binding, synthetic

# index of each projection's input among the three per-layer inputs
_INPUT_OF = {"qkv": 0, "out": 1, "gate": 0, "up": 0, "down": 2}
_NAMES = [p[0] for p in synthetic.LAYER_PROJECTIONS]
_GATE, _UP = _NAMES.index("gate"), _NAMES.index("up")


def _adjacent(a, b):
    """b starts where a ends (a and b contiguous, same dtype and row length)."""
    return (a.is_contiguous() and b.is_contiguous() and a.dtype == b.dtype and a.shape[1:] == b.shape[1:]
            and b.data_ptr() == a.data_ptr() + a.numel() * a.element_size())


class PrefillPass:
    """Packed weights of all layers (or given ones), the three activation
    inputs, their A8 workspaces and one output per projection."""

    def __init__(self, m, layers=synthetic.N_LAYERS, device="cuda", weights=None, keep_rows=None):
        """weights: optional per-layer [(codes, scales)] in LAYER_PROJECTIONS
        order (e.g. another PrefillPass's ``layers``); else generated here,
        with each layer's gate and up weights packed back to back.
        keep_rows: {(layer, proj_index): row indices} whose fp32 weight rows
        are copied to the host for spot checks."""
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
                # gate and up in one allocation each for codes and scales
                (cg, sg), (cu, su) = projs[_GATE], projs[_UP]
                codes, scales = torch.cat([cg, cu]), torch.cat([sg, su])
                n = cg.shape[0]
                projs[_GATE] = (codes[:n], scales[:n])
                projs[_UP] = (codes[n:], scales[n:])
                del cg, sg, cu, su
                weights.append(projs)
        self.layers = weights[:layers]
        # per layer: the gate|up pair as one matmul, when the weights allow it
        self.fused = []
        for projs in self.layers:
            (cg, sg), (cu, su) = projs[_GATE], projs[_UP]
            if _adjacent(cg, cu) and _adjacent(sg, su):
                n2 = cg.shape[0] + cu.shape[0]
                self.fused.append((cg.as_strided((n2, cg.shape[1]), cg.stride()),
                                   sg.as_strided((n2, sg.shape[1]), sg.stride())))
            else:
                self.fused.append(None)
        ks = {}
        for name, k, _ in synthetic.LAYER_PROJECTIONS:
            ks[_INPUT_OF[name]] = k
        self.xs = [synthetic.activations_device(m, ks[i], synthetic.ACT_SEED + 10 + i, device=device)
                   for i in range(3)]
        self.ws = [torch.empty(max(binding.a8w4_ws_bytes(m, ks[i]), 1), dtype=torch.uint8, device=device)
                   for i in range(3)]
        ns = [n for (_, _, n) in synthetic.LAYER_PROJECTIONS]
        self.y_gate_up = torch.empty((m, ns[_GATE] + ns[_UP]), dtype=torch.float16, device=device)
        self.ys = [torch.empty((m, n), dtype=torch.float16, device=device) for n in ns]
        self.int_ops = 2 * m * len(self.layers) * sum(k * n for _, k, n in synthetic.LAYER_PROJECTIONS)

    def output(self, layer, pi):
        """The output of projection pi as the given layer's run left it."""
        if pi in (_GATE, _UP) and self.fused[layer] is not None:
            n = self.ys[_GATE].shape[1]
            return self.y_gate_up[:, :n] if pi == _GATE else self.y_gate_up[:, n:]
        return self.ys[pi]

    def run(self, layers=None):
        """Enqueue the pass (or the given layer indices) on the current stream."""
        for layer in (range(len(self.layers)) if layers is None else layers):
            done = set()
            for pi, name in enumerate(_NAMES):
                fused = self.fused[layer]
                if fused is not None and pi == _UP:
                    continue                      # ran with gate
                i = _INPUT_OF[name]
                if i not in done:                 # quantize this layer's input once
                    binding.a8w4_prepare(self.xs[i], self.ws[i])
                    done.add(i)
                _, k, _ = synthetic.LAYER_PROJECTIONS[pi]
                if fused is not None and pi == _GATE:
                    binding.a8w4_gemm_prepared(self.ws[i], self.m, k, fused[0], fused[1], self.y_gate_up)
                else:
                    codes, scales = self.layers[layer][pi]
                    binding.a8w4_gemm_prepared(self.ws[i], self.m, k, codes, scales, self.ys[pi])
