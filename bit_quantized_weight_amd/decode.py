"""Full decode-step weight pass: every projection of a 64-layer dense decoder
streamed once through the skinny matmul, back to back on one stream.

The pages' model streams all of its quantized weights once per decode step
(page 3, "Qwen3.8-27B at 256K on a 24GB RTX PRO 4000 SFF", the paragraph on
weight streaming during decode); with speculative verification the step
carries M = 1 + drafted tokens rows.  Layer widths: hidden 5120, FFN 17408,
per layer qkv 5120 -> 7168, out 5120 -> 5120, gate and up 5120 -> 17408 and
down 17408 -> 5120.  Weights are synthetic (seeded) and packed on the GPU.

The projections of a step are independent here (each reads its own input
buffer), so the pass measures the weight stream itself; a model would chain
them through its mixers.  ``run`` issues one skinny matmul per projection;
``run_batched`` computes the same outputs with one persistent launch over
all of them (planned once by ``plan_batched``).
"""

from . import binding, synthetic


class DecodeStep:
    """Packed weights of all layers plus the per-projection activation/output buffers."""

    def __init__(self, m, layers=synthetic.N_LAYERS, device="cuda", keep_rows=None, weights=None):
        """keep_rows: optional {(layer, proj_index): row_index_array} whose fp32
        weight rows are copied to the host before the fp32 matrix is freed
        (for spot checks against a CPU reference).  weights: optional packed
        per-layer [(codes, scales)] in LAYER_PROJECTIONS order, e.g. another
        DecodeStep's ``layers`` (the same weights at another M)."""
        import torch
        self.m = m
        self.layers = []
        self.kept = {}
        self.weight_bytes = 0
        for layer in range(layers):
            projs = []
            for pi, (_, k, n) in enumerate(synthetic.LAYER_PROJECTIONS):
                if weights is not None:
                    projs.append(weights[layer][pi])
                else:
                    w = synthetic.weights_device(n, k, synthetic.layer_weight_seed(layer, pi), device=device)
                    if keep_rows and (layer, pi) in keep_rows:
                        idx = torch.as_tensor(keep_rows[(layer, pi)], device=device)
                        self.kept[(layer, pi)] = w.index_select(0, idx).cpu().numpy()
                    projs.append(binding.pack(w))
                    del w
                self.weight_bytes += n * k * 9 // 16
            self.layers.append(projs)
        self.xs = [synthetic.activations_device(m, k, synthetic.ACT_SEED + pi, device=device)
                   for pi, (_, k, _) in enumerate(synthetic.LAYER_PROJECTIONS)]
        self.ys = [[torch.empty((m, n), dtype=torch.float16, device=device)
                    for (_, _, n) in synthetic.LAYER_PROJECTIONS] for _ in range(layers)]
        nbytes = max(binding.gemv_ws_bytes(m, n, k, 0) for _, k, n in synthetic.LAYER_PROJECTIONS)
        self.ws = torch.zeros(max(nbytes, 1), dtype=torch.uint8, device=device)
        self.io_bytes = layers * sum(2 * m * k + 2 * m * n for _, k, n in synthetic.LAYER_PROJECTIONS)
        self.batch = None

    @property
    def launches(self):
        return len(self.layers) * len(synthetic.LAYER_PROJECTIONS)

    def run(self):
        """Enqueue one decode step (one skinny GEMV per projection) on the current stream."""
        for layer, projs in enumerate(self.layers):
            for pi, (codes, scales) in enumerate(projs):
                binding.q4_gemv_skinny_raw(self.xs[pi], codes, scales, self.ys[layer][pi], 0, self.ws)

    def plan_batched(self):
        """Plan every projection of the step as one batch (a blocking set-up call)."""
        items = [(self.xs[pi], codes, scales, self.ys[layer][pi])
                 for layer, projs in enumerate(self.layers)
                 for pi, (codes, scales) in enumerate(projs)]
        self.batch = binding.batched_plan(items)
        return self.batch

    def run_batched(self):
        """Enqueue the whole step as one persistent launch on the current stream."""
        if self.batch is None:
            self.plan_batched()
        self.batch.run()
