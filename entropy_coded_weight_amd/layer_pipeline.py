"""Decode/compute overlap: layer-by-layer decoding into two bf16 layer
buffers, the decode of layer l+1 running on its own stream while the
consumer's work on layer l runs on another.

Weights stay compressed in device memory and are expanded right before the
block that uses them [EntQuant, "Float8@2bits ...", technical summary §2
"Decodificación en Tiempo de Inferencia"]; the pages interleave the
decompression with the forward kernels [EntQuant, technical summary §2] and
decode one transformer block's matrices as one batch [DFloat11 write-up,
"Descompresión por bloque transformer"]. Here each layer's batch is one
``entq_decode`` launch; what overlaps it is whatever the consumer enqueues
for the previous layer.

Ordering (HIP events, no host waits inside a pass):
  decoded[b]  -- recorded on the decode stream after layer l's decode into
                 buffer b = l % 2; the compute stream waits for it before
                 running the consumer on buffer b;
  consumed[b] -- recorded on the compute stream after the consumer's work on
                 buffer b; the decode stream waits for it before decoding
                 layer l + 2 into the same buffer.
"""
from __future__ import annotations

from . import OUT_BF16, decode


class LayerPipeline:
    """Two layer buffers and two streams over a list of compressed layers.

    layers: list of (plan, blob, scales) -- one ``entq_plan`` per layer, its
    compressed bytes (device uint8) and per-row scales (device float32).
    out_elems: decoded elements per layer (the buffer size)."""

    def __init__(self, layers, out_elems: int, device, decode_stream=None, compute_stream=None):
        import torch
        self.layers = layers
        self.device = torch.device(device)
        # int16 storage holding bf16 bit patterns (the decode writes them);
        # consumers view them as bfloat16
        self.buffers = [torch.empty(out_elems, dtype=torch.int16, device=self.device)
                        for _ in range(2)]
        self.decode_stream = decode_stream or torch.cuda.Stream(self.device)
        self.compute_stream = compute_stream or torch.cuda.Stream(self.device)
        # the plans' workspace uploads and the blobs' copies were enqueued on
        # the current stream: order both streams after them
        here = torch.cuda.current_stream(self.device)
        self.decode_stream.wait_stream(here)
        self.compute_stream.wait_stream(here)
        # the buffers are used on both streams: their memory is not handed out
        # again before the work queued there has finished
        for buf in self.buffers:
            buf.record_stream(self.decode_stream)
            buf.record_stream(self.compute_stream)
        self.decoded = [torch.cuda.Event() for _ in range(2)]
        self.consumed = [torch.cuda.Event() for _ in range(2)]

    def weights(self, b: int):
        """Buffer b as bfloat16."""
        import torch
        return self.buffers[b].view(torch.bfloat16)

    def _decode(self, layer: int, b: int):
        plan, blob, scales = self.layers[layer]
        decode(plan, blob, self.buffers[b], OUT_BF16, scales, None, self.decode_stream)

    def run_overlapped(self, consume, n_layers: int | None = None):
        """Enqueues one pass over the layers. consume(layer, weights) is
        called with the compute stream current and enqueues the layer's
        work there. Returns without waiting; the pass ends on the compute
        stream."""
        import torch
        n = len(self.layers) if n_layers is None else n_layers
        sd, sc = self.decode_stream, self.compute_stream
        # the previous pass's consumers may still read both buffers
        sd.wait_stream(sc)
        if n == 0:
            return
        with torch.cuda.stream(sd):
            self._decode(0, 0)
            self.decoded[0].record(sd)
        for layer in range(n):
            b = layer % 2
            if layer + 1 < n:
                nb = 1 - b
                with torch.cuda.stream(sd):
                    if layer >= 1:
                        sd.wait_event(self.consumed[nb])
                    self._decode(layer + 1, nb)
                    self.decoded[nb].record(sd)
            with torch.cuda.stream(sc):
                sc.wait_event(self.decoded[b])
                consume(layer, self.weights(b))
                self.consumed[b].record(sc)

    def run_serial(self, consume, n_layers: int | None = None):
        """The same work on one stream (the compute stream): decode layer l,
        then its consumer, then layer l + 1. The reference schedule."""
        import torch
        n = len(self.layers) if n_layers is None else n_layers
        sc = self.compute_stream
        with torch.cuda.stream(sc):
            for layer in range(n):
                b = layer % 2
                plan, blob, scales = self.layers[layer]
                decode(plan, blob, self.buffers[b], OUT_BF16, scales, None, sc)
                consume(layer, self.weights(b))
