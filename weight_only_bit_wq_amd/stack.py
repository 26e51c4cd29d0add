"""The mixed-bit 64-layer stack with an 8-bit vocabulary head, on the device.

Depth-tiered allocation from the model card "Qwen3.8-27B-INT6-Mixed-AutoRound"
(Layout: the 20 edge layers 0-9 and 54-63 vs the 44 middle layers): b = 7 on
the edge layers, 5 / 6 alternating in the middle (synth.layer_bits).  Each
layer is an up projection (K 5120 -> N 17408) then a down projection
(K 17408 -> N 5120), chained with no nonlinearity; the head is an 8-bit
[248320 x 5120] layer ("vLLM Can Run INT5-7", section 3: INT8 vocabulary
layers, vocabulary 248,320, hidden 5,120).

Every layer's weights sit in their own device memory (the body is ~8.7 GB,
the head ~1.3 GB), so a forward pass streams all of them from HBM.  Weight
contents come from one seeded set per (bit width, projection) and are copied
per layer on the device (synthetic weights; distinct addresses are what
matter for the memory system).  All arithmetic runs in wq_gemm.
"""
from __future__ import annotations

import numpy as np

from . import synth


class DeviceLayer:
    def __init__(self, blob, b: int, N: int, K: int):
        self.blob, self.b, self.N, self.K = blob, b, N, K

    def bytes(self, M: int) -> int:
        return self.N * (self.K * self.b // 32) * 4 + self.N * (self.K // 128) * 2 \
            + M * self.K * 2 + M * self.N * 2


class Stack:
    """Device weights of the stack.  `host` keeps the (codes, scales) of each
    distinct weight set, keyed (b, kind), for parity checks."""

    def __init__(self, torch, wq, n_layers: int = synth.STACK_LAYERS, keep_host: bool = False,
                 seed: int = 4):
        self.torch, self.wq = torch, wq
        self.host = {}
        proto = {}
        for b in sorted({synth.layer_bits(i, n_layers) for i in range(n_layers)}):
            for kind in ("up", "down"):
                proto[(b, kind)] = self._upload(b, kind, seed, keep_host)
        self.layers = []
        used = set()
        for i in range(n_layers):
            b = synth.layer_bits(i, n_layers)
            pair = []
            for kind in ("up", "down"):
                src = proto[(b, kind)]
                blob = src.blob.clone() if (b, kind) in used else src.blob
                used.add((b, kind))
                pair.append(DeviceLayer(blob, b, src.N, src.K))
            self.layers.append(tuple(pair))
        self.head = self._upload(8, "head", seed, keep_host)

    def _upload(self, b, kind, seed, keep_host):
        torch, wq = self.torch, self.wq
        codes, scales = synth.stack_weights(b, kind, seed)
        N, K = codes.shape
        packed = wq.wq_pack(codes, b)
        if keep_host:
            self.host[(b, kind)] = (codes, scales, packed)
        packed_d = torch.from_numpy(packed.view(np.int32)).cuda()
        scales_d = torch.from_numpy(scales.view(np.int16)).cuda().view(torch.bfloat16)
        blob = wq.wq_repack(packed_d, scales_d, K, b)
        del packed_d, scales_d
        return DeviceLayer(blob, b, N, K)

    def all_layers(self):
        for up, down in self.layers:
            yield up
            yield down
        yield self.head

    def bytes(self, M: int) -> int:
        return sum(l.bytes(M) for l in self.all_layers())

    def flops(self, M: int) -> float:
        return sum(2.0 * M * l.N * l.K for l in self.all_layers())

    def buffers(self, M: int):
        torch = self.torch
        dev = "cuda"
        h = torch.empty((M, synth.STACK_INTER), dtype=torch.bfloat16, device=dev)
        xs = [torch.empty((M, synth.STACK_HIDDEN), dtype=torch.bfloat16, device=dev)
              for _ in range(2)]
        logits = torch.empty((M, synth.STACK_VOCAB), dtype=torch.bfloat16, device=dev)
        need = max(self.wq.wq_workspace_bytes(self.wq.WQ_OP_GEMM, M, l.N, l.K, l.b)
                   for l in self.all_layers())
        ws = torch.zeros(max(need, 256), dtype=torch.uint8, device=dev)
        return h, xs, logits, ws

    def forward(self, x, bufs, record=None, record_layers=None):
        """x: bf16 [M, 5120] on the device.  Returns the logits buffer.  If
        `record` is a list, (layer index, kind, input, output) copies of the
        GEMMs of `record_layers` (all if None; the head has index n_layers)
        are appended."""
        wq = self.wq
        h, xs, logits, ws = bufs
        cur = x
        for i, (up, down) in enumerate(self.layers):
            wq.wq_gemm(cur, up.blob, wq.WQ_LAYOUT_TILED, None, up.N, up.b, Y=h, ws=ws)
            keep = record is not None and (record_layers is None or i in record_layers)
            if keep:
                record.append((i, "up", cur.clone(), h.clone()))
            nxt = xs[i & 1]
            wq.wq_gemm(h, down.blob, wq.WQ_LAYOUT_TILED, None, down.N, down.b, Y=nxt, ws=ws)
            if keep:
                record.append((i, "down", h.clone(), nxt.clone()))
            cur = nxt
        wq.wq_gemm(cur, self.head.blob, wq.WQ_LAYOUT_TILED, None, self.head.N, 8, Y=logits, ws=ws)
        if record is not None and (record_layers is None or len(self.layers) in record_layers):
            record.append((len(self.layers), "head", cur.clone(), logits.clone()))
        return logits
