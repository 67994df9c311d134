"""Workload configurations of the routed-expert MoE layer (sizes only)."""
from dataclasses import dataclass, field, replace
from typing import Tuple


def record_bytes(fmt: str, d: int, f: int) -> int:
    """Bytes of one complete layer-expert record (all banks of gate, up, down)."""
    if fmt == "bf16":
        return 3 * d * f * 2
    if fmt == "fp8":
        return 3 * d * f + 3 * (d // 128) * (f // 128) * 4
    if fmt == "mxfp4":
        return 3 * d * f // 2 + 3 * d * f // 32
    raise ValueError(fmt)


@dataclass(frozen=True)
class MoEConfig:
    name: str
    cfg_id: int          # seed-key component
    layers: int          # MoE layers in the host bank
    d: int               # hidden size
    E: int               # experts per layer
    k: int               # routed experts per token
    f: int               # expert FFN width
    fmt: str             # 'bf16' | 'fp8' | 'mxfp4'
    slots: int           # slot-cache capacity N (complete records)
    bp_mbps: int         # profiled host->GPU fill bandwidth, MB/s
    bh_mbps: int         # profiled host expert-execution bandwidth, MB/s
    tokens: Tuple[int, ...] = (1,)   # tokens per call (one entry per sub-run)
    steps: Tuple[int, ...] = (1,)    # calls per layer for each sub-run
    max_fetch: int = -1
    seed: int = 0
    layer_alias: int = 0  # >0: layer l's weights are layer (l mod alias)'s (flat ids stay distinct)
    stream_layers: int = 0  # layers streamed through the double buffer

    @property
    def S(self) -> int:
        return record_bytes(self.fmt, self.d, self.f)

    def with_(self, **kw) -> "MoEConfig":
        return replace(self, **kw)


CONFIGS = {
    # One MoE layer, 16 tokens, 8 experts top-2, 4 slots, B_P/B_H 25/50 GB/s.
    "tiny": MoEConfig("tiny", 1, layers=1, d=256, E=8, k=2, f=128, fmt="bf16", slots=4,
                      bp_mbps=25000, bh_mbps=50000, tokens=(16,), steps=(1,)),
    # Decode: 48 layers, 1 token per step for 256 steps, 1024 of 6144 layer-experts cached.
    "decode": MoEConfig("decode", 2, layers=48, d=2048, E=128, k=8, f=768, fmt="bf16", slots=1024,
                        bp_mbps=20000, bh_mbps=60000, tokens=(1,), steps=(256,)),
    # Prefill chunk: one layer of 8192 tokens; the stream variant passes 24 layers
    # through two full-layer buffers (slots = 2E).
    "prefill": MoEConfig("prefill", 3, layers=24, d=2048, E=128, k=8, f=768, fmt="bf16", slots=256,
                         bp_mbps=20000, bh_mbps=60000, tokens=(8192,), steps=(1,), stream_layers=24),
    # Block-FP8 experts, token batches 1 / 64 / 2048, 64 slots, Zipf(1.1) expert popularity.
    "fp8": MoEConfig("fp8", 4, layers=1, d=4096, E=256, k=8, f=2048, fmt="fp8", slots=64,
                     bp_mbps=20000, bh_mbps=60000, tokens=(1, 64, 2048), steps=(256, 256, 16)),
    # MXFP4 experts, 61 layers; slots sized to 60% of 288e9 bytes of HBM.
    "mxfp4": MoEConfig("mxfp4", 5, layers=61, d=7168, E=256, k=8, f=2048, fmt="mxfp4",
                       slots=int(0.6 * 288e9) // record_bytes("mxfp4", 7168, 2048),
                       bp_mbps=20000, bh_mbps=60000, tokens=(4096, 1), steps=(1, 128),
                       stream_layers=61),
}
