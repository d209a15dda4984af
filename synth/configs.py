"""Workload shapes of the routed MoE layer, as the pages describe the models.

Shapes only: no arithmetic of the method lives here.  Each entry names the model
the shape comes from and the page that gives it:

* ``xing4``  -- PocketLLM, "Xing4.0-29B-A4B", section "Overview", model table:
  hidden 3,584; 64 routed experts activated top-4 plus one shared; expert_ffn 1,024;
  sigmoid-routed MoE with a shared expert; 38 of the 40 blocks are MoE blocks
  (blocks 0-1 are dense, section "Overview", "Dense blocks").
* ``qwen3next_like`` -- Red Lite, "What we learned", section "1. The idea": 48 layers,
  each a mixture of 512 experts of which a token uses 10.  Hidden 2,048 and expert FFN 512
  are a synthetic shape of that family (the page does not print them).
* ``dsv41_like`` -- "DeepSeek-V4.1-Flash at 27 Tokens/s on One RTX 4090", section
  "Why build an engine at all": 384 experts per layer, 6 picked per token.  Hidden 7,168 and
  expert FFN 1,536 are a synthetic shape.

Token counts: decode batches of 1 / 2 / 16 tokens; prefill chunks of 2,048 tokens (Red Lite,
"3. Speed by release", 2048-token chunks) and 8,192 tokens.
"""
from dataclasses import dataclass, field, asdict
from typing import Optional, Tuple

SIGMOID = 0
SOFTMAX = 1


@dataclass(frozen=True)
class LayerShape:
    hidden: int
    ffn: int
    n_experts: int
    top_k: int
    n_shared: int
    gating: int          # SIGMOID or SOFTMAX
    renormalize: int     # 1: selected weights divided by their sum

    @property
    def blocks_h(self) -> int:
        return self.hidden // 32

    @property
    def blocks_f(self) -> int:
        return self.ffn // 32

    # IQ4_NL: 18 bytes per 32 weights.
    @property
    def gate_bytes(self) -> int:
        return self.ffn * self.blocks_h * 18

    @property
    def down_bytes(self) -> int:
        return self.hidden * self.blocks_f * 18

    @property
    def expert_bytes(self) -> int:
        return 2 * self.gate_bytes + self.down_bytes

    @property
    def bank_bytes(self) -> int:
        return (self.n_experts + self.n_shared) * self.expert_bytes


@dataclass(frozen=True)
class Workload:
    name: str
    cfg_id: int                  # selects the generator stream family
    shape: LayerShape
    layers: int                  # chained layers for decode
    decode_tokens: Tuple[int, ...] = ()
    prefill_tokens: Tuple[int, ...] = ()
    zipf_s: Optional[float] = None   # router-bias skew exponent (None: no bias)
    weight_sigma: float = 0.02
    router_sigma: float = 0.02
    x_sigma: float = 1.0
    seed: int = 0


TINY = Workload(
    name="tiny", cfg_id=1,
    shape=LayerShape(hidden=256, ffn=128, n_experts=8, top_k=2, n_shared=1,
                     gating=SIGMOID, renormalize=1),
    layers=1, decode_tokens=(4,), prefill_tokens=(4,))

XING4_DECODE = Workload(
    name="xing4_decode", cfg_id=2,
    shape=LayerShape(hidden=3584, ffn=1024, n_experts=64, top_k=4, n_shared=1,
                     gating=SIGMOID, renormalize=1),
    layers=38, decode_tokens=(1, 16))

XING4_PREFILL = Workload(
    name="xing4_prefill", cfg_id=3,
    shape=XING4_DECODE.shape, layers=1, prefill_tokens=(2048,), zipf_s=1.1)

QWEN3NEXT_LIKE = Workload(
    name="qwen3next_like", cfg_id=4,
    shape=LayerShape(hidden=2048, ffn=512, n_experts=512, top_k=10, n_shared=1,
                     gating=SOFTMAX, renormalize=0),
    layers=48, decode_tokens=(1, 2), prefill_tokens=(2048,))

DSV41_LIKE = Workload(
    name="dsv41_like", cfg_id=5,
    shape=LayerShape(hidden=7168, ffn=1536, n_experts=384, top_k=6, n_shared=1,
                     gating=SIGMOID, renormalize=1),
    layers=1, decode_tokens=(16,), prefill_tokens=(8192,), zipf_s=1.1)

WORKLOADS = {w.name: w for w in (TINY, XING4_DECODE, XING4_PREFILL, QWEN3NEXT_LIKE, DSV41_LIKE)}
