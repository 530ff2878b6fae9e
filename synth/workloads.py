"""The synthetic workloads: shapes, dtypes, distributions and seeds.

Shapes follow the MoE decode stacks this project measures: a tiny fp32 stack
for exact checks, a 16-layer MoE-only bf16 stack (batch 1 and 8), and a
92-layer stack with GQA attention over a 4096-position bf16 KV cache (batch 1
and 8, plus a speculative-verify pass of 8 rows per sequence).  The pages
describe such a model only in outline (92 MoE layers, attention then MoE per
layer, a KV cache; P3 "TPU Megakernel Achieves 709 tokens/s on Kimi K3"
sections "The Key Innovation..." and "Cross-Layer Weight Prefetching", P2
section "同样 16 块芯片，TPU 快 57%" for batch 1/8 and speculative decoding with
acceptance length 6); every value here is synthetic.

Distributions: weights N(0, 0.02) rounded to the stack dtype; RMSNorm gains
U(0.9, 1.1); router bias N(0, 0.5) fp32 where present; hidden rows N(0, 1)
fp32; KV cache N(0, 1) bf16 for the past positions.
"""
from dataclasses import dataclass, replace

from . import BF16, F32


@dataclass(frozen=True)
class Workload:
    name: str
    L: int
    d: int
    E: int
    k: int
    F: int
    n_shared: int
    dtype: int
    router_bias: bool
    has_attn: bool
    H: int = 0
    G: int = 0
    hd: int = 0
    rope_theta: float = 1e6
    past: int = 0            # cached positions 0..past-1 per sequence
    M: int = 1               # rows per step
    rows_per_seq: int = 1
    weight_seed: int = 0
    input_seed: int = 0
    steps: int = 1
    cap_extra: int = 64       # KV capacity beyond past + rows_per_seq (room for more steps)
    rms_eps: float = 1e-6
    weight_std: float = 0.02
    bias_std: float = 0.5

    @property
    def n_seq(self) -> int:
        return self.M // self.rows_per_seq

    @property
    def capacity(self) -> int:
        # room for the step's new rows plus a few more steps of growth
        return self.past + self.rows_per_seq + self.cap_extra if self.has_attn else 0

    def positions(self, step: int = 0):
        """Row r of sequence s sits at past + step*rows_per_seq + (r % rows_per_seq)."""
        return [self.past + step * self.rows_per_seq + (r % self.rows_per_seq) for r in range(self.M)]

    def with_(self, **kw):
        return replace(self, **kw)


TINY = Workload("tiny_fp32_b1", L=2, d=256, E=8, k=2, F=512, n_shared=0, dtype=F32, router_bias=False,
                has_attn=False, M=1, weight_seed=0, input_seed=0, steps=1)
MOE16_B1 = Workload("moe16_b1", L=16, d=2048, E=64, k=6, F=1024, n_shared=1, dtype=BF16, router_bias=True,
                    has_attn=False, M=1, weight_seed=1, input_seed=1, steps=256)
MOE16_B8 = MOE16_B1.with_(name="moe16_b8", M=8, input_seed=2)
ATTN92_B1 = Workload("attn92_b1", L=92, d=4096, E=64, k=8, F=1024, n_shared=1, dtype=BF16, router_bias=False,
                     has_attn=True, H=32, G=8, hd=128, rope_theta=1e6, past=4096, M=1, weight_seed=3,
                     input_seed=3, steps=20)
ATTN92_B8 = ATTN92_B1.with_(name="attn92_b8", M=8)
VERIFY92_M8 = ATTN92_B1.with_(name="verify92_m8", M=8, rows_per_seq=8, input_seed=4)
VERIFY92_M64 = ATTN92_B1.with_(name="verify92_m64", M=64, rows_per_seq=8, input_seed=4)

ALL = {w.name: w for w in (TINY, MOE16_B1, MOE16_B8, ATTN92_B1, ATTN92_B8, VERIFY92_M8, VERIFY92_M64)}


def weight_bytes_per_layer(w: Workload) -> int:
    es = 2 if w.dtype == BF16 else 4
    b = 3 * w.d * w.F * es * (w.E + w.n_shared) + w.d * w.E * es
    if w.has_attn:
        b += (2 * w.d * w.H * w.hd + 2 * w.d * w.G * w.hd) * es
    return b
