"""The five synthetic MoE-layer workloads, with every size and seed fixed.

Each workload is one MoE layer forward + backward on one GPU.  Shapes follow
the layer statement: tokens x[T,d], gate Wg[d,E], experts W1[E,d,f],
W2[E,f,d] (and W3[E,d,f] for SwiGLU experts), top-k routing.

The pages name model families (FairSeq MoE-S/M/L in the ES-MoE review,
section 五 实验结果; MoE-GPT3/MoE-BERT on the MPipeMoE page, 研究成果; a
96-expert GPT on the FastMoE review, 주요 결과) but print no layer shapes and
ship no data, so seeded synthetic tensors of these shapes stand in for them.

Routing skew: a per-expert logit bias b_e = -alpha * s * ln(rank_e), where
rank is a seeded permutation of 1..E, makes expert popularity roughly
Zipf(s).  alpha was calibrated once per workload so that the routed load
lands in the band each workload asks for (heaviest expert about 4x the mean
for the 16-expert workload; some empty and some >1000-row experts for the
64-expert one); the calibration outcome is asserted by the CPU tests.
"""
from dataclasses import dataclass
from typing import Optional


@dataclass(frozen=True)
class MoEConfig:
    name: str
    T: int          # tokens
    d: int          # model width
    f: int          # expert hidden width
    E: int          # experts
    k: int          # experts per token
    act: str        # "gelu" or "swiglu"
    dtype: str      # "f32" or "bf16": storage type of every tensor the layer reads/writes
    zipf_s: Optional[float] = None   # routing skew exponent (None: no bias)
    alpha: float = 0.0               # bias scale, see module docstring
    renorm: int = 1                  # softmax renormalised over the selected k
    seed: int = 0

    @property
    def R(self) -> int:
        """Routed rows T*k."""
        return self.T * self.k

    @property
    def swiglu(self) -> bool:
        return self.act == "swiglu"

    def gemm_flops_fwd_bwd(self) -> float:
        """Algorithmic grouped-GEMM FLOPs of one layer forward+backward.

        GeLU experts: 2 GEMMs forward (x W1, a W2), 4 backward (dA, dW2, dW1,
        dX), each 2*R*d*f.  SwiGLU adds x W3 forward and dW3 plus the second
        half of dX backward: 9 products of 2*R*d*f.
        """
        per = 2.0 * self.R * self.d * self.f
        return per * (9 if self.swiglu else 6)

    def short(self) -> str:
        return (f"T{self.T}_d{self.d}_f{self.f}_E{self.E}_k{self.k}_"
                f"{self.act}_{self.dtype}")


TINY_F32 = MoEConfig("tiny_fp32", T=256, d=64, f=256, E=4, k=1, act="gelu",
                     dtype="f32")
MOE_S_LIKE = MoEConfig("moe_s_like", T=8192, d=1024, f=4096, E=8, k=2,
                       act="gelu", dtype="bf16")
SKEWED = MoEConfig("skewed_zipf1.2", T=16384, d=2048, f=8192, E=16, k=2,
                   act="gelu", dtype="bf16", zipf_s=1.2, alpha=0.55)
MANY_EXPERT = MoEConfig("many_expert_zipf1.0", T=32768, d=1024, f=4096, E=64,
                        k=2, act="gelu", dtype="bf16", zipf_s=1.0, alpha=1.2)
LONG_CTX = MoEConfig("long_ctx_swiglu", T=65536, d=4096, f=14336, E=128, k=8,
                     act="swiglu", dtype="bf16", zipf_s=0.8, alpha=1.0)

CONFIGS = {c.name: c for c in (TINY_F32, MOE_S_LIKE, SKEWED, MANY_EXPERT,
                                LONG_CTX)}
ORDER = [TINY_F32.name, MOE_S_LIKE.name, SKEWED.name, MANY_EXPERT.name,
         LONG_CTX.name]


def small_variant(name: str, **kw) -> MoEConfig:
    """A copy of a workload with some fields replaced (tests use this)."""
    from dataclasses import replace
    return replace(CONFIGS[name], **kw)
