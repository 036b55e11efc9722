"""The five workloads the library is checked and measured on.

Each workload is a frozen description: token count, hidden size, expert
layout, routing distribution, the synthetic expert stage that stands in for
the experts between dispatch and combine, and which combine is run.

Symbols follow the problem statement of the FlashInfer one-sided all-to-all
as the InferenceX/CollectiveX PR describes it ("The adapter" table: a padded
receive of shape [ep_size, runtime_max_tokens_per_rank, hidden]; the
workspace sized once from the ladder maximum; each call passes its rung):

  T    tokens in the call            H    hidden size (bf16 elements)
  E    experts  (E = ep * epr)       k    top-k experts per token
  ep   destination regions           epr  experts per region
  cap  allocated rows per region     R    runtime rung (bound on T)

`cap` is None where the workload sizes it from the routing it draws (the
skewed workload: "sized to the worst region's count").
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional


@dataclass(frozen=True)
class Workload:
    name: str
    T: int
    H: int
    E: int
    k: int
    ep: int
    cap: Optional[int]
    R: int
    routing: str          # "uniform" (distinct, uniform) or "zipf1.2" (without replacement)
    expert: str           # synthetic expert stage, see synth.inputs.expert_outputs
    combine: str          # "weighted", "unweighted", "both" or "fused"
    eps: float = 1e-6     # RMSNorm epsilon (fused workload only)

    @property
    def epr(self) -> int:
        return self.E // self.ep

    @property
    def n_items(self) -> int:
        return self.T * self.k

    def algorithmic_bytes(self) -> dict:
        """Bytes the method must move per call, padding never touched.

        dispatch : read x once, write k rows, read ids, write slot_index and
                   src_index                      = 2H(1+k) + 12k per token
        combine  : read k rows, write one row, read slot_index and weights
                                                  = 2H(k+1) + 8k per token
        fused    : combine + read residual + write residual and normed
                   + gamma once                   = 2H(k+3) + 8k per token + 2H
        """
        T, H, k = self.T, self.H, self.k
        return {
            "dispatch": T * (2 * H * (1 + k) + 12 * k),
            "combine": T * (2 * H * (k + 1) + 8 * k),
            "fused": T * (2 * H * (k + 3) + 8 * k) + 2 * H,
        }


TINY = Workload("tiny", T=64, H=128, E=8, k=2, ep=4, cap=128, R=64,
                routing="uniform", expert="identity", combine="both")
DECODE = Workload("decode", T=128, H=7168, E=256, k=8, ep=8, cap=1024, R=128,
                  routing="uniform", expert="scale_by_expert", combine="weighted")
PREFILL = Workload("prefill", T=4096, H=7168, E=256, k=8, ep=8, cap=32768, R=4096,
                   routing="uniform", expert="scale_by_expert_times_weight",
                   combine="unweighted")
SKEWED = Workload("skewed", T=8192, H=7168, E=256, k=8, ep=16, cap=None, R=8192,
                  routing="zipf1.2", expert="scale_by_expert", combine="weighted")
FUSED = Workload("fused", T=2048, H=7168, E=256, k=8, ep=8, cap=16384, R=2048,
                 routing="uniform", expert="gaussian", combine="fused")

ALL = (TINY, DECODE, PREFILL, SKEWED, FUSED)
BY_NAME = {w.name: w for w in ALL}


@dataclass(frozen=True)
class PartialsWorkload:
    """The local reduction of a tensor-parallel all-reduce fused with the
    residual add and RMSNorm: P ranks' partial hidden states [P, T, H] sit in
    local memory and are summed once, then normalised."""
    name: str
    P: int
    T: int
    H: int
    eps: float = 1e-6

    def algorithmic_bytes(self) -> dict:
        """reduce: read P rows, write one = 2H(P+1) per token;
        fused : read P rows and the residual, write residual and normed,
                gamma once                  = 2H(P+3) per token + 2H"""
        T, H, P = self.T, self.H, self.P
        return {"reduce": T * 2 * H * (P + 1), "fused": T * 2 * H * (P + 3) + 2 * H}


# eight tensor-parallel ranks, at the fused workload's token count and hidden size
PARTIALS = PartialsWorkload("partials", P=8, T=2048, H=7168)
