"""The five synthetic workloads and their per-level budgets.

The workloads take the layer shape of LLaDA-8B-Instruct (32 MHA heads,
head dim 128), the model the WaveFilter pages evaluate (section 1,
Figure 1), and prompt lengths from 1K to 128K tokens.  Each names the number
of Haar levels L and the final prompt-token budget; some also name the
coarse Top-K.  The pages give no per-level budgets (their section 3.2 and
appendix are not part of the text), so the integers k_L .. k_0 are resolved
here once by a fixed rule and handed unchanged to both the oracle and the
library.

This module holds configuration only; it computes nothing of the method.
"""

from dataclasses import dataclass, replace
import math


@dataclass(frozen=True)
class Config:
    cid: int            # 1..5
    name: str
    layers: int
    batch: int
    heads: int
    head_dim: int
    dtype: str          # "f32" or "bf16"
    n_q: int            # query-block rows
    n_prompt: int       # N_p
    n_gen: int          # N_g
    levels: int         # Haar levels L
    final_budget: int   # prompt tokens to attend (upper bound, see resolve_budgets)
    coarse_k: int       # explicit coarse Top-K, or 0 when the rule picks it
    n_spans: int        # planted spans per head
    span_len: tuple     # (lo, hi) inclusive
    alpha: float        # planted key = alpha * mean(query) + noise * N(0, 1)
    noise: float
    key_law: str        # "normal" or "student_t4"

    @property
    def n_tot(self):
        return self.n_prompt + self.n_gen

    @property
    def budgets(self):
        return resolve_budgets(self.n_prompt, self.levels, self.final_budget, self.coarse_k)


CONFIGS = {
    1: Config(1, "tiny-1k-f32", 1, 1, 2, 64, "f32", 32, 1024, 32, 3, 64, 8,
              1, (16, 16), 3.0, 0.1, "normal"),
    2: Config(2, "llada-4k", 1, 1, 32, 128, "bf16", 32, 4096, 256, 4, 512, 0,
              2, (32, 32), 2.5, 0.1, "normal"),
    3: Config(3, "llada-16k", 1, 1, 32, 128, "bf16", 32, 16384, 256, 5, 1024, 16,
              4, (32, 32), 2.5, 0.1, "normal"),
    4: Config(4, "llada-64k", 1, 1, 32, 128, "bf16", 64, 65536, 512, 6, 2048, 0,
              8, (16, 64), 2.5, 0.1, "student_t4"),
    5: Config(5, "llada-128k-32layer-b2", 32, 2, 32, 128, "bf16", 32, 131072, 512, 7, 4096, 0,
              16, (32, 32), 2.5, 0.1, "normal"),
}


# The 16K workload names both a coarse Top-K of 16 and a final budget of
# 1 024, which 16 regions of 32 tokens cannot reach.  Two readings:
#   "capped": the coarse Top-K is honoured and the final budget is a cap
#             (k_0 = 512), the default;
#   "full":   the coarse Top-K is dropped and the default rule picks
#             k_L = 64, so that k_0 = 1 024 is reached.
# Both run on the same inputs (same workload id, same seeds); every result
# names the reading it used.
C3_READINGS = {
    "capped": CONFIGS[3],
    "full": replace(CONFIGS[3], name="llada-16k-full-budget", coarse_k=0),
}


def budget_reading(cfg):
    """The reading of the 16K workload's budgets that ``cfg`` uses, or None
    for the other workloads."""
    if cfg.cid != 3:
        return None
    return "full" if cfg.coarse_k == 0 else "capped"


def resolve_budgets(n_prompt, levels, final_budget, coarse_k=0):
    """Per-level keep counts ``[k_L, k_{L-1}, ..., k_0]``.

    Rule: n_j = N_p / 2^j.  k_L is the stated coarse Top-K, else
    ``min(n_L, 2 * ceil(B / 2^L))`` (twice the regions the final budget needs,
    so that refinement has something to prune).  k_0 = min(B, k_L 2^L): the
    final budget is a cap, since the kept coarse regions cover only
    k_L 2^L tokens.  In between, the number of covered tokens falls linearly
    from k_L 2^L to k_0:  k_j = ceil((k_0 L + (k_L 2^L - k_0) j) / (L 2^j)).
    """
    if levels < 0 or n_prompt % (1 << levels) != 0:
        raise ValueError("N_p must be a multiple of 2**L")
    n_top = n_prompt >> levels
    if coarse_k:
        k_top = min(coarse_k, n_top)
    else:
        k_top = min(n_top, 2 * math.ceil(final_budget / (1 << levels)))
    if levels == 0:
        return [min(final_budget, n_top)]
    k0 = min(final_budget, k_top << levels)
    out = [k_top]
    for j in range(levels - 1, 0, -1):
        num = k0 * levels + ((k_top << levels) - k0) * j
        den = levels << j
        out.append(-(-num // den))
    out.append(k0)
    return out


def check_budgets(n_prompt, levels, budgets):
    """True when the schedule is feasible: 1 <= k_L <= n_L and
    k_j <= min(2 k_{j+1}, n_j) for j < L."""
    if len(budgets) != levels + 1:
        return False
    n_top = n_prompt >> levels
    if not 1 <= budgets[0] <= n_top:
        return False
    for i in range(1, levels + 1):
        j = levels - i
        if not 1 <= budgets[i] <= min(2 * budgets[i - 1], n_prompt >> j):
            return False
    return True
