"""Workload shapes of the decode path (sizes only, no arithmetic).

Shapes follow the pages' examples: the 27B specimen of "Interconnects e
clusters" (lesson 9.9, section 01 · Conceito: hidden 5120, 64 layers with two
reconciliation points each, tensor parallel degree 2 or 4), a hidden-4096
model split 4 or 8 ways ("8x B200 и GLM-5.2", section TP=4 vs TP=8), and an
expert-parallel MoE decode share with 128 experts and top-8 routing
("Hosting Qwen on Blackwell", sections Prefillers and Expert Parallel).
"""
from __future__ import annotations

from dataclasses import dataclass, replace


@dataclass(frozen=True)
class Workload:
    name: str
    hidden: int          # H
    inter: int           # FFN intermediate I (K of the down projection)
    k_attn: int          # K of the mixer output projection
    n_ranks: int         # N virtual ranks
    batch: int           # decode tokens b
    layers: int          # L
    # MoE share (None for dense stacks)
    n_experts: int = 0
    top_k: int = 0
    ep: int = 0
    moe_inter: int = 0

    @property
    def ka_r(self) -> int:
        return self.k_attn // self.n_ranks

    @property
    def ki_r(self) -> int:
        return self.inter // self.n_ranks

    def weight_bytes_per_step(self, weight_format: int = 0) -> int:
        """Weight bytes one rank streams per decode step (2L points)."""
        return self.layers * (self.weight_slice_bytes(self.ka_r, weight_format)
                              + self.weight_slice_bytes(self.ki_r, weight_format))

    def weight_slice_bytes(self, kr: int, weight_format: int = 0) -> int:
        """Bytes of one point's weight slice [kr x H]: bf16, or MX codes (1 or
        1/2 byte per weight) plus one 8-bit scale per 32 rows of a column."""
        h = self.hidden
        if weight_format == 0:
            return kr * h * 2
        return kr * h // (1 if weight_format == 1 else 2) + (kr // 32) * h

    def projection_bytes_per_step(self, weight_format: int = 0) -> int:
        """Bytes the rank's 2L partial projections must move per step: per
        point its weight slice, its activation slice (bf16) and its fp32
        partial written."""
        b, h = self.batch, self.hidden
        per_layer = 0
        for kr in (self.ka_r, self.ki_r):
            per_layer += self.weight_slice_bytes(kr, weight_format) + b * kr * 2 + b * h * 4
        return self.layers * per_layer

    def reduce_io_bytes_per_step(self) -> int:
        """Bytes of the emulated ring reductions per step: per point the N
        partials and the residual read and the sum written, fp32."""
        return self.layers * 2 * (self.n_ranks + 2) * self.batch * self.hidden * 4

    def algorithmic_bytes_per_step(self) -> int:
        """Both of the above: every byte the fused step moves at least."""
        return self.projection_bytes_per_step() + self.reduce_io_bytes_per_step()

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


TINY = Workload("tiny-h512-n2-b1", hidden=512, inter=1376, k_attn=512,
                n_ranks=2, batch=1, layers=1)
PAGE1 = Workload("page1-h5120-i17408-l64-n4-b1", hidden=5120, inter=17408,
                 k_attn=5120, n_ranks=4, batch=1, layers=64)
PAGE1_N2 = PAGE1.with_(name="page1-h5120-i17408-l64-n2", n_ranks=2)
H4096 = Workload("h4096-i12288-l48", hidden=4096, inter=12288, k_attn=4096,
                 n_ranks=4, batch=1, layers=48)
MOE = Workload("moe-h4096-attn8192-e128-top8-ep4-t64", hidden=4096, inter=0,
               k_attn=8192, n_ranks=4, batch=64, layers=1, n_experts=128,
               top_k=8, ep=4, moe_inter=1536)


# The prefill of "Interconnects e clusters" (lesson 9.9, Conceito): the
# page-1 stack with a 4,096-token prompt (batch = tokens of one prefill).
PREFILL = PAGE1.with_(name="prefill-page1-h5120-i17408-l64-n4-t4096", batch=4096)


def page1_n2(batch: int) -> Workload:
    return PAGE1_N2.with_(name="page1-h5120-i17408-l64-n2-b%d" % batch, batch=batch)


def page1_n4(batch: int) -> Workload:
    return PAGE1.with_(name="page1-h5120-i17408-l64-n4-b%d" % batch, batch=batch)


def h4096(n_ranks: int, batch: int) -> Workload:
    return H4096.with_(name="h4096-i12288-l48-n%d-b%d" % (n_ranks, batch),
                       n_ranks=n_ranks, batch=batch)


ALL = {w.name: w for w in [TINY, PAGE1] + [page1_n4(b) for b in (2, 4, 8, 16)]
       + [page1_n2(b) for b in (1, 2, 4, 8, 16, 32)]
       + [h4096(n, b) for n in (4, 8) for b in (1, 2, 4, 8, 16, 32, 64)] + [MOE, PREFILL]}
