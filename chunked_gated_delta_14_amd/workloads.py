"""Seeded synthetic inputs with the shapes and value ranges of the pages' workloads.

This module only draws random tensors; it holds none of the method's
arithmetic and is shared by the tests, the benchmark and the smoke check.

Workloads (FlashInfer PR #8218, workload paragraph: one packed batch of 4
documents, 42024 / 57573 / 73122 / 88673 tokens, q k v BF16 [T,H,128] with q
and k L2-normalised, g FP32 [T,H,128] pre-activated in (-5, 0), beta BF16
[T,H]; PR #7723, GB300 table: the 6-document GDN pack P1 of 241817 tokens at
(H_qk, H_v) = (16, 48) with FP32 scalar g and beta):

  0  KDA, 2 documents (200, 312), T = 512, H = 1
  1  KDA, one 32674-token shard of a document entered with h0 ~ 0.01 N(0,1), H = 16
  2  KDA, the 4-document pack, T = 261392, H = 4 or 16 (the measured workload)
  3  GDN, the 6-document pack, T = 241817, H_qk = 16, H_v = 48
  4  KDA, the 4-document pack at H = 64

Recipe: seed base = 1000 * (config + 1) + H (H_v for GDN); tensors q, k, v,
g, beta, dout, h0 are drawn in that order, tensor i from a generator seeded
base + i.  Draws are fp32: q, k ~ N(0,1) divided by max(||row||, 1e-6) per
(token, head); v, dout ~ N(0,1); g = -5 U[0,1); beta = sigmoid(N(0,1));
h0 = 0.01 N(0,1) (and, for tests that feed a final-state gradient,
dht = 0.02 N(0,1)).  Then q, k, v, dout (and KDA's beta) are rounded to bf16
(nearest even); the stored bits are what both the GPU and the oracle read.
"""
from __future__ import annotations

from dataclasses import dataclass

PACK4 = (42024, 57573, 73122, 88673)
PACK6 = (18000, 27500, 36000, 44317, 52000, 64000)


@dataclass(frozen=True)
class Workload:
    index: int
    name: str
    variant: str           # "kda" or "gdn"
    docs: tuple
    H_qk: int
    H_v: int
    with_h0: bool = False
    K: int = 128
    V: int = 128

    @property
    def T(self) -> int:
        return int(sum(self.docs))

    @property
    def seed_base(self) -> int:
        return 1000 * (self.index + 1) + self.H_v


def workload(index: int, H: int | None = None) -> Workload:
    if index == 0:
        return Workload(0, "kda_T512_H1", "kda", (200, 312), 1, 1)
    if index == 1:
        return Workload(1, "kda_shard_T32674_H16_h0", "kda", (32674,), 16, 16, with_h0=True)
    if index == 2:
        H = 16 if H is None else H
        return Workload(2, "kda_pack4_T261392_H%d" % H, "kda", PACK4, H, H)
    if index == 3:
        return Workload(3, "gdn_pack6_T241817_Hqk16_Hv48", "gdn", PACK6, 16, 48)
    if index == 4:
        return Workload(4, "kda_pack4_T261392_H64", "kda", PACK4, 64, 64)
    raise ValueError("unknown workload %d" % index)


def custom(variant: str, docs, H_qk: int, H_v: int, with_h0: bool = False, seed: int = 7) -> Workload:
    """A small workload of the same distributions (ragged packs for parity tests)."""
    return Workload(1000 + seed, "custom_%s_%s" % (variant, "_".join(map(str, docs))), variant,
                    tuple(int(d) for d in docs), H_qk, H_v, with_h0)


def make_inputs(w: Workload, device="cpu", gen_device=None, with_dout=True, dht=False):
    """Draw the workload's tensors.  Returns a dict of torch tensors on `device`:
    q, k, v, g, beta, cu_seqlens (int32, host), h0 (or None), dout, dht (or None)."""
    import torch

    gen_device = device if gen_device is None else gen_device
    T, Hqk, Hv, K, V = w.T, w.H_qk, w.H_v, w.K, w.V
    N = len(w.docs)

    def gen(i):
        g = torch.Generator(device=gen_device)
        g.manual_seed(w.seed_base + i)
        return g

    def unit_rows(x):
        return x / x.norm(dim=-1, keepdim=True).clamp_min(1e-6)

    q = unit_rows(torch.randn(T, Hqk, K, generator=gen(0), device=gen_device)).to(torch.bfloat16)
    k = unit_rows(torch.randn(T, Hqk, K, generator=gen(1), device=gen_device)).to(torch.bfloat16)
    v = torch.randn(T, Hv, V, generator=gen(2), device=gen_device).to(torch.bfloat16)
    gshape = (T, Hv, K) if w.variant == "kda" else (T, Hv)
    g = -5.0 * torch.rand(gshape, generator=gen(3), device=gen_device)
    beta = torch.sigmoid(torch.randn(T, Hv, generator=gen(4), device=gen_device))
    if w.variant == "kda":
        beta = beta.to(torch.bfloat16)
    out = dict(q=q, k=k, v=v, g=g, beta=beta)
    if with_dout:
        out["dout"] = torch.randn(T, Hv, V, generator=gen(5), device=gen_device).to(torch.bfloat16)
    out["h0"] = (0.01 * torch.randn(N, Hv, K, V, generator=gen(6), device=gen_device)) if w.with_h0 else None
    out["dht"] = (0.02 * torch.randn(N, Hv, K, V, generator=gen(7), device=gen_device)) if dht else None
    for key, val in list(out.items()):
        if val is not None:
            out[key] = val.to(device).contiguous()
    cu = [0]
    for d in w.docs:
        cu.append(cu[-1] + int(d))
    out["cu_seqlens"] = torch.tensor(cu, dtype=torch.int32)
    return out
