"""Seeded input generators for the decode workloads.

Everything is drawn with one ``torch.Generator`` seeded with the workload's
seed, on the device the tensors are made on, in a fixed order:

1. lengths (variable-context workloads only): ``randint(lo, hi + 1, (B,))``;
2. the query ``q``: ``randn(B, Hq, d)`` (for a decode loop: ``randn(steps, B, Hq, d)``;
   for T > 1 new query tokens per sequence: ``randn(B, T, Hq, d)``, token t at
   position length - T + t);
3. the keys, one (sequence, KV head) slice at a time in (b, g) order: the
   filled rows ``randn(rows, d)``, or Student-t(3) as
   ``z0 / sqrt((z1^2 + z2^2 + z3^2) / 3)`` from four normal slices drawn in the
   order z0, z1, z2, z3; on planted workloads each slice is followed by its
   planted block ids ``randperm(n_b)[:n_plant]``, and every key of those blocks
   gets ``+2.0 * u`` before rounding, where ``u`` is the unit vector along the
   sum of the group's (rounded) query vectors (a direction for synthesis only);
4. the values, like the keys (always normal, never planted);
5. the page permutation (paged workloads only): ``randperm(num_pages)``.

bf16 tensors are the round-to-nearest-even cast of the fp32 draws.  Both the
GPU path and the oracle read the stored (rounded) values.

Layouts (the library's documented layouts):
* contiguous KV: ``k, v`` of shape ``[B][Hkv][T][d]`` with ``T = max_blocks * S``;
* paged KV: pools ``[num_pages][Hkv][S][d]`` and ``page_table[B][max_blocks]``
  (int32, -1 past each sequence's last block); page ids are a seeded
  permutation handed out in (b, block) order.

Token slots at or past a sequence's length (the tail of its last block and,
for the contiguous layout, all later blocks) hold zeros, or NaN when
``poison=True``; the decode must never read them into a result.
"""

from __future__ import annotations

import dataclasses
from typing import Optional

import torch

from .configs import Workload

_DT = {"f32": torch.float32, "bf16": torch.bfloat16}


@dataclasses.dataclass
class Case:
    wl: Workload
    q: torch.Tensor                    # [B][Hq][d], [steps][B][Hq][d] or [B][T][Hq][d]
    k: torch.Tensor                    # contiguous [B][Hkv][T][d] or pool [P][Hkv][S][d]
    v: torch.Tensor
    lens: torch.Tensor                 # int32 [B]: tokens in the cache incl. the new one
                                       # (decode loops: the length before the first step)
    page_table: Optional[torch.Tensor] = None   # int32 [B][max_blocks]
    top_k: Optional[torch.Tensor] = None        # int32 [B] (explicit counts) or None
    planted: Optional[torch.Tensor] = None      # int64 [B][Hkv][n_plant]
    num_pages: int = 0

    @property
    def device(self) -> torch.device:
        return self.k.device


def _normal(g: torch.Generator, shape, device) -> torch.Tensor:
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32)


def _student_t3(g: torch.Generator, shape, device) -> torch.Tensor:
    z0 = _normal(g, shape, device)
    z1 = _normal(g, shape, device)
    z2 = _normal(g, shape, device)
    z3 = _normal(g, shape, device)
    return z0 / torch.sqrt((z1 * z1 + z2 * z2 + z3 * z3) / 3.0)


def make_case(wl: Workload, device="cpu", poison: bool = False) -> Case:
    """Draws one workload instance on ``device`` (see the module docstring)."""
    device = torch.device(device)
    dt = _DT[wl.dtype]
    B, Hq, Hkv, d, S = wl.batch, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.block_size
    G = Hq // Hkv
    nbmax = wl.max_blocks
    T = nbmax * S
    g = torch.Generator(device=device)
    g.manual_seed(wl.seed)

    # 1. lengths
    if wl.variable_context is not None:
        lo, hi = wl.variable_context
        lens = torch.randint(lo, hi + 1, (B,), generator=g, device=device, dtype=torch.int64)
    else:
        lens = torch.full((B,), wl.context, device=device, dtype=torch.int64)
    # The cache is filled up to its capacity for a decode loop: the rows of later
    # steps are pre-written and only become visible when the length advances.
    fill = lens + wl.decode_steps

    # 2. query
    Tq = wl.query_tokens
    qshape = ((wl.decode_steps, B, Hq, d) if wl.decode_steps
              else (B, Tq, Hq, d) if Tq > 1 else (B, Hq, d))
    q = _normal(g, qshape, device).to(dt)

    # Direction used to plant blocks: the group's summed query, normalised.
    plant_dir = None
    if wl.planted_fraction is not None:
        qs = q.float().reshape(B, Tq, Hkv, G, d).sum(dim=(1, 3))
        plant_dir = qs / qs.norm(dim=-1, keepdim=True)

    nblk = [-(-int(x) // S) for x in lens.tolist()]
    fill_l = fill.tolist()

    def draw_kv(heavy: bool, plant: bool):
        out = torch.zeros((B, Hkv, T, d), device=device, dtype=dt)
        planted = None
        if plant:
            a, bb = wl.planted_fraction
            n_pl = -(-nblk[0] * a // bb)
            planted = torch.empty((B, Hkv, n_pl), dtype=torch.int64, device=device)
        for b in range(B):
            for h in range(Hkv):
                n = fill_l[b]
                x = _student_t3(g, (n, d), device) if heavy else _normal(g, (n, d), device)
                if plant:
                    idx = torch.randperm(nblk[b], generator=g, device=device)[:n_pl]
                    planted[b, h] = torch.sort(idx).values
                    for j in idx.tolist():
                        x[j * S: min((j + 1) * S, n)] += 2.0 * plant_dir[b, h]
                out[b, h, :n] = x.to(dt)
                if poison:
                    out[b, h, n:] = float("nan")
        return out, planted

    k, planted = draw_kv(wl.heavy_tailed_keys, wl.planted_fraction is not None)
    v, _ = draw_kv(False, False)

    top_k = None
    if wl.top_k is not None:
        top_k = torch.full((B,), wl.top_k, device=device, dtype=torch.int32)

    if not wl.paged:
        return Case(wl, q, k, v, lens.to(torch.int32), None, top_k, planted)

    # 5. paged layout: page ids are a seeded permutation, handed out in (b, j) order.
    num_pages = sum(-(-x // S) for x in fill_l)
    perm = torch.randperm(num_pages, generator=g, device=device).to(torch.int32)
    table = torch.full((B, nbmax), -1, dtype=torch.int32, device=device)
    kp = torch.empty((num_pages, Hkv, S, d), device=device, dtype=dt)
    vp = torch.empty_like(kp)
    nxt = 0
    for b in range(B):
        nb = -(-fill_l[b] // S)
        ids = perm[nxt: nxt + nb]
        nxt += nb
        table[b, :nb] = ids
        ids_l = ids.long()
        kp[ids_l] = k[b, :, : nb * S].reshape(Hkv, nb, S, d).transpose(0, 1)
        vp[ids_l] = v[b, :, : nb * S].reshape(Hkv, nb, S, d).transpose(0, 1)
    return Case(wl, q, kp, vp, lens.to(torch.int32), table, top_k, planted, num_pages)


@dataclasses.dataclass
class GateWeights:
    """Weights of the learned gate network, one set per KV head (CPU tensors).

    w1 int8 [Hkv][H][d], w1_scale float32 [Hkv][H], b1 float32 [Hkv][H],
    wq float32 [Hkv][H][d]; H is the hidden width.
    """
    w1: torch.Tensor
    w1_scale: torch.Tensor
    b1: torch.Tensor
    wq: torch.Tensor

    def to(self, device) -> "GateWeights":
        return GateWeights(*(t.to(device) for t in (self.w1, self.w1_scale, self.b1, self.wq)))


def make_gate_weights(num_kv_heads: int, head_dim: int, hidden: int = 256,
                      seed: int = 0) -> GateWeights:
    """Seeded random gate weights, drawn on the CPU in a fixed order: w1 as
    ``randint(-127, 128)``, w1_scale as ``(0.5 + rand) / (127 sqrt(d))``, b1 as
    ``0.05 * randn``, wq as ``randn / sqrt(d)``.  Untrained: they give the gate
    its shape and a realistic spread of scores, nothing more."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    H, d = hidden, head_dim
    w1 = torch.randint(-127, 128, (num_kv_heads, H, d), generator=g, dtype=torch.int64).to(torch.int8)
    w1_scale = (0.5 + torch.rand((num_kv_heads, H), generator=g)) / (127.0 * d ** 0.5)
    b1 = 0.05 * torch.randn((num_kv_heads, H), generator=g)
    wq = torch.randn((num_kv_heads, H, d), generator=g) / d ** 0.5
    return GateWeights(w1.contiguous(), w1_scale.float().contiguous(), b1.float().contiguous(),
                       wq.float().contiguous())
