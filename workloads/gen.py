"""Seeded generator for DSA workloads in the paged-cache layout.

Shapes follow the Kimi K3.1 Pro sparse layer as the pages describe it: a
lightning indexer with 32 heads of 128 dims over one FP8 index key per token
(128 FP8 values plus a 4-byte scale), top-2048 selection, and MLA over a
576-wide FP8 latent row (512 compressed KV + 64 RoPE dims) per token, stored in
64-token paged blocks ("TokenSpeed Kimi K3.1", sections "Sparse attention in
Kimi K3.1 Pro" and "Storing index keys in the flat KV cache"; "Kimi K3.1 Pro on
AMD Instinct", model overview).

Everything here is input preparation: random draws, per-token absmax FP8
quantisation of those draws (through torch's own float8_e4m3fn cast) and the
placement of tokens into pages. No scoring, selection or attention happens in
this module.
"""

from __future__ import annotations

import dataclasses
import math
from typing import Optional, Sequence

import torch

BLOCK = 64  # tokens per cache page
H_IDX = 32  # indexer heads
D_IDX = 128  # indexer head dim
H_MLA = 16  # MLA heads served by one call
D_LAT = 576  # latent width (512 compressed KV + 64 RoPE)
D_V = 512  # value width (first 512 latent dims)
TOPK = 2048
E4M3_MAX = 448.0


@dataclasses.dataclass
class DsaCase:
    """One synthetic batch. Rows are request-major: row = b * R + r.

    Row r of request b sits at position ctx_len[b] - R + r and sees the
    tokens 0..position (its own token included).
    """

    name: str
    B: int
    R: int
    ctx_len: torch.Tensor  # int32 [B]
    block_table: torch.Tensor  # int32 [B, max_blocks], -1 = unused
    key_fp8: torch.Tensor  # uint8 [num_blocks, 64, 128]  (OCP E4M3 codes)
    key_scale: torch.Tensor  # fp32  [num_blocks, 64]
    lat_fp8: torch.Tensor  # uint8 [num_blocks, 64, 576]
    lat_scale: torch.Tensor  # fp32  [num_blocks, 64]
    q_idx: torch.Tensor  # bf16 [rows, 32, 128], or uint8 E4M3 codes when q_idx_scale is set
    q_idx_scale: Optional[torch.Tensor]  # fp32 [rows] (FP8 query rows) or None (bf16)
    w: torch.Tensor  # bf16 [rows, 32]
    q_mla: torch.Tensor  # bf16 [rows, 16, 576]
    sm_scale: float
    topk: int = TOPK
    planted: Optional[torch.Tensor] = None  # bool [B, max_ctx] planted tokens (structure record)
    key_format: str = "fp8"  # "fp8" or "mxfp4"
    key_fp4: Optional[torch.Tensor] = None  # uint8 [num_blocks, 64, 64] E2M1 pairs (mxfp4 keys)
    key_e8m0: Optional[torch.Tensor] = None  # uint8 [num_blocks, 64, 4] E8M0 block scales (mxfp4 keys)

    @property
    def rows(self) -> int:
        return self.B * self.R

    @property
    def max_ctx(self) -> int:
        return int(self.ctx_len.max().item())

    @property
    def max_blocks(self) -> int:
        return int(self.block_table.shape[1])

    @property
    def num_blocks(self) -> int:
        return int(self.lat_fp8.shape[0])

    def positions(self) -> torch.Tensor:
        """int64 [rows]: the position of each query row."""
        L = self.ctx_len.to(torch.int64).cpu()
        r = torch.arange(self.R, dtype=torch.int64)
        return (L[:, None] - self.R + r[None, :]).reshape(-1)

    def to(self, device) -> "DsaCase":
        fields = {}
        for f in dataclasses.fields(self):
            v = getattr(self, f.name)
            fields[f.name] = v.to(device) if isinstance(v, torch.Tensor) else v
        return DsaCase(**fields)


def quantize_e4m3_rows(x: torch.Tensor):
    """Per-row absmax quantisation of the last dim to OCP E4M3 codes.

    scale = absmax / 448 (1 for an all-zero row); codes = e4m3(x / scale) with
    round-to-nearest-even and saturation at +-448. Returns (uint8 codes, fp32 scale).
    """
    x = x.float()
    amax = x.abs().amax(dim=-1)
    scale = torch.where(amax > 0, amax / E4M3_MAX, torch.ones_like(amax))
    y = (x / scale.unsqueeze(-1)).clamp_(-E4M3_MAX, E4M3_MAX)
    codes = y.to(torch.float8_e4m3fn).view(torch.uint8)
    return codes, scale.float()


def _bf16_normal(shape, gen, device):
    return torch.randn(shape, generator=gen, device=device, dtype=torch.float32).to(torch.bfloat16)


def make_case(
    B: int,
    R: int,
    lengths: Sequence[int],
    *,
    seed: int,
    device="cpu",
    permute_blocks: bool = False,
    plant_frac: float = 0.0,
    plant_sigma: float = 3.0,
    plant_window: Optional[int] = None,
    fp8_query: bool = False,
    topk: int = TOPK,
    name: str = "custom",
    extra_blocks: int = 0,
    key_format: str = "fp8",
) -> DsaCase:
    """Build one batch.

    lengths[b] is the context length of request b, counting its R new rows.
    permute_blocks scatters every request's pages over a random permutation of
    the pool. plant_frac > 0 plants structure: that fraction of each request's
    tokens gets plant_sigma added along the unit vector of the request's
    head-weighted query sum before quantisation; with plant_window set, only
    tokens among the request's last plant_window positions are planted (a
    recency cluster: the row's highest scores sit in its most recent tokens). fp8_query stores the indexer
    queries as E4M3 codes with one fp32 scale per query row (prefill chunks).
    key_format "mxfp4" stores the index keys as MXFP4 instead (68 B per token:
    64 bytes of E2M1 pairs and four E8M0 block scales), drawn directly in
    that format: uniform random codes and block scales 2^-2 .. 2^1 (no
    planted structure).
    """
    assert key_format in ("fp8", "mxfp4")
    assert not (key_format == "mxfp4" and plant_frac > 0), "planted keys are FP8 only"
    device = torch.device(device)
    lengths = [int(x) for x in lengths]
    assert len(lengths) == B and all(L >= R for L in lengths)
    cpu = torch.Generator(device="cpu")
    cpu.manual_seed(seed)
    gen = torch.Generator(device=device)
    gen.manual_seed(seed + 1)

    nblk_req = [math.ceil(L / BLOCK) for L in lengths]
    max_blocks = max(nblk_req)
    num_blocks = sum(nblk_req) + extra_blocks
    if permute_blocks:
        pool = torch.randperm(num_blocks, generator=cpu)
    else:
        pool = torch.arange(num_blocks)
    table = torch.full((B, max_blocks), -1, dtype=torch.int32)
    off = 0
    for b, nb in enumerate(nblk_req):
        table[b, :nb] = pool[off : off + nb].to(torch.int32)
        off += nb

    rows = B * R
    if fp8_query:
        qf = torch.randn((rows, H_IDX, D_IDX), generator=gen, device=device)
        codes, qs = quantize_e4m3_rows(qf.reshape(rows, H_IDX * D_IDX))
        q_idx = codes.reshape(rows, H_IDX, D_IDX)
        q_idx_scale = qs
        q_dir = (q_idx.view(torch.float8_e4m3fn).float() * qs[:, None, None])
    else:
        q_idx = _bf16_normal((rows, H_IDX, D_IDX), gen, device)
        q_idx_scale = None
        q_dir = q_idx.float()
    w = torch.rand((rows, H_IDX), generator=gen, device=device, dtype=torch.float32).to(torch.bfloat16)
    q_mla = _bf16_normal((rows, H_MLA, D_LAT), gen, device)

    f4 = key_format == "mxfp4"
    if f4:
        key_fp8 = key_scale = None
        key_fp4 = torch.zeros((num_blocks, BLOCK, D_IDX // 2), dtype=torch.uint8, device=device)
        key_e8m0 = torch.full((num_blocks, BLOCK, D_IDX // 32), 127, dtype=torch.uint8, device=device)
    else:
        key_fp8 = torch.empty((num_blocks, BLOCK, D_IDX), dtype=torch.uint8, device=device)
        key_scale = torch.ones((num_blocks, BLOCK), dtype=torch.float32, device=device)
        key_fp4 = key_e8m0 = None
    lat_fp8 = torch.empty((num_blocks, BLOCK, D_LAT), dtype=torch.uint8, device=device)
    lat_scale = torch.ones((num_blocks, BLOCK), dtype=torch.float32, device=device)
    if extra_blocks:
        if not f4:
            key_fp8.zero_()
        lat_fp8.zero_()

    planted = torch.zeros((B, max_blocks * BLOCK), dtype=torch.bool) if plant_frac > 0 else None
    CH = 64 * BLOCK * 16  # tokens generated per chunk (bounds transient memory)
    for b in range(B):
        ntok = nblk_req[b] * BLOCK
        blocks = table[b, : nblk_req[b]].to(torch.int64).to(device)
        if plant_frac > 0:
            wq = (w[b * R : (b + 1) * R].float()[:, :, None] * q_dir[b * R : (b + 1) * R]).sum(dim=(0, 1))
            u = wq / wq.norm()
            mask = torch.rand(ntok, generator=cpu) < plant_frac
            if plant_window is not None:
                mask &= torch.arange(ntok) >= lengths[b] - int(plant_window)
            planted[b, :ntok] = mask
            mask_d = mask.to(device)
        for t0 in range(0, ntok, CH):
            t1 = min(ntok, t0 + CH)
            bsel = blocks[t0 // BLOCK : t1 // BLOCK]
            if f4:
                kb = torch.randint(0, 256, (t1 - t0, D_IDX // 2), generator=gen, device=device, dtype=torch.int32)
                ke = torch.randint(125, 129, (t1 - t0, D_IDX // 32), generator=gen, device=device, dtype=torch.int32)
                key_fp4[bsel] = kb.to(torch.uint8).reshape(-1, BLOCK, D_IDX // 2)
                key_e8m0[bsel] = ke.to(torch.uint8).reshape(-1, BLOCK, D_IDX // 32)
            else:
                k = torch.randn((t1 - t0, D_IDX), generator=gen, device=device)
                if plant_frac > 0:
                    k += plant_sigma * mask_d[t0:t1, None].float() * u[None, :]
                kc, ks = quantize_e4m3_rows(k)
                key_fp8[bsel] = kc.reshape(-1, BLOCK, D_IDX)
                key_scale[bsel] = ks.reshape(-1, BLOCK)
            c = torch.randn((t1 - t0, D_LAT), generator=gen, device=device)
            cc, cs = quantize_e4m3_rows(c)
            lat_fp8[bsel] = cc.reshape(-1, BLOCK, D_LAT)
            lat_scale[bsel] = cs.reshape(-1, BLOCK)

    return DsaCase(
        name=name,
        B=B,
        R=R,
        ctx_len=torch.tensor(lengths, dtype=torch.int32, device=device),
        block_table=table.to(device),
        key_fp8=key_fp8,
        key_scale=key_scale,
        lat_fp8=lat_fp8,
        lat_scale=lat_scale,
        q_idx=q_idx,
        q_idx_scale=q_idx_scale,
        w=w,
        q_mla=q_mla,
        sm_scale=1.0 / math.sqrt(D_LAT),
        topk=topk,
        planted=planted,
        key_format=key_format,
        key_fp4=key_fp4,
        key_e8m0=key_e8m0,
    )


# The workloads the path is measured and checked on. Seeds are fixed per
# workload so every run regenerates the same bytes on the same device.
WORKLOADS = {
    "decode_1x1_8k": dict(B=1, R=1, lengths=[8192], seed=20260001),
    "decode_16x4_32k": dict(B=16, R=4, lengths=[32768] * 16, seed=20260002),
    "decode_16x4_ragged_128k_256k": dict(B=16, R=4, lengths=None, seed=20260003, permute_blocks=True,
                                         length_range=(131072, 262144)),
    "decode_16x8_32k": dict(B=16, R=8, lengths=[32768] * 16, seed=20260006),
    "decode_4x4_1m_planted": dict(B=4, R=4, lengths=[1 << 20] * 4, seed=20260004, plant_frac=0.01),
    "decode_4x4_1m_mxfp4": dict(B=4, R=4, lengths=[1 << 20] * 4, seed=20260007, key_format="mxfp4"),
    # 10% of the last 32K positions planted at +12 sigma: nearly all of each row's top-2048 lies in
    # its most recent 32K tokens (a recency cluster)
    "decode_4x4_1m_recent": dict(B=4, R=4, lengths=[1 << 20] * 4, seed=20260008, plant_frac=0.1,
                                 plant_window=32768, plant_sigma=12.0),
    # 16 requests x 4 verification rows at U[256K, 1M] tokens each, permuted pages
    "decode_16x4_256k_1m": dict(B=16, R=4, lengths=None, seed=20260009, permute_blocks=True,
                                length_range=(262144, 1048576)),
    "prefill_4096_on_128k": dict(B=1, R=4096, lengths=[131072 + 4096], seed=20260005, fp8_query=True),
    # the 1M workload with E4M3 index queries (row scales), as the pages' decode indexer takes them
    "decode_4x4_1m_fp8q": dict(B=4, R=4, lengths=[1 << 20] * 4, seed=20260010, plant_frac=0.01, fp8_query=True),
    # the target shape with E4M3 index queries
    "decode_16x4_256k_1m_fp8q": dict(B=16, R=4, lengths=None, seed=20260011, permute_blocks=True,
                                     length_range=(262144, 1048576), fp8_query=True),
}


def case_config(name: str, seed_offset: int = 0) -> dict:
    """Keyword arguments of make_case for a named workload."""
    cfg = dict(WORKLOADS[name])
    cfg["seed"] = cfg["seed"] + seed_offset
    cfg["name"] = name
    lo_hi = cfg.pop("length_range", None)
    if cfg["lengths"] is None:  # ragged: U[lo, hi] per request, seeded
        g = torch.Generator(device="cpu")
        g.manual_seed(cfg["seed"] + 7)
        cfg["lengths"] = torch.randint(lo_hi[0], lo_hi[1] + 1, (cfg["B"],), generator=g).tolist()
    return cfg


STRUCTURE_KEYS = ("permute_blocks", "plant_frac", "plant_window", "plant_sigma", "fp8_query", "key_format")


def structure_kwargs(cfg: dict) -> dict:
    """The make_case keyword arguments of a workload config that shape its
    structure (page permutation, planted keys, query and key formats)."""
    return {k: v for k, v in cfg.items() if k in STRUCTURE_KEYS}
