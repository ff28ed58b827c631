"""Workload shapes and seeded synthetic input generators for the DSA hot path.

This module holds input generation only: shapes, random draws and the upstream
quantisation of indexer activations to FP8 bytes plus per-token scales.  None
of the method's arithmetic (indexer scoring, selection, attention) lives here,
so the float64 oracle and the HIP path can both take their inputs from it.

The pages (DeepSeek-V3.2 summaries) describe no dataset for this path; every
tensor is synthetic with the shapes and value laws listed per workload.

Random draws use a seeded ``torch.Generator`` on the device the tensors are
made on, so a workload is reproducible per device; the oracle always reads
the very tensors the kernels read (copied to the host), never a re-draw.
"""
from __future__ import annotations

import dataclasses
import math
from dataclasses import dataclass

import torch

FP8_MAX = 448.0  # largest finite OCP e4m3fn magnitude


@dataclass(frozen=True)
class Workload:
    """One DSA problem shape.

    Prefill workloads have one sequence of ``seq_len`` tokens, every token a
    query against its causal prefix.  Decode workloads have ``decode_batch``
    sequences, each with one query (the last cached token) against a cache
    whose length is drawn uniformly from ``[ctx_min, ctx_max]``.  Chunked
    prefill splits the query rows of a prefill sequence into ``chunk``-row
    slices, each run against the full causal prefix.
    """

    name: str
    seq_len: int
    idx_heads: int          # H_I: lightning-indexer heads
    idx_dim: int            # d_I: indexer head dimension
    topk: int               # k: selected key positions per query
    heads: int              # H: attention query heads sharing one latent KV row
    d_latent: int           # latent part of the KV row (also the value width)
    d_rope: int             # rotary part of the KV row (keys only)
    softmax_scale: float
    attn_std: float         # q and kv drawn from N(0, attn_std^2)
    seed: int
    decode_batch: int = 0   # > 0: decode step over this many sequences
    ctx_min: int = 0
    ctx_max: int = 0
    chunk: int = 0          # > 0: chunked prefill with this many query rows per chunk
    boost_frac: float = 0.0  # fraction of indexer key positions scaled up in norm
    boost_factor: float = 1.0

    @property
    def d_qk(self) -> int:
        return self.d_latent + self.d_rope

    @property
    def is_decode(self) -> bool:
        return self.decode_batch > 0

    def scaled(self, **changes) -> "Workload":
        """A copy with some fields replaced (used for parity cases at reduced sizes)."""
        return dataclasses.replace(self, **changes)


# The five workloads of the method's hot path, named by what they are.
TINY_PREFILL = Workload(
    name="tiny_prefill_L256", seq_len=256, idx_heads=4, idx_dim=32, topk=32,
    heads=8, d_latent=64, d_rope=16, softmax_scale=1.0 / math.sqrt(80.0),
    attn_std=1.0 / math.sqrt(80.0), seed=18000)
PREFILL_4K = Workload(
    name="prefill_L4096", seq_len=4096, idx_heads=64, idx_dim=128, topk=2048,
    heads=128, d_latent=512, d_rope=64, softmax_scale=1.0 / math.sqrt(192.0),
    attn_std=1.0, seed=18001)
PREFILL_32K_BOOSTED = Workload(
    name="prefill_L32768_boosted_keys", seq_len=32768, idx_heads=64, idx_dim=128,
    topk=2048, heads=128, d_latent=512, d_rope=64,
    softmax_scale=1.0 / math.sqrt(192.0), attn_std=1.0, seed=18002,
    boost_frac=0.05, boost_factor=3.0)
DECODE_B64 = Workload(
    name="decode_B64_ctx8K_128K", seq_len=131072, idx_heads=64, idx_dim=128,
    topk=2048, heads=128, d_latent=512, d_rope=64,
    softmax_scale=1.0 / math.sqrt(192.0), attn_std=1.0, seed=18003,
    decode_batch=64, ctx_min=8192, ctx_max=131072)
CHUNKED_PREFILL_128K = Workload(
    name="chunked_prefill_L131072_chunk4096", seq_len=131072, idx_heads=64,
    idx_dim=128, topk=2048, heads=128, d_latent=512, d_rope=64,
    softmax_scale=1.0 / math.sqrt(192.0), attn_std=1.0, seed=18004, chunk=4096)

WORKLOADS = {w.name: w for w in
             (TINY_PREFILL, PREFILL_4K, PREFILL_32K_BOOSTED, DECODE_B64, CHUNKED_PREFILL_128K)}


def quantize_rows_e4m3(x: torch.Tensor) -> tuple[torch.Tensor, torch.Tensor]:
    """Upstream activation quantiser: one fp32 scale per leading-dim row.

    ``scale = max(amax(|row|), 1e-12) / 448``; codes = RNE(row / scale) clamped
    to +-448, stored as e4m3fn bytes.  Parity is defined on the bytes and the
    scales this returns, so the quantiser itself is not under test.
    """
    flat = x.reshape(x.shape[0], -1).float()
    amax = flat.abs().amax(dim=1).clamp_min(1e-12)
    scale = (amax / FP8_MAX).float()
    y = (flat / scale[:, None]).clamp(-FP8_MAX, FP8_MAX)
    codes = y.to(torch.float8_e4m3fn).view(torch.uint8).reshape(x.shape)
    return codes.contiguous(), scale.contiguous()


def _randn_bf16(shape, std, gen, device, rows_per_step=4096):
    """N(0, std^2) in bfloat16, drawn in row slices to bound fp32 temporaries."""
    out = torch.empty(shape, dtype=torch.bfloat16, device=device)
    n = shape[0]
    for r0 in range(0, n, rows_per_step):
        r1 = min(n, r0 + rows_per_step)
        tmp = torch.randn((r1 - r0,) + tuple(shape[1:]), generator=gen, device=device,
                          dtype=torch.float32)
        out[r0:r1] = (tmp * std).to(torch.bfloat16)
    return out


def _indexer_q(n, wl, gen, device, rows_per_step=8192):
    codes = torch.empty((n, wl.idx_heads, wl.idx_dim), dtype=torch.uint8, device=device)
    scales = torch.empty((n,), dtype=torch.float32, device=device)
    for r0 in range(0, n, rows_per_step):
        r1 = min(n, r0 + rows_per_step)
        x = torch.randn((r1 - r0, wl.idx_heads, wl.idx_dim), generator=gen, device=device)
        codes[r0:r1], scales[r0:r1] = quantize_rows_e4m3(x)
    return codes, scales


def generate(wl: Workload, device="cpu", seed: int | None = None) -> dict:
    """Seeded synthetic inputs for ``wl`` on ``device``.

    Returns a dict of tensors plus the sequence layout:

    * ``q_fp8 [T_q, H_I, d_I] u8``, ``q_scale [T_q] f32``, ``w [T_q, H_I] f32``
    * ``k_fp8 [T_k, d_I] u8``, ``k_scale [T_k] f32``
    * ``q [T_q, H, d_latent + d_rope] bf16``, ``kv [T_k, d_latent + d_rope] bf16``
    * ``q_offsets``, ``kv_offsets`` (lists, length B+1), ``q_pos0`` (list, length B):
      packed query / key rows per sequence and the position of each sequence's
      first query row.
    * ``boosted``: the key rows scaled up before quantising (empty if none).

    Value laws: indexer q and k ~ N(0,1) before per-token e4m3 quantisation,
    w ~ U(0,1), attention q and kv ~ N(0, attn_std^2) in bf16.  With
    ``boost_frac`` > 0 a seeded set of round(boost_frac * T_k) key positions is
    multiplied by ``boost_factor`` before quantising (bytes unchanged, scale
    multiplied).  Decode cache lengths are integers uniform on
    ``[ctx_min, ctx_max]``; each sequence's query sits at its last position.
    """
    seed = wl.seed if seed is None else seed
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    D = wl.d_qk
    if wl.is_decode:
        B = wl.decode_batch
        lens = torch.randint(wl.ctx_min, wl.ctx_max + 1, (B,), generator=gen, device=device)
        lens = [int(x) for x in lens.cpu()]
        kv_offsets = [0]
        for n in lens:
            kv_offsets.append(kv_offsets[-1] + n)
        T_q, T_k = B, kv_offsets[-1]
        q_offsets = list(range(B + 1))
        q_pos0 = [n - 1 for n in lens]
    else:
        T_q = T_k = wl.seq_len
        q_offsets, kv_offsets, q_pos0 = [0, T_q], [0, T_k], [0]
    q_fp8, q_scale = _indexer_q(T_q, wl, gen, device)
    w = torch.rand((T_q, wl.idx_heads), generator=gen, device=device, dtype=torch.float32)
    k_f32 = torch.randn((T_k, wl.idx_dim), generator=gen, device=device)
    boosted = torch.empty(0, dtype=torch.int64, device=device)
    if wl.boost_frac > 0:
        nb = int(round(wl.boost_frac * T_k))
        boosted = torch.randperm(T_k, generator=gen, device=device)[:nb]
        k_f32[boosted] *= wl.boost_factor
    k_fp8, k_scale = quantize_rows_e4m3(k_f32)
    del k_f32
    q = _randn_bf16((T_q, wl.heads, D), wl.attn_std, gen, device)
    kv = _randn_bf16((T_k, D), wl.attn_std, gen, device)
    return dict(q_fp8=q_fp8, q_scale=q_scale, w=w, k_fp8=k_fp8, k_scale=k_scale,
                q=q, kv=kv, q_offsets=q_offsets, kv_offsets=kv_offsets, q_pos0=q_pos0,
                boosted=boosted)


def chunk_views(inputs: dict, chunk: int):
    """Yield (q_pos0, q-row slice) for chunked prefill of a single sequence.

    Chunk c covers query rows [c*chunk, (c+1)*chunk) against keys
    [0, (c+1)*chunk); the key/KV tensors stay whole and resident.
    """
    L = inputs["q_offsets"][1]
    for r0 in range(0, L, chunk):
        yield r0, slice(r0, min(L, r0 + chunk))


def paged_caches(inp: dict, block_size: int, seed: int = 0, extra_blocks: int = 5,
                 high_base_rows: int = 0, device="cuda"):
    """Block-table copies of a workload's packed key and latent KV caches
    (the serving layout of dsa_paged_kv): every sequence's rows are cut into
    blocks of ``block_size`` and scattered over shuffled physical blocks,
    with ``extra_blocks`` unused ones among them.  With ``high_base_rows`` the
    used blocks start that many rows into the caches (the rows below stay
    zero), e.g. to place them past 4 GB.  Unused table entries are -1.
    Returns (block_table [B, max_blocks] int32 on the CPU, num_blocks,
    k_cache [nb, bs, d_I] u8, ks_cache [nb, bs] f32, kv_cache [nb, bs, D] bf16)."""
    kv_off = [int(x) for x in inp["kv_offsets"]]
    B = len(kv_off) - 1
    lens = [kv_off[b + 1] - kv_off[b] for b in range(B)]
    nblk = [(n + block_size - 1) // block_size for n in lens]
    max_blocks = max(1, max(nblk))
    used = sum(nblk)
    g = torch.Generator().manual_seed(seed)
    base_blk = (high_base_rows + block_size - 1) // block_size
    phys = (torch.randperm(used + extra_blocks, generator=g)[:used] + base_blk).tolist()
    num_blocks = base_blk + used + extra_blocks
    table = torch.full((B, max_blocks), -1, dtype=torch.int32)
    src, dst = [], []
    it = iter(phys)
    for b in range(B):
        for j in range(nblk[b]):
            pb = next(it)
            table[b, j] = pb
            n = min(block_size, lens[b] - j * block_size)
            src.append(torch.arange(kv_off[b] + j * block_size, kv_off[b] + j * block_size + n))
            dst.append(torch.arange(pb * block_size, pb * block_size + n))
    src = torch.cat(src).to(device) if src else torch.zeros(0, dtype=torch.long, device=device)
    dst = torch.cat(dst).to(device) if dst else torch.zeros(0, dtype=torch.long, device=device)
    nrows = num_blocks * block_size
    k, ks, kv = inp["k_fp8"].to(device), inp["k_scale"].to(device), inp["kv"].to(device)
    k_cache = torch.zeros(nrows, k.shape[1], dtype=k.dtype, device=device)
    ks_cache = torch.zeros(nrows, dtype=ks.dtype, device=device)
    kv_cache = torch.zeros(nrows, kv.shape[1], dtype=kv.dtype, device=device)
    k_cache[dst] = k[src]
    ks_cache[dst] = ks[src]
    kv_cache[dst] = kv[src]
    return (table, num_blocks, k_cache.view(num_blocks, block_size, -1),
            ks_cache.view(num_blocks, block_size), kv_cache.view(num_blocks, block_size, -1))


# Prefill-mode (per-head) attention: per-head widths of that form.
MHA_NOPE, MHA_ROPE, MHA_V = 128, 64, 128


def mha_prefill_inputs(q_rows: int, kv_rows: int, heads: int, seed: int, device="cpu",
                       std: float = 1.0) -> dict:
    """Seeded inputs of the prefill-mode attention: q [q_rows, heads, 192],
    k_nope [kv_rows, heads, 128], k_rope [kv_rows, 64], v [kv_rows, heads, 128],
    each N(0, std^2) in bfloat16 (the law of keys and values decompressed from
    unit-variance latents by projections of unit gain)."""
    gen = torch.Generator(device=device).manual_seed(seed)
    return dict(q=_randn_bf16((q_rows, heads, MHA_NOPE + MHA_ROPE), std, gen, device),
                k_nope=_randn_bf16((kv_rows, heads, MHA_NOPE), std, gen, device),
                k_rope=_randn_bf16((kv_rows, MHA_ROPE), std, gen, device),
                v=_randn_bf16((kv_rows, heads, MHA_V), std, gen, device))
