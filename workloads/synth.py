"""Seeded synthetic workloads for QK-norm + RoPE + causal GQA attention.

Every tensor here is drawn from a seeded generator; nothing is computed from
the drawn values.  The shapes follow the layouts of the attention layer the
pages describe:

* packed ``qkv`` rows ``[N, (Hq + 2*Hkv) * D]`` -- Q heads, then K heads, then
  V heads, each ``D`` columns wide (zero-to-sglang "Chapter 3 ... (Code
  Walkthrough)", section 3.3; jq-wei "transformer basics", "Attention
  calculation: part 1");
* per-head norm weights ``[D]``, drawn as ``1 + 0.1 * N(0, 1)``;
* requests packed back to back and delimited by ``cu_seqlens`` (the packed
  ``[N, C]`` batch of the code walkthrough, section 3.1);
* a contiguous K/V cache ``[B, Hkv, S_cap, D]`` per request and KV head (the
  per-layer cache that prefill fills and decode extends, "transformer
  basics", "Prefill vs Decode").

Draw order for one workload (all on one CPU ``torch.Generator`` seeded with the
workload's seed): request / cache lengths, then ``qkv`` (fp32 normal, rounded
to the storage dtype), then the Q-norm weight, then the K-norm weight.  Decode
cache contents (K slots below each cache length, then V) are drawn afterwards
from a second generator, seeded with ``seed + 1``, on the device that will hold
the cache, because the long-context caches run to gigabytes.  Cache slots that
hold no token are filled with NaN in parity runs (so any stray read or write
shows) and with zeros in timing runs.
"""

from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional, Sequence

import torch


@dataclasses.dataclass(frozen=True)
class HeadConfig:
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    rms_eps: float = 1e-6
    rope_base: float = 1e6

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads


def qkv_width(h: HeadConfig) -> int:
    return (h.num_q_heads + 2 * h.num_kv_heads) * h.head_dim


@dataclasses.dataclass
class PrefillInputs:
    heads: HeadConfig
    qkv: torch.Tensor            # [N, (Hq+2Hkv)*D]
    q_norm_weight: torch.Tensor  # [D]
    k_norm_weight: torch.Tensor  # [D]
    positions: torch.Tensor      # int32 [N]
    cu_seqlens: torch.Tensor     # int32 [B+1]
    seqlens: List[int]
    cache_capacity: int
    k_cache: torch.Tensor        # [B, Hkv, S_cap, D], initial contents
    v_cache: torch.Tensor

    @property
    def num_tokens(self) -> int:
        return int(sum(self.seqlens))

    @property
    def num_seqs(self) -> int:
        return len(self.seqlens)

    @property
    def max_seqlen(self) -> int:
        return max(self.seqlens) if self.seqlens else 0


@dataclasses.dataclass
class DecodeInputs:
    heads: HeadConfig
    qkv: torch.Tensor            # [B, (Hq+2Hkv)*D], one new token per request
    q_norm_weight: torch.Tensor
    k_norm_weight: torch.Tensor
    positions: torch.Tensor      # int32 [B]
    cache_lens: torch.Tensor     # int32 [B], valid entries before this step
    cache_capacity: int
    k_cache: torch.Tensor        # [B, Hkv, S_cap, D]
    v_cache: torch.Tensor

    @property
    def num_seqs(self) -> int:
        return int(self.qkv.shape[0])

    @property
    def max_cache_len(self) -> int:
        return int(self.cache_lens.max().item()) if self.num_seqs else 0


@dataclasses.dataclass
class AppendInputs:
    heads: HeadConfig
    qkv: torch.Tensor            # [N, (Hq+2Hkv)*D], the chunks' new tokens, packed
    q_norm_weight: torch.Tensor
    k_norm_weight: torch.Tensor
    positions: torch.Tensor      # int32 [N]: P_r + j for token j of request r
    cu_seqlens: torch.Tensor     # int32 [B+1] over the new tokens
    seqlens: List[int]           # T_r
    cache_lens: torch.Tensor     # int32 [B]: P_r, entries cached before the chunk
    past_lens: List[int]
    cache_capacity: int
    k_cache: torch.Tensor        # [B, Hkv, S_cap, D]
    v_cache: torch.Tensor

    @property
    def num_tokens(self) -> int:
        return int(sum(self.seqlens))

    @property
    def num_seqs(self) -> int:
        return len(self.seqlens)

    @property
    def max_seqlen(self) -> int:
        return max(self.seqlens) if self.seqlens else 0

    @property
    def max_cache_len(self) -> int:
        return max(self.past_lens) if self.past_lens else 0


@dataclasses.dataclass
class NormInputs:
    """Inputs of the fused residual add + RMSNorm over hidden-size rows."""
    x: torch.Tensor                   # [N, C] sublayer output
    residual: Optional[torch.Tensor]  # [N, C] residual stream (None: first call of a forward pass)
    weight: torch.Tensor              # [C]
    rms_eps: float = 1e-6

    @property
    def has_residual(self) -> bool:
        return self.residual is not None


@dataclasses.dataclass
class NextTokenInputs:
    """Packed hidden states and one logits row per request, for next-token selection."""
    hidden: torch.Tensor       # [N, C]
    cu_seqlens: torch.Tensor   # int32 [B+1]
    seqlens: List[int]
    logits: torch.Tensor       # [B, V], drawn directly (the LM head is outside the path)


@dataclasses.dataclass
class WorkloadInputs:
    name: str
    description: str
    prefill: Optional[PrefillInputs]
    decode: Optional[DecodeInputs]
    # Rows for decode steps that continue the prefill's own cache: one
    # [B_prefill, W] tensor per step; step s runs at position T_r + s.
    chained_decode_qkv: List[torch.Tensor] = dataclasses.field(default_factory=list)
    append: Optional[AppendInputs] = None
    norm: Optional[NormInputs] = None
    next_token: Optional[NextTokenInputs] = None


def _sentinel(parity: bool) -> float:
    return float("nan") if parity else 0.0


def _empty_cache(h: HeadConfig, batch: int, capacity: int, dtype, device, parity: bool):
    shape = (batch, h.num_kv_heads, capacity, h.head_dim)
    k = torch.full(shape, _sentinel(parity), dtype=dtype, device=device)
    v = torch.full(shape, _sentinel(parity), dtype=dtype, device=device)
    return k, v


def _draw_rows(g: torch.Generator, rows: int, h: HeadConfig, dtype) -> torch.Tensor:
    return torch.randn((rows, qkv_width(h)), generator=g, dtype=torch.float32).to(dtype)


def _draw_norm_weight(g: torch.Generator, h: HeadConfig, dtype) -> torch.Tensor:
    return (1.0 + 0.1 * torch.randn((h.head_dim,), generator=g, dtype=torch.float32)).to(dtype)


def _fill_decode_cache(h: HeadConfig, cache_lens: torch.Tensor, capacity: int, seed: int,
                       dtype, device, parity: bool):
    """K then V cache with N(0,1) in slots < cache_len, sentinel elsewhere."""
    batch = int(cache_lens.numel())
    shape = (batch, h.num_kv_heads, capacity, h.head_dim)
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    lens_dev = cache_lens.to(device=device, dtype=torch.int64)
    unused = (torch.arange(capacity, device=device)[None, :] >= lens_dev[:, None])  # [B, S]
    unused = unused[:, None, :, None]
    caches = []
    for _ in range(2):
        c = torch.empty(shape, dtype=dtype, device=device)
        c.normal_(generator=g)
        c.masked_fill_(unused, _sentinel(parity))
        caches.append(c)
    return caches[0], caches[1]


def _prefill_from_rows(h: HeadConfig, rows: torch.Tensor, wq, wk, seqlens: Sequence[int],
                       capacity: Optional[int], dtype, device, parity: bool) -> PrefillInputs:
    seqlens = [int(t) for t in seqlens]
    cu = [0]
    for t in seqlens:
        cu.append(cu[-1] + t)
    positions = torch.cat([torch.arange(t, dtype=torch.int32) for t in seqlens]) if seqlens else \
        torch.zeros((0,), dtype=torch.int32)
    cap = capacity if capacity is not None else max(seqlens + [1])
    k_cache, v_cache = _empty_cache(h, len(seqlens), cap, dtype, device, parity)
    return PrefillInputs(
        heads=h, qkv=rows.to(device), q_norm_weight=wq.to(device), k_norm_weight=wk.to(device),
        positions=positions.to(device), cu_seqlens=torch.tensor(cu, dtype=torch.int32).to(device),
        seqlens=seqlens, cache_capacity=cap, k_cache=k_cache, v_cache=v_cache)


def make_prefill_inputs(h: HeadConfig, seqlens: Sequence[int], seed: int, dtype=torch.bfloat16,
                        device="cpu", capacity: Optional[int] = None, parity: bool = True) -> PrefillInputs:
    """A prefill batch of requests with the given lengths (positions 0..T_r-1 each)."""
    g = torch.Generator().manual_seed(seed)
    rows = _draw_rows(g, int(sum(seqlens)), h, dtype)
    wq = _draw_norm_weight(g, h, dtype)
    wk = _draw_norm_weight(g, h, dtype)
    return _prefill_from_rows(h, rows, wq, wk, seqlens, capacity, dtype, device, parity)


def prefill_inputs_from_rows(h: HeadConfig, rows: torch.Tensor, q_norm_weight: torch.Tensor,
                             k_norm_weight: torch.Tensor, seqlens: Sequence[int], dtype=torch.bfloat16,
                             device="cpu", capacity: Optional[int] = None, parity: bool = True) -> PrefillInputs:
    """A prefill batch over given packed rows and norm weights (e.g. a prefix of another batch's rows)."""
    return _prefill_from_rows(h, rows.cpu(), q_norm_weight.cpu(), k_norm_weight.cpu(), seqlens, capacity, dtype,
                              device, parity)


def make_decode_inputs(h: HeadConfig, cache_lens: Sequence[int], seed: int, dtype=torch.bfloat16,
                       device="cpu", capacity: Optional[int] = None, parity: bool = True) -> DecodeInputs:
    """One new token per request on top of a cache holding ``cache_lens[b]`` entries."""
    g = torch.Generator().manual_seed(seed)
    lens = torch.tensor([int(x) for x in cache_lens], dtype=torch.int32)
    rows = _draw_rows(g, int(lens.numel()), h, dtype)
    wq = _draw_norm_weight(g, h, dtype)
    wk = _draw_norm_weight(g, h, dtype)
    cap = capacity if capacity is not None else (int(lens.max().item()) + 1 if lens.numel() else 1)
    k_cache, v_cache = _fill_decode_cache(h, lens, cap, seed + 1, dtype, device, parity)
    return DecodeInputs(heads=h, qkv=rows.to(device), q_norm_weight=wq.to(device),
                        k_norm_weight=wk.to(device), positions=lens.clone().to(device),
                        cache_lens=lens.to(device), cache_capacity=cap, k_cache=k_cache, v_cache=v_cache)


def make_append_inputs(h: HeadConfig, past_lens: Sequence[int], chunk_lens: Sequence[int], seed: int,
                       dtype=torch.bfloat16, device="cpu", capacity: Optional[int] = None,
                       parity: bool = True) -> AppendInputs:
    """A chunk of T_r new tokens per request on a cache holding P_r entries (N(0,1), as decode's)."""
    g = torch.Generator().manual_seed(seed)
    past = [int(x) for x in past_lens]
    chunks = [int(x) for x in chunk_lens]
    rows = _draw_rows(g, int(sum(chunks)), h, dtype)
    wq = _draw_norm_weight(g, h, dtype)
    wk = _draw_norm_weight(g, h, dtype)
    cu = [0]
    for t in chunks:
        cu.append(cu[-1] + t)
    positions = torch.cat([torch.arange(p, p + t, dtype=torch.int32) for p, t in zip(past, chunks)]) \
        if chunks else torch.zeros((0,), dtype=torch.int32)
    # Default capacity: the library's bound max_r P_r + max_r T_r.
    cap = capacity if capacity is not None else max(max(past + [0]) + max(chunks + [0]), 1)
    lens = torch.tensor(past, dtype=torch.int32)
    k_cache, v_cache = _fill_decode_cache(h, lens, cap, seed + 1, dtype, device, parity)
    return AppendInputs(heads=h, qkv=rows.to(device), q_norm_weight=wq.to(device), k_norm_weight=wk.to(device),
                        positions=positions.to(device),
                        cu_seqlens=torch.tensor(cu, dtype=torch.int32, device=device), seqlens=chunks,
                        cache_lens=lens.to(device), past_lens=past, cache_capacity=cap, k_cache=k_cache,
                        v_cache=v_cache)


# ---------------------------------------------------------------------------
# Paged caches: the same per-request cache contents stored in pages of a pool
# [num_pages, Hkv, P, D], found through a block table [B, pages_per_seq].
# Tables are random permutations of the pool's pages, so pages are out of
# order and the pool has pages no request owns (holes, filled like unused
# slots).  Values are the seeded contiguous contents, copied page by page.
# ---------------------------------------------------------------------------

@dataclasses.dataclass
class PagedCache:
    page_size: int
    block_table: torch.Tensor   # int32 [B, pages_per_seq]
    k_pool: torch.Tensor        # [num_pages, Hkv, page_size, D]
    v_pool: torch.Tensor

    @property
    def num_pages(self) -> int:
        return int(self.k_pool.shape[0])

    @property
    def pages_per_seq(self) -> int:
        return int(self.block_table.shape[1])


def make_block_table(num_seqs: int, pages_per_seq: int, num_pages: int, seed: int,
                     shared_prefix_pages: int = 0) -> torch.Tensor:
    """Distinct random pages for every (request, page index); with shared_prefix_pages = k every request's
    first k entries name the same k pages (a prefix stored once)."""
    own = pages_per_seq - shared_prefix_pages
    need = shared_prefix_pages + num_seqs * own
    if num_pages < need:
        raise ValueError(f"{num_pages} pages cannot hold {need}")
    g = torch.Generator().manual_seed(seed)
    perm = torch.randperm(num_pages, generator=g)
    shared = perm[:shared_prefix_pages]
    rest = perm[shared_prefix_pages:need].reshape(num_seqs, own)
    table = torch.cat([shared.expand(num_seqs, shared_prefix_pages), rest], dim=1)
    return table.to(torch.int32).contiguous()


def paged_from_contiguous(k_cache: torch.Tensor, v_cache: torch.Tensor, page_size: int, seed: int,
                          spare_pages: int = 3, parity: bool = True, shared_prefix_pages: int = 0) -> PagedCache:
    """A paged copy of contiguous caches [B, Hkv, S, D]: request b's slot s goes to row s % P of page
    table[b, s // P].  The pool holds `spare_pages` pages that no request owns.  With shared_prefix_pages = k the
    first k * P slots of request 0 are the shared prefix every request reads (the other requests' own values
    there are not kept)."""
    b, hkv, cap, d = k_cache.shape
    pps = max(1, -(-cap // page_size))
    num_pages = shared_prefix_pages + b * (pps - shared_prefix_pages) + spare_pages
    table = make_block_table(b, pps, num_pages, seed, shared_prefix_pages)
    fill = _sentinel(parity)
    pools = []
    for c in (k_cache, v_cache):
        pool = torch.full((num_pages, hkv, page_size, d), fill, dtype=c.dtype, device=c.device)
        padded = torch.full((b, hkv, pps * page_size, d), fill, dtype=c.dtype, device=c.device)
        padded[:, :, :cap] = c
        pages = padded.reshape(b, hkv, pps, page_size, d).permute(0, 2, 1, 3, 4)  # [B, pps, Hkv, P, D]
        tab = table.to(c.device).long()
        for r in reversed(range(b)):  # request 0 last: the shared pages hold its values
            pool[tab[r]] = pages[r]
        pools.append(pool)
    return PagedCache(page_size, table.to(k_cache.device), pools[0], pools[1])


# ---------------------------------------------------------------------------
# Named workloads.  Head shapes follow the Qwen3 configurations the pages
# trace (Qwen3-4B: 32 query heads, 8 KV heads, head_dim 128 -- "transformer
# basics", "Qwen3 analogies"); lengths and mixes are the benchmark's.
# ---------------------------------------------------------------------------

def _pages_t12_decode9(dtype, device, parity):
    # The pages' own run: a 12-token prompt, then 9 generated tokens, on
    # Qwen3-4B heads ("transformer basics", "Prefill vs Decode").
    h = HeadConfig(32, 8, 128, 1e-6, 1e6)
    g = torch.Generator().manual_seed(1000)
    rows = _draw_rows(g, 12 + 9, h, dtype)
    wq = _draw_norm_weight(g, h, dtype)
    wk = _draw_norm_weight(g, h, dtype)
    pre = _prefill_from_rows(h, rows[:12], wq, wk, [12], 21, dtype, device, parity)
    steps = [rows[12 + s: 13 + s].to(device) for s in range(9)]
    return WorkloadInputs("pages_t12_decode9",
                          "prefill T=12 then 9 chained decode steps, Hq=32 Hkv=8 D=128, base 1e6",
                          pre, None, steps)


def _single_t64(dtype, device, parity):
    h = HeadConfig(4, 2, 64, 1e-6, 1e4)
    g = torch.Generator().manual_seed(1001)
    rows = _draw_rows(g, 64 + 1, h, dtype)
    wq = _draw_norm_weight(g, h, dtype)
    wk = _draw_norm_weight(g, h, dtype)
    pre = _prefill_from_rows(h, rows[:64], wq, wk, [64], 65, dtype, device, parity)
    return WorkloadInputs("single_t64_hq4_hkv2_d64",
                          "one request T=64, Hq=4 Hkv=2 D=64, base 1e4; then one decode at position 64",
                          pre, None, [rows[64:65].to(device)])


def _qwen3_0p6b_varlen8(dtype, device, parity):
    h = HeadConfig(16, 8, 128, 1e-6, 1e6)
    g = torch.Generator().manual_seed(1002)
    lens = torch.randint(128, 2048 + 1, (8,), generator=g).tolist()
    rows = _draw_rows(g, int(sum(lens)), h, dtype)
    wq = _draw_norm_weight(g, h, dtype)
    wk = _draw_norm_weight(g, h, dtype)
    pre = _prefill_from_rows(h, rows, wq, wk, lens, max(lens), dtype, device, parity)
    return WorkloadInputs("qwen3_0p6b_prefill_varlen8",
                          "prefill of 8 packed requests, lengths U[128,2048], Hq=16 Hkv=8 D=128",
                          pre, None)


def _qwen3_4b_decode64(dtype, device, parity):
    h = HeadConfig(32, 8, 128, 1e-6, 1e6)
    g = torch.Generator().manual_seed(1003)
    lens = torch.randint(512, 8192 + 1, (64,), generator=g).to(torch.int32)
    rows = _draw_rows(g, 64, h, dtype)
    wq = _draw_norm_weight(g, h, dtype)
    wk = _draw_norm_weight(g, h, dtype)
    k, v = _fill_decode_cache(h, lens, 8193, 1003 + 1, dtype, device, parity)
    dec = DecodeInputs(h, rows.to(device), wq.to(device), wk.to(device), lens.clone().to(device),
                       lens.to(device), 8193, k, v)
    return WorkloadInputs("qwen3_4b_decode64",
                          "decode of 64 requests, cache lengths U[512,8192], Hq=32 Hkv=8 D=128",
                          None, dec)


def _long_prefill_32k(dtype, device, parity):
    h = HeadConfig(32, 8, 128, 1e-6, 1e6)
    g = torch.Generator().manual_seed(1004)
    rows = _draw_rows(g, 32768, h, dtype)
    wq = _draw_norm_weight(g, h, dtype)
    wk = _draw_norm_weight(g, h, dtype)
    pre = _prefill_from_rows(h, rows, wq, wk, [32768], 32768, dtype, device, parity)
    return WorkloadInputs("long_prefill_32k",
                          "one request T=32768, Hq=32 Hkv=8 D=128, base 1e6", pre, None)


def _mixed_qwen3_8b(dtype, device, parity):
    h = HeadConfig(32, 8, 128, 1e-6, 1e6)
    g = torch.Generator().manual_seed(1005)
    lens = torch.randint(1, 16384 + 1, (128,), generator=g).to(torch.int32)
    rows = _draw_rows(g, 4 * 4096 + 128, h, dtype)
    wq = _draw_norm_weight(g, h, dtype)
    wk = _draw_norm_weight(g, h, dtype)
    pre = _prefill_from_rows(h, rows[:4 * 4096], wq, wk, [4096] * 4, 4096, dtype, device, parity)
    k, v = _fill_decode_cache(h, lens, 16385, 1005 + 1, dtype, device, parity)
    dec = DecodeInputs(h, rows[4 * 4096:].contiguous().to(device), wq.to(device), wk.to(device),
                       lens.clone().to(device), lens.to(device), 16385, k, v)
    return WorkloadInputs("mixed_qwen3_8b",
                          "one step: prefill of 4x4096 tokens plus decode of 128 requests with cache "
                          "lengths U[1,16384], Hq=32 Hkv=8 D=128", pre, dec)


def _prefill_4x4096_qwen3_8b(dtype, device, parity):
    # The mixed step's prefill half alone: the same draws as mixed_qwen3_8b, without its decode caches.
    h = HeadConfig(32, 8, 128, 1e-6, 1e6)
    g = torch.Generator().manual_seed(1005)
    torch.randint(1, 16384 + 1, (128,), generator=g)  # the decode lengths, drawn first there
    rows = _draw_rows(g, 4 * 4096 + 128, h, dtype)
    wq = _draw_norm_weight(g, h, dtype)
    wk = _draw_norm_weight(g, h, dtype)
    pre = _prefill_from_rows(h, rows[:4 * 4096], wq, wk, [4096] * 4, 4096, dtype, device, parity)
    return WorkloadInputs("prefill_4x4096_qwen3_8b",
                          "the mixed step's prefill half alone: 4x4096 tokens, Hq=32 Hkv=8 D=128", pre, None)


def _chunked_qwen3_8b(dtype, device, parity):
    h = HeadConfig(32, 8, 128, 1e-6, 1e6)
    g = torch.Generator().manual_seed(1006)
    past = torch.randint(2048, 14336 + 1, (8,), generator=g).tolist()
    app = make_append_inputs(h, past, [2048] * 8, 1006, dtype, device, capacity=16384, parity=parity)
    return WorkloadInputs("chunked_qwen3_8b",
                          "2048-token chunks appended to 8 caches holding U[2048,14336] entries, "
                          "Hq=32 Hkv=8 D=128, base 1e6", None, None, append=app)


def make_norm_inputs(num_rows: int, hidden: int, seed: int, dtype=torch.bfloat16, device="cpu",
                     has_residual: bool = True, rms_eps: float = 1e-6) -> NormInputs:
    """x, then the residual stream (when there is one), N(0,1); then the weight 1 + 0.1 N(0,1)."""
    g = torch.Generator().manual_seed(seed)
    x = torch.randn((num_rows, hidden), generator=g, dtype=torch.float32).to(dtype)
    res = torch.randn((num_rows, hidden), generator=g, dtype=torch.float32).to(dtype) if has_residual else None
    w = (1.0 + 0.1 * torch.randn((hidden,), generator=g, dtype=torch.float32)).to(dtype)
    return NormInputs(x.to(device), None if res is None else res.to(device), w.to(device), rms_eps)


def make_next_token_inputs(seqlens: Sequence[int], hidden: int, vocab: int, seed: int, dtype=torch.bfloat16,
                           device="cpu") -> NextTokenInputs:
    """Hidden states N(0,1) for the packed requests, then one logits row per request N(0,1)."""
    g = torch.Generator().manual_seed(seed)
    n = int(sum(seqlens))
    cu = torch.zeros(len(seqlens) + 1, dtype=torch.int32)
    cu[1:] = torch.cumsum(torch.tensor(list(seqlens), dtype=torch.int64), 0).to(torch.int32)
    h = torch.randn((n, hidden), generator=g, dtype=torch.float32).to(dtype)
    z = torch.randn((len(seqlens), vocab), generator=g, dtype=torch.float32).to(dtype)
    return NextTokenInputs(h.to(device), cu.to(device), [int(t) for t in seqlens], z.to(device))


def _residual_rmsnorm_qwen3_8b(dtype, device, parity):
    norm = make_norm_inputs(4 * 4096 + 128, 4096, 1007, dtype, device, has_residual=True)
    return WorkloadInputs("residual_rmsnorm_qwen3_8b",
                          "fused residual add + RMSNorm over the mixed step's 16512 token rows, hidden 4096",
                          None, None, norm=norm)


def _next_token_qwen3_8b(dtype, device, parity):
    nt = make_next_token_inputs([4096] * 4 + [1] * 128, 4096, 151936, 1008, dtype, device)
    return WorkloadInputs("next_token_qwen3_8b",
                          "last-row gather over the mixed step's 132 requests (hidden 4096) and greedy argmax "
                          "over 132 logits rows of 151936", None, None, next_token=nt)


WORKLOADS: Dict[str, object] = {
    "pages_t12_decode9": _pages_t12_decode9,
    "single_t64_hq4_hkv2_d64": _single_t64,
    "qwen3_0p6b_prefill_varlen8": _qwen3_0p6b_varlen8,
    "qwen3_4b_decode64": _qwen3_4b_decode64,
    "long_prefill_32k": _long_prefill_32k,
    "mixed_qwen3_8b": _mixed_qwen3_8b,
    "chunked_qwen3_8b": _chunked_qwen3_8b,
    "prefill_4x4096_qwen3_8b": _prefill_4x4096_qwen3_8b,
    "residual_rmsnorm_qwen3_8b": _residual_rmsnorm_qwen3_8b,
    "next_token_qwen3_8b": _next_token_qwen3_8b,
}


def build_workload(name: str, dtype=torch.bfloat16, device="cpu", parity: bool = True) -> WorkloadInputs:
    try:
        fn = WORKLOADS[name]
    except KeyError:
        raise KeyError(f"unknown workload {name!r}; known: {sorted(WORKLOADS)}") from None
    return fn(dtype, device, parity)
