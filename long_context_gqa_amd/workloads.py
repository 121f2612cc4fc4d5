"""Seeded synthetic inputs for the target-verify path.

This module only draws random numbers and lays them out in the layouts the
library consumes. It holds none of the method's arithmetic: no attention, no
softmax, no argmax, no dequantisation. Both the CPU oracle tests and the GPU
path take their inputs from here.

Workloads follow the shapes of the pages:
  * the full-attention layer of the 27B hybrid model on the PocketLLM page
    ("Qwen3.8-27B-FP8", model specification table): 24 query heads, 4 KV
    heads, head dimension 256, vocabulary 248,320;
  * verify blocks of 8 (current token + 7 drafts) and 16 (DFlash block);
  * paged KV in 16- or 64-token pages, fp16 or FP8 E4M3 with per-token,
    per-KV-head fp16 scales over 64-channel blocks (PocketLLM page,
    "Implemented execution path" and "KV cache dtype").

Two value variants:
  * ``literal``: Q/K/V elements N(0,1)/sqrt(head_dim) as the workload
    statement gives them (FP8 K/V are quantised from N(0,1));
  * ``unit``: Q/K/V elements N(0,1), so attention logits have unit std and
    softmax rows are far from uniform.

Layouts (all row-major):
  q          [batch*q_len, num_q_heads, head_dim]            fp16
  k_pages    [num_pages, num_kv_heads, page_size, head_dim]   fp16 | uint8 (E4M3 codes)
  v_pages    same as k_pages
  k_scales   [num_pages, num_kv_heads, page_size, head_dim//64] fp16 (FP8 only)
  v_scales   same as k_scales
  page_table [batch, max_pages_per_req] int32, unused entries -1
  kv_lens    [batch] int32, prefix + q_len (the verify block's K/V is in the cache)
  logits     [batch*q_len, vocab] fp32
  draft_ids  [batch, q_len-1] int32

Slots past a request's kv_len in its last page and spare pages that no table
entry references are filled with NaN, so a kernel that reads them into a
result is caught.
"""
from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field, replace

import torch

NUM_Q_HEADS = 24
NUM_KV_HEADS = 4
HEAD_DIM = 256
VOCAB = 248_320
FP8_MAX = 448.0
FP16_NAN_BITS = 0x7E00
E4M3_NAN_CODE = 0x7F


@dataclass(frozen=True)
class Workload:
    """One synthetic verify workload."""

    name: str
    batch: int
    q_len: int
    prefix: tuple  # ("fixed", L) or ("uniform", lo, hi)
    page_size: int
    kv_dtype: str = "fp16"  # "fp16" | "fp8_e4m3"
    page_order: str = "per_request"  # "per_request" | "shared"
    bias_keys: bool = False
    accept_dist: str = "uniform"  # "uniform" over 0..q-1 | "geometric" p=0.5 capped
    seed: int = 0
    num_q_heads: int = NUM_Q_HEADS
    num_kv_heads: int = NUM_KV_HEADS
    head_dim: int = HEAD_DIM
    vocab: int = VOCAB

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


# The five workloads: single request at 4K, batch 8 at 32K, one request at
# 512K with biased keys, a ragged batch of 32 DFlash blocks at 8K-131K with
# 64-token pages in a shared pool, and FP8 E4M3 KV at 262K.
WORKLOADS = {
    1: Workload("b1_q8_ctx4k_fp16_p16", 1, 8, ("fixed", 4096), 16, seed=1001),
    2: Workload("b8_q8_ctx32k_fp16_p16", 8, 8, ("fixed", 32768), 16, seed=1002),
    3: Workload("b1_q8_ctx512k_fp16_p16_biased", 1, 8, ("fixed", 524288), 16,
                bias_keys=True, seed=1003),
    4: Workload("b32_q16_ctx8k-131k_fp16_p64_shared", 32, 16, ("uniform", 8192, 131072), 64,
                page_order="shared", accept_dist="geometric", seed=1004),
    5: Workload("b4_q8_ctx262k_fp8e4m3_p16", 4, 8, ("fixed", 262144), 16,
                kv_dtype="fp8_e4m3", seed=1005),
}


def _seed(base: int, stream: int, chunk: int = 0) -> int:
    # Fixed derivation of a 63-bit seed per (workload, stream, chunk); the
    # stream ids below are part of the recipe.
    return (base * 1_000_003 + stream * 10_007 + chunk * 7_919 + 12_345) & ((1 << 63) - 1)


S_PREFIX, S_PAGES, S_Q, S_K, S_V, S_BIAS, S_LOGITS, S_ACCEPT, S_DRAFT, S_WIDTH, S_SAMPLE = range(11)


def _gen(device, base, stream, chunk=0):
    g = torch.Generator(device=device)
    g.manual_seed(_seed(base, stream, chunk))
    return g


def prefix_lengths(wl: Workload) -> list[int]:
    if wl.prefix[0] == "fixed":
        return [int(wl.prefix[1])] * wl.batch
    _, lo, hi = wl.prefix
    g = _gen("cpu", wl.seed, S_PREFIX)
    return [int(x) for x in torch.randint(lo, hi + 1, (wl.batch,), generator=g)]


@dataclass
class VerifyInputs:
    wl: Workload
    variant: str
    kv_lens: torch.Tensor  # int32 [B] (host)
    page_table: torch.Tensor  # int32 [B, max_pages] (host)
    num_pages: int
    q: torch.Tensor
    k_pages: torch.Tensor
    v_pages: torch.Tensor
    k_scales: torch.Tensor | None
    v_scales: torch.Tensor | None
    sm_scale: float
    bias_positions: list = field(default_factory=list)  # [(b, g, [token positions])]

    @property
    def max_kv_len(self) -> int:
        return int(self.kv_lens.max())


@dataclass
class AcceptInputs:
    logits: torch.Tensor  # fp32 [B*q, V]
    draft_ids: torch.Tensor  # int32 [B, q-1]
    planted_accept: torch.Tensor  # int32 [B] (host)
    planted_targets: torch.Tensor  # int32 [B, q] (host): the planted peak of each row


def page_layout(wl: Workload, kv_lens: list[int], spare_pages: int | None = None):
    """Physical page ids for each request's logical pages.

    per_request: request b owns a contiguous block of physical pages whose
    order inside the block is a random permutation.
    shared: one pool in random order dealt out to the requests.
    Returns (page_table int32 [B, max_pages] with -1 padding, num_pages).
    """
    P = wl.page_size
    npg = [(n + P - 1) // P for n in kv_lens]
    total = sum(npg)
    if spare_pages is None:
        spare_pages = max(1, total // 64)
    num_pages = total + spare_pages
    g = _gen("cpu", wl.seed, S_PAGES)
    width = max(npg)
    table = torch.full((wl.batch, width), -1, dtype=torch.int32)
    if wl.page_order == "shared":
        perm = torch.randperm(num_pages, generator=g)[:total].to(torch.int32)
        off = 0
        for b, n in enumerate(npg):
            table[b, :n] = perm[off:off + n]
            off += n
    else:
        # spare pages sit at random places between request blocks
        base = 0
        for b, n in enumerate(npg):
            table[b, :n] = (torch.randperm(n, generator=g) + base).to(torch.int32)
            base += n
        if spare_pages:
            # rotate the whole id space so spare pages are not all at the end
            shift = int(torch.randint(0, num_pages, (1,), generator=g))
            used = table >= 0
            table[used] = (table[used] + shift) % num_pages
    return table, num_pages


def _fill_normal(out16: torch.Tensor, base: int, stream: int, sigma: float, device, chunk_pages: int):
    """Fill an fp16 tensor [num_pages, ...] with N(0, sigma^2) page-chunk by page-chunk."""
    n = out16.shape[0]
    chunks = [(i, min(n, i + chunk_pages)) for i in range(0, n, chunk_pages)]

    def work(ci):
        lo, hi = chunks[ci]
        g = _gen(device, base, stream, ci)
        x = torch.randn(out16[lo:hi].shape, generator=g, device=device, dtype=torch.float32)
        if sigma != 1.0:
            x.mul_(sigma)
        out16[lo:hi] = x.to(torch.float16)

    _run_chunks(work, len(chunks), device)


def _run_chunks(work, n, device):
    if str(device).startswith("cuda") or n == 1:
        for ci in range(n):
            work(ci)
    else:
        with ThreadPoolExecutor(max_workers=min(16, n, max(1, torch.get_num_threads()))) as ex:
            list(ex.map(work, range(n)))


def _fill_fp8(codes: torch.Tensor, scales: torch.Tensor, base: int, stream: int, device, chunk_pages: int):
    """Quantise N(0,1) data to E4M3 codes with one fp16 scale per 64 channels.

    scale = fp16(amax / 448) (1.0 for an all-zero block); code = E4M3 of
    clamp(x / scale, +-448) rounded to nearest even by torch's float8 cast.
    """
    n = codes.shape[0]
    chunks = [(i, min(n, i + chunk_pages)) for i in range(0, n, chunk_pages)]
    nb = codes.shape[-1] // 64

    def work(ci):
        lo, hi = chunks[ci]
        g = _gen(device, base, stream, ci)
        x = torch.randn(codes[lo:hi].shape, generator=g, device=device, dtype=torch.float32)
        xb = x.view(*x.shape[:-1], nb, 64)
        amax = xb.abs().amax(dim=-1)
        sc = (amax / FP8_MAX).to(torch.float16)
        sc = torch.where(amax == 0, torch.ones_like(sc), sc)
        y = (xb / sc.float().unsqueeze(-1)).clamp_(-FP8_MAX, FP8_MAX)
        codes[lo:hi] = y.view(x.shape).to(torch.float8_e4m3fn).view(torch.uint8)
        scales[lo:hi] = sc

    _run_chunks(work, len(chunks), device)


def make_verify_inputs(wl: Workload, variant: str = "literal", device="cpu",
                       kv_lens: list[int] | None = None, spare_pages: int | None = None,
                       poison: bool = True) -> VerifyInputs:
    """Build the attention inputs of one workload on ``device``.

    The random stream depends on (workload seed, device type): CPU and GPU
    draws differ, each is reproducible.
    """
    assert variant in ("literal", "unit")
    B, q, Hq, Hkv, D, P = wl.batch, wl.q_len, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.page_size
    if kv_lens is None:
        kv_lens = [L + q for L in prefix_lengths(wl)]
    table, num_pages = page_layout(wl, kv_lens, spare_pages)
    sig = 1.0 if variant == "unit" else 1.0 / math.sqrt(D)
    dev_type = torch.device(device).type
    gq = _gen(dev_type, wl.seed, S_Q)
    qt = torch.randn((B * q, Hq, D), generator=gq, device=device, dtype=torch.float32)
    qt = (qt * sig).to(torch.float16)
    chunk_pages = max(1, (1 << 22) // (Hkv * P * D))  # about 4M elements per chunk
    k_scales = v_scales = None
    if wl.kv_dtype == "fp16":
        kp = torch.empty((num_pages, Hkv, P, D), dtype=torch.float16, device=device)
        vp = torch.empty_like(kp)
        _fill_normal(kp, wl.seed, S_K, sig, dev_type, chunk_pages)
        _fill_normal(vp, wl.seed, S_V, sig, dev_type, chunk_pages)
    elif wl.kv_dtype == "fp8_e4m3":
        kp = torch.empty((num_pages, Hkv, P, D), dtype=torch.uint8, device=device)
        vp = torch.empty_like(kp)
        k_scales = torch.empty((num_pages, Hkv, P, D // 64), dtype=torch.float16, device=device)
        v_scales = torch.empty_like(k_scales)
        _fill_fp8(kp, k_scales, wl.seed, S_K, dev_type, chunk_pages)
        # (FP8 K/V are quantised from N(0,1) in both variants)
        _fill_fp8(vp, v_scales, wl.seed, S_V, dev_type, chunk_pages)
    else:
        raise ValueError(wl.kv_dtype)

    bias_positions = []
    if wl.bias_keys:
        bias_positions = _plant_key_bias(wl, kp, table, kv_lens, sig, device)

    if poison:
        _poison(wl, kp, vp, k_scales, v_scales, table, kv_lens, num_pages)

    return VerifyInputs(wl, variant, torch.tensor(kv_lens, dtype=torch.int32), table, num_pages,
                        qt, kp, vp, k_scales, v_scales, 1.0 / math.sqrt(D), bias_positions)


def _plant_key_bias(wl, kp, table, kv_lens, sig, device):
    """+4 sigma on every channel of a seeded subset of keys (1 in 4,096 per
    (request, KV head)), always including one key inside the verify block and
    one on a page boundary."""
    g = _gen("cpu", wl.seed, S_BIAS)
    P, q = wl.page_size, wl.q_len
    out = []
    for b, n in enumerate(kv_lens):
        L = n - q
        for h in range(wl.num_kv_heads):
            cnt = max(2, n // 4096)
            pos = set(int(x) for x in torch.randint(0, n, (cnt,), generator=g))
            pos.add(L + int(torch.randint(0, q, (1,), generator=g)))
            pos.add(P * int(torch.randint(0, max(1, L // P), (1,), generator=g)))
            pos = sorted(pos)
            for t in pos:
                page = int(table[b, t // P])
                row = kp[page, h, t % P].float() + 4.0 * sig
                kp[page, h, t % P] = row.to(kp.dtype)
            out.append((b, h, pos))
    return out


def _poison(wl, kp, vp, ks, vs, table, kv_lens, num_pages):
    """NaN in slots no valid token owns: the tail of each request's last page
    and every spare page."""
    P = wl.page_size
    nan_code = FP16_NAN_BITS if kp.dtype == torch.float16 else E4M3_NAN_CODE
    used = torch.zeros(num_pages, dtype=torch.bool)
    for b, n in enumerate(kv_lens):
        npg = (n + P - 1) // P
        used[table[b, :npg].long()] = True
        if n % P:
            last = int(table[b, npg - 1])
            for t in (kp, vp):
                t.view(torch.int16 if t.dtype == torch.float16 else torch.uint8)[last, :, n % P:] = \
                    _as_bits(nan_code, t.dtype)
            for s in (ks, vs):
                if s is not None:
                    s.view(torch.int16)[last, :, n % P:] = _as_bits(FP16_NAN_BITS, torch.float16)
    spare = (~used).nonzero().flatten()
    if len(spare):
        idx = spare.to(kp.device)
        for t in (kp, vp):
            t.view(torch.int16 if t.dtype == torch.float16 else torch.uint8)[idx] = _as_bits(nan_code, t.dtype)
        for s in (ks, vs):
            if s is not None:
                s.view(torch.int16)[idx] = _as_bits(FP16_NAN_BITS, torch.float16)


def _as_bits(code, dtype):
    if dtype == torch.float16:
        return code - (1 << 16) if code >= (1 << 15) else code
    return code


def make_accept_inputs(wl: Workload, device="cpu", planted: list[int] | None = None) -> AcceptInputs:
    """fp32 logits N(0,1) [B*q, V] with a planted peak (value 8.0) in every
    row, and draft ids built so that the first A* drafts equal the planted
    peaks of rows 0..A*-1 and draft A* does not equal row A*'s peak."""
    B, q, V = wl.batch, wl.q_len, wl.vocab
    dev_type = torch.device(device).type
    gl = _gen(dev_type, wl.seed, S_LOGITS)
    logits = torch.randn((B * q, V), generator=gl, device=device, dtype=torch.float32)
    ga = _gen("cpu", wl.seed, S_ACCEPT)
    if planted is None:
        if wl.accept_dist == "uniform":
            planted = [int(x) for x in torch.randint(0, q, (B,), generator=ga)]
        elif wl.accept_dist == "geometric":
            # P(A = k) = 0.5^(k+1) on k = 0, 1, ...; capped at 15 and at q-1
            u = torch.rand((B,), generator=ga, dtype=torch.float64)
            planted = [min(int(math.floor(math.log(1.0 - float(x)) / math.log(0.5))), 15, q - 1) for x in u]
        else:
            raise ValueError(wl.accept_dist)
    gd = _gen("cpu", wl.seed, S_DRAFT)
    targets = torch.randint(0, V, (B, q), generator=gd, dtype=torch.int64)
    drafts = torch.randint(0, V, (B, max(q - 1, 0)), generator=gd, dtype=torch.int64)
    for b in range(B):
        a = planted[b]
        for j in range(q - 1):
            if j < a:
                drafts[b, j] = targets[b, j]
            elif j == a:
                off = int(torch.randint(1, V, (1,), generator=gd))
                drafts[b, j] = (targets[b, j] + off) % V
    rows = torch.arange(B * q, device=device)
    logits[rows, targets.flatten().to(device)] = 8.0
    return AcceptInputs(logits, drafts.to(torch.int32).to(device),
                        torch.tensor(planted, dtype=torch.int32), targets.to(torch.int32))


@dataclass
class SamplingInputs:
    draft_probs: torch.Tensor  # fp32 [B, q-1, V]: each row a distribution
    draft_ids: torch.Tensor    # int32 [B, q-1], drawn from draft_probs
    u_accept: torch.Tensor     # fp32 [B, q-1] uniforms on [0, 1)
    u_final: torch.Tensor      # fp32 [B]


def make_sampling_inputs(wl: Workload, device="cpu") -> SamplingInputs:
    """The draft side of a stochastic verify: a distribution per draft
    position (normalised exponential draws, i.e. Dirichlet(1) over the
    vocabulary), the draft tokens drawn from them, and the uniforms of the
    acceptance tests and of the final draw. Random numbers only."""
    B, q, V = wl.batch, wl.q_len, wl.vocab
    g = _gen(torch.device(device).type, wl.seed, S_SAMPLE)
    e = torch.empty((B, max(q - 1, 0), V), dtype=torch.float32, device=device).exponential_(generator=g)
    probs = e / e.sum(dim=-1, keepdim=True)
    ids = torch.multinomial(probs.view(-1, V), 1, generator=g).view(B, max(q - 1, 0)).to(torch.int32) \
        if q > 1 else torch.zeros((B, 0), dtype=torch.int32, device=device)
    ua = torch.rand((B, max(q - 1, 0)), generator=g, device=device)
    uf = torch.rand((B,), generator=g, device=device)
    return SamplingInputs(probs.contiguous(), ids.contiguous(), ua.contiguous(), uf.contiguous())


def rejection_accept_bytes(batch, q_len, vocab) -> int:
    """Target logits read once, the draft distribution of the first rejected
    row, the tested draft elements, uniforms and outputs."""
    return batch * q_len * vocab * 4 + batch * vocab * 4 + batch * max(q_len - 1, 0) * (4 + 4 + 4) + 4 * batch * 4


# ---------------------------------------------------------------------------
# Blocks of a width per request

def block_widths(wl: Workload, lo: int = 2) -> list[int]:
    """Seeded per-request verify widths, uniform over lo..q_len. (An adaptive
    width policy verifies at least two rows and at most the block, PocketLLM
    page, DFlash2 adaptive width; the draw stands in for such a policy.)"""
    g = _gen("cpu", wl.seed, S_WIDTH)
    return [int(x) for x in torch.randint(lo, wl.q_len + 1, (wl.batch,), generator=g)]


def pack_rows(t: torch.Tensor, q_len: int, widths: list[int]) -> torch.Tensor:
    """The first widths[b] of request b's q_len rows of t, packed request by
    request (the row layout of blocks of different widths)."""
    return torch.cat([t[b * q_len:b * q_len + w] for b, w in enumerate(widths)], 0).contiguous()


def row_offsets(widths: list[int]) -> torch.Tensor:
    """int32 [B+1]: where each request's rows start in the packed layout."""
    out = [0]
    for w in widths:
        out.append(out[-1] + int(w))
    return torch.tensor(out, dtype=torch.int32)


# ---------------------------------------------------------------------------
# Byte accounting (what one verify must move at minimum)

def kv_bytes_per_token_head(head_dim: int, kv_dtype: str) -> int:
    """K and V bytes for one token of one KV head, scales included."""
    if kv_dtype == "fp16":
        return 2 * head_dim * 2
    if kv_dtype == "fp8_e4m3":
        return 2 * head_dim * 1 + 2 * (head_dim // 64) * 2
    raise ValueError(kv_dtype)


def verify_algorithmic_bytes(kv_lens, q_len, num_q_heads, num_kv_heads, head_dim, page_size, kv_dtype) -> int:
    """Visible K/V (+scales) of every request read once, Q read, out written,
    the page-table entries in use and kv_lens. Split partials excluded.
    q_len: one width for every request, or a list of per-request widths
    (then the row offsets, B+1 int32, are counted too)."""
    kv_lens = [int(x) for x in kv_lens]
    B = len(kv_lens)
    kv = sum(kv_lens) * num_kv_heads * kv_bytes_per_token_head(head_dim, kv_dtype)
    rows = B * q_len if isinstance(q_len, int) else sum(int(w) for w in q_len)
    qo = 2 * rows * num_q_heads * head_dim * 2
    pt = sum((n + page_size - 1) // page_size for n in kv_lens) * 4
    offs = 0 if isinstance(q_len, int) else 4 * (B + 1)
    return kv + qo + pt + 4 * B + offs


def accept_algorithmic_bytes(batch, q_len, vocab) -> int:
    """fp32 logits read once, drafts read, accept/bonus written."""
    return batch * q_len * vocab * 4 + batch * max(q_len - 1, 0) * 4 + 2 * batch * 4
