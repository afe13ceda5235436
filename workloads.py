"""Seeded synthetic inputs for the NVFP4 paged-KV append + causal prefill path.

This module only draws inputs: bf16 Q/K/V, global decode scales, page tables,
slot mappings and request lengths.  It holds none of the method's arithmetic
(no quantization, no attention) and is the one module that both the HIP path's
tests/benchmark and the oracle's checks take their inputs from.

Every draw comes from torch's counter-based (Philox) generator seeded with
(seed, stream), so a workload is reproducible on a given device; values drawn
on the CPU differ from values drawn on the GPU, and a test uses one or the
other throughout.

The shapes follow the workloads the source pages discuss (Qwen3-8B attention
shapes: 32 query heads, 8 KV heads, head_dim 128; page size 16; the 2048x2048
prefill of the PR #4769 page; the batch-1024 / seqlen-1024 case of the
PR #3575 page; chunked prefill from the PR #6204 page).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch

# streams of the per-workload generator
Q_STREAM, K_STREAM, V_STREAM, PAGE_STREAM, LEN_STREAM, SCALE_STREAM, SLOT_STREAM = range(7)


def _gen(seed: int, stream: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(1_000_003 * (seed + 1) + 7919 * stream)
    return g


def normal_bf16(shape, seed, stream, device, std=1.0, chunk_rows=1 << 16) -> torch.Tensor:
    """bf16 tensor ~ std * N(0,1), drawn in fp32 and rounded to nearest-even."""
    g = _gen(seed, stream, device)
    out = torch.empty(shape, dtype=torch.bfloat16, device=device)
    flat = out.view(shape[0], math.prod(shape[1:]))  # (also for zero rows)
    for r0 in range(0, shape[0], chunk_rows):
        r1 = min(shape[0], r0 + chunk_rows)
        x = torch.randn((r1 - r0, flat.shape[1]), generator=g, device=device, dtype=torch.float32)
        if std != 1.0:
            x.mul_(std)
        flat[r0:r1] = x.to(torch.bfloat16)
    return out


def student_t3_bf16(shape, seed, stream, device, chunk_rows=1 << 14) -> torch.Tensor:
    """bf16 tensor ~ Student-t with 3 degrees of freedom: Z / sqrt(chi2_3 / 3)."""
    g = _gen(seed, stream, device)
    out = torch.empty(shape, dtype=torch.bfloat16, device=device)
    flat = out.view(shape[0], math.prod(shape[1:]))  # (also for zero rows)
    for r0 in range(0, shape[0], chunk_rows):
        r1 = min(shape[0], r0 + chunk_rows)
        n = (r1 - r0, flat.shape[1])
        z = torch.randn(n, generator=g, device=device, dtype=torch.float32)
        c = torch.zeros(n, device=device, dtype=torch.float32)
        for _ in range(3):
            w = torch.randn(n, generator=g, device=device, dtype=torch.float32)
            c.addcmul_(w, w)
        flat[r0:r1] = (z / torch.sqrt(c / 3.0)).to(torch.bfloat16)
    return out


def lognormal_scales(seed, mu, sigma, n=2):
    """n fp32 values exp(mu + sigma Z), drawn on the CPU."""
    g = _gen(seed, SCALE_STREAM, "cpu")
    z = torch.randn(n, generator=g, dtype=torch.float64)
    return [float(np.float32(math.exp(mu + sigma * float(t)))) for t in z]


def amax_scale(x: torch.Tensor) -> float:
    """Per-tensor global decode scale amax(|x|) / (6 * 448) (fp32)."""
    a = x.float().abs().amax().item()
    return float(np.float32(np.float32(a) / np.float32(6.0 * 448.0)))


def permutation(n, seed, stream, device="cpu") -> torch.Tensor:
    return torch.randperm(n, generator=_gen(seed, stream, "cpu")).to(device)


@dataclass
class AttentionWorkload:
    """A batch of requests: K/V for every cached position (appended through the
    slot mapping), Q for the trailing q_len positions of each request."""
    name: str
    q_lens: np.ndarray          # int32 [B]
    kv_lens: np.ndarray         # int32 [B]
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    page_size: int
    num_pages: int
    sm_scale: float
    k_scale: float
    v_scale: float
    qo_indptr: np.ndarray       # int32 [B+1]
    kv_indptr: np.ndarray       # int32 [B+1] (into page_table)
    page_table: np.ndarray      # int32 [sum ceil(kv/ps)]
    kv_token_indptr: np.ndarray  # int64 [B+1] (row offsets into k/v)
    q: torch.Tensor             # bf16 [total_q, H_q, D]
    k: torch.Tensor             # bf16 [total_kv, H_kv, D]
    v: torch.Tensor
    slot_mapping: torch.Tensor  # int64 [total_kv]
    meta: dict = field(default_factory=dict)

    @property
    def batch(self):
        return int(self.kv_lens.shape[0])


@dataclass
class AppendWorkload:
    name: str
    num_kv_heads: int
    head_dim: int
    page_size: int
    num_pages: int
    k_scale: float
    v_scale: float
    k: torch.Tensor             # bf16 [T, H_kv, D]
    v: torch.Tensor
    slot_mapping: torch.Tensor  # int64 [T]


def _pages_and_slots(q_lens, kv_lens, page_size, num_pages, seed, device):
    B = len(kv_lens)
    npages = (kv_lens + page_size - 1) // page_size
    need = int(npages.sum())
    assert need <= num_pages, "page pool too small"
    perm = permutation(num_pages, seed, PAGE_STREAM).numpy().astype(np.int32)
    kv_indptr = np.zeros(B + 1, np.int32)
    kv_indptr[1:] = np.cumsum(npages)
    page_table = perm[:need].copy()
    kv_tok = np.zeros(B + 1, np.int64)
    kv_tok[1:] = np.cumsum(kv_lens.astype(np.int64))
    # slot of token j of request r: page_table[kv_indptr[r] + j // ps] * ps + j % ps
    req = np.repeat(np.arange(B), kv_lens)
    j = np.arange(int(kv_tok[-1]), dtype=np.int64) - kv_tok[req]
    slots = page_table[kv_indptr[req] + j // page_size].astype(np.int64) * page_size + j % page_size
    qo = np.zeros(B + 1, np.int32)
    qo[1:] = np.cumsum(q_lens)
    return kv_indptr, page_table, kv_tok, torch.from_numpy(slots).to(device), qo


def make_attention(name, q_lens, kv_lens, num_q_heads, num_kv_heads, head_dim, page_size,
                   num_pages, seed, device, std=1.0, scales="one", sm_scale=None,
                   lognormal=(-4.0, 0.5)) -> AttentionWorkload:
    q_lens = np.asarray(q_lens, np.int32)
    kv_lens = np.asarray(kv_lens, np.int32)
    kv_indptr, page_table, kv_tok, slots, qo = _pages_and_slots(
        q_lens, kv_lens, page_size, num_pages, seed, device)
    total_q, total_kv = int(qo[-1]), int(kv_tok[-1])
    q = normal_bf16((total_q, num_q_heads, head_dim), seed, Q_STREAM, device, std)
    k = normal_bf16((total_kv, num_kv_heads, head_dim), seed, K_STREAM, device, std)
    v = normal_bf16((total_kv, num_kv_heads, head_dim), seed, V_STREAM, device, std)
    if scales == "one":
        ks, vs = 1.0, 1.0
    elif scales == "amax":
        ks, vs = amax_scale(k), amax_scale(v)
    elif scales == "lognormal":
        ks, vs = lognormal_scales(seed, *lognormal)
    else:
        raise ValueError(scales)
    return AttentionWorkload(
        name, q_lens, kv_lens, num_q_heads, num_kv_heads, head_dim, page_size, num_pages,
        float(sm_scale if sm_scale is not None else 1.0 / math.sqrt(head_dim)), ks, vs, qo,
        kv_indptr, page_table, kv_tok, q, k, v, slots)


# ---------------------------------------------------------------------------
# The five workloads.  Seeds are the workload's position in this list.
# ---------------------------------------------------------------------------

def tiny(device="cpu") -> AttentionWorkload:
    """2 requests x 128/128, 4 Q heads / 2 KV heads, head_dim 64, page 16,
    pages from a random permutation of 32, scales 1.0, sm_scale 1/8."""
    return make_attention("tiny_2x128_h4_kv2_d64", [128, 128], [128, 128], 4, 2, 64, 16, 32,
                          seed=0, device=device, scales="one", sm_scale=1.0 / 8.0)


def prefill_2k(device="cpu") -> AttentionWorkload:
    """1 request x 2048/2048, 32 Q / 8 KV heads, head_dim 128, page 16,
    scales = per-tensor amax / (6*448)."""
    return make_attention("prefill_1x2048_h32_kv8_d128", [2048], [2048], 32, 8, 128, 16, 128,
                          seed=1, device=device, scales="amax")


def uniform_batch_1k(device="cpu", batch=1024) -> AttentionWorkload:
    """1024 requests x 1024/1024, 32/8 heads, head_dim 128, values 0.5*N(0,1),
    scales lognormal(-4, 0.5), random page table over 65536 pages."""
    return make_attention(f"uniform_{batch}x1024_h32_kv8_d128", [1024] * batch, [1024] * batch,
                          32, 8, 128, 16, 65536 * batch // 1024, seed=2, device=device, std=0.5,
                          scales="lognormal", lognormal=(-4.0, 0.5))


def ragged_chunked(device="cpu", batch=256) -> AttentionWorkload:
    """256 requests, kv_len ~ U[1, 4096], q_len = min(kv_len, 512) (the trailing
    chunk), 32/8 heads, head_dim 128, scales per-tensor amax / (6*448)."""
    g = _gen(3, LEN_STREAM, "cpu")
    kv = torch.randint(1, 4097, (batch,), generator=g).numpy().astype(np.int32)
    q = np.minimum(kv, 512).astype(np.int32)
    pool = int(((kv + 15) // 16).sum())
    w = make_attention(f"ragged_{batch}_kvU1-4096_q512_h32_kv8_d128", q, kv, 32, 8, 128, 16,
                       pool, seed=3, device=device, scales="amax")
    return w


def steady_state(device="cpu", batch=64, q_len=32, kv_len=8192) -> AttentionWorkload:
    """64 requests x 32 queries at the end of 8192 keys each, 32/8 heads,
    head_dim 128, page 16, random page table, scales per-tensor amax /
    (6*448): every 4-wave Q tile visits 128 KV tiles, so the prefill runs
    equal-cost tiles, two per CU, with a negligible prologue."""
    return make_attention(f"steady_{batch}x{q_len}x{kv_len}_h32_kv8_d128", [q_len] * batch, [kv_len] * batch,
                          32, 8, 128, 16, batch * kv_len // 16 + 8, seed=6, device=device, scales="amax")


def decode_batch(device="cpu", batch=32, kv_len=8192) -> AttentionWorkload:
    """One decode step: 32 requests x 1 new query token over 8192 cached keys
    each (the token at position kv_len - 1), 32/8 heads, head_dim 128, page
    16, random page table, scales per-tensor amax / (6*448)."""
    return make_attention(f"decode_{batch}x{kv_len}_h32_kv8_d128", [1] * batch, [kv_len] * batch,
                          32, 8, 128, 16, batch * kv_len // 16, seed=5, device=device, scales="amax")


def append_stress(device="cpu", tokens=65536) -> AppendWorkload:
    """65536 new tokens, 8 KV heads x head_dim 128, page 16, 32768 pages; slot
    mapping = first T entries of a seeded permutation of all slots; values
    Student-t(3); scales lognormal(-4, 1)."""
    H, D, ps, P = 8, 128, 16, 32768
    k = student_t3_bf16((tokens, H, D), 4, K_STREAM, device)
    v = student_t3_bf16((tokens, H, D), 4, V_STREAM, device)
    slots = permutation(P * ps, 4, SLOT_STREAM)[:tokens].to(torch.int64).to(device)
    ks, vs = lognormal_scales(4, -4.0, 1.0)
    return AppendWorkload(f"append_{tokens}tok_h8_d128", H, D, ps, P, ks, vs, k, v, slots)


ATTENTION_WORKLOADS = {"tiny": tiny, "prefill_2k": prefill_2k, "uniform_batch_1k": uniform_batch_1k,
                       "ragged_chunked": ragged_chunked, "decode_batch": decode_batch}


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """Host uint16 view of a bf16 tensor's bit patterns."""
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)
