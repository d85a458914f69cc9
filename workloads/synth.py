"""Seeded synthetic workloads for the selected-token logprob and the three-way
comparison.

Shapes follow the Qwen3-style scoring workloads the pages discuss (hidden size
2048/4096, vocabulary 151 936 rows, 512-2048-token responses); no dataset or
trained weight exists here, so every value is drawn from a seeded generator:

* hidden rows: bf16 N(0, 1), optionally followed by an RMSNorm-style per-row
  rescale x / sqrt(mean(x^2) + 1e-6) taken in fp32 before the bf16 rounding;
* LM-head weight: bf16 N(0, std) with std = 1/sqrt(H) for the tiny case and
  0.02 for the Qwen-shaped cases (the second argument of N is a standard
  deviation);
* target ids: uniform, or Zipf(1.1) over the finite vocabulary support
  P(k) proportional to (k + 1)^-1.1, drawn by inverse CDF;
* comparison records: 256 prompt positions (masked out), a response of
  uniform length in [1, 2048] whose last token is EOS, padding afterwards.

Normals come from Box-Muller over PCG64 uniforms (numpy's own normal sampler
is an order of magnitude slower on this host); only reproducibility matters,
not the particular sampler. bf16 values are stored as their uint16 bit
patterns, rounded to nearest-even from fp32.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

BASE_SEED = 1234  # the fixture seed the AMD blog's experiments use

# Per-tensor seed offsets, so every tensor of every workload has its own stream.
_OFF_X, _OFF_W, _OFF_IDS, _OFF_ROWSCALE = 0, 1, 2, 3
_OFF_TINY, _OFF_QWEN, _OFF_PROBE, _OFF_FILL, _OFF_CMP, _OFF_STALE = (
    100, 200, 300, 400, 500, 600)


def _rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(int(seed)))


def normal_f32(seed: int, n: int, std: float = 1.0,
               chunk: int = 1 << 23) -> np.ndarray:
    """n float32 samples of N(0, std^2) via Box-Muller on PCG64 uniforms."""
    out = np.empty(n, dtype=np.float32)
    rng = _rng(seed)
    half = (min(chunk, n) + 1) // 2
    # Work buffers are reused across chunks: first-touch of fresh pages is the
    # dominant cost on some hosts.
    u1 = np.empty(half, np.float32)
    u2 = np.empty(half, np.float32)
    r = np.empty(half, np.float32)
    z = np.empty(2 * half, np.float32)
    pos = 0
    while pos < n:
        m = min(chunk, n - pos)
        h = (m + 1) // 2
        a, b_, rr, zz = u1[:h], u2[:h], r[:h], z[:2 * h]
        rng.random(out=a, dtype=np.float32)
        np.subtract(np.float32(1.0), a, out=a)     # (0, 1]: log is finite
        rng.random(out=b_, dtype=np.float32)
        np.log(a, out=rr)
        np.multiply(rr, np.float32(-2.0), out=rr)
        np.sqrt(rr, out=rr)
        np.multiply(rr, np.float32(std), out=rr)
        np.multiply(b_, np.float32(2.0 * np.pi), out=b_)
        np.cos(b_, out=a)
        np.multiply(rr, a, out=zz[:h])
        np.sin(b_, out=a)
        np.multiply(rr, a, out=zz[h:])
        out[pos:pos + m] = zz[:m]
        pos += m
    return out


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest, ties to even); return the uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).reshape(-1).view(np.uint32)
    out = np.empty(u.shape, np.uint16)
    step = 1 << 22
    t = np.empty(min(step, u.size), np.uint32)
    for p in range(0, u.size, step):
        s = u[p:p + step]
        tt = t[:s.size]
        np.right_shift(s, np.uint32(16), out=tt)
        np.bitwise_and(tt, np.uint32(1), out=tt)
        np.add(tt, np.uint32(0x7FFF), out=tt)
        np.add(tt, s, out=tt)
        np.right_shift(tt, np.uint32(16), out=tt)
        out[p:p + s.size] = tt
    return out.reshape(np.shape(x))


def f32_from_bf16_bits(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32)
            << np.uint32(16)).view(np.float32)


def uniform_ids(seed: int, n: int, V: int) -> np.ndarray:
    return _rng(seed).integers(0, V, size=n, dtype=np.int64)


def zipf_ids(seed: int, n: int, V: int, s: float = 1.1) -> np.ndarray:
    """Zipf(s) over the finite support [0, V): P(k) ~ (k + 1)^-s."""
    w = np.arange(1, V + 1, dtype=np.float64) ** (-s)
    cdf = np.cumsum(w)
    cdf /= cdf[-1]
    u = _rng(seed).random(n)
    ids = np.searchsorted(cdf, u, side="right")
    return np.minimum(ids, V - 1).astype(np.int64)


def rmsnorm_rows_f32(x: np.ndarray, eps: float = 1e-6) -> np.ndarray:
    """Per-row RMS rescale in fp32 (shapes the hidden rows like a final norm)."""
    x = x.astype(np.float32, copy=False)
    ms = np.mean(x.astype(np.float64) ** 2, axis=1, keepdims=True)
    return (x / np.sqrt(ms + eps).astype(np.float32)).astype(np.float32)


@dataclass
class ScoreCase:
    """Inputs of one selected-token-logprob call (bf16 as uint16 bits)."""
    name: str
    x_bits: np.ndarray          # [T, H] uint16
    w_bits: np.ndarray          # [V, H] uint16
    ids: np.ndarray             # [T] int64
    temperature: float = 1.0
    v_true: int | None = None   # defaults to V
    meta: dict = field(default_factory=dict)

    @property
    def T(self): return self.x_bits.shape[0]

    @property
    def H(self): return self.x_bits.shape[1]

    @property
    def V(self): return self.w_bits.shape[0]


def _hidden_bits(seed: int, T: int, H: int, rms: bool) -> np.ndarray:
    x = normal_f32(seed, T * H).reshape(T, H)
    if rms:
        x = rmsnorm_rows_f32(x)
    return bf16_bits_from_f32(x)


def _weight_bits(seed: int, V: int, H: int, std: float) -> np.ndarray:
    return bf16_bits_from_f32(normal_f32(seed, V * H, std)).reshape(V, H)


def tiny_case(T: int = 64, H: int = 256, V: int = 4096, seed: int = 0,
              temperature: float = 1.0) -> ScoreCase:
    """Tiny fused logprob: X bf16 N(0,1), W bf16 N(0, 1/sqrt(H)), uniform ids."""
    b = BASE_SEED + _OFF_TINY + 16 * seed
    return ScoreCase(
        name=f"tiny T={T} H={H} V={V}",
        x_bits=_hidden_bits(b + _OFF_X, T, H, rms=False),
        w_bits=_weight_bits(b + _OFF_W, V, H, 1.0 / np.sqrt(H)),
        ids=uniform_ids(b + _OFF_IDS, T, V),
        temperature=temperature)


def qwen_weight(H: int, V: int = 151936, seed: int = 0) -> np.ndarray:
    """Qwen3-shaped LM head: bf16 N(0, 0.02), [V, H]."""
    return _weight_bits(BASE_SEED + _OFF_QWEN + 16 * seed + _OFF_W + H, V, H, 0.02)


def qwen_case(T: int, H: int, V: int = 151936, seed: int = 0,
              temperature: float = 1.0, w_bits: np.ndarray | None = None) -> ScoreCase:
    """Qwen3-shaped scoring: RMS-scaled bf16 hidden rows, bf16 N(0, 0.02) LM
    head, Zipf(1.1) target ids."""
    b = BASE_SEED + _OFF_QWEN + 16 * seed
    if w_bits is None:
        w_bits = qwen_weight(H, V, seed)
    return ScoreCase(
        name=f"qwen T={T} H={H} V={V}",
        x_bits=_hidden_bits(b + _OFF_X + 7 * T, T, H, rms=True),
        w_bits=w_bits,
        ids=zipf_ids(b + _OFF_IDS + 7 * T, T, V),
        temperature=temperature)


def probe_set(H: int = 4096, V: int = 151936, n: int = 512, seed: int = 0):
    """Fixed probe rows (RMS-scaled bf16) and Zipf target ids."""
    b = BASE_SEED + _OFF_PROBE + 16 * seed
    return _hidden_bits(b + _OFF_X, n, H, rms=True), zipf_ids(b + _OFF_IDS, n, V)


def filler_rows(seed: int, n: int, H: int, V: int):
    """Unrelated bf16 N(0,1) rows with uniform target ids."""
    b = BASE_SEED + _OFF_FILL + 16 * seed
    return _hidden_bits(b + _OFF_X, n, H, rms=False), uniform_ids(b + _OFF_IDS, n, V)


# ---------------------------------------------------------------------------
# Three-way comparison records
# ---------------------------------------------------------------------------

@dataclass
class CompareCase:
    """Response-aligned generation (A), replay (B) and trainer (C) scores."""
    name: str
    A: np.ndarray      # [N, L] float32
    B: np.ndarray
    C: np.ndarray
    mask: np.ndarray   # [N, L] uint8
    prompt_len: int
    resp_len: np.ndarray  # [N] int64, includes the EOS token
    meta: dict = field(default_factory=dict)

    @property
    def N(self): return self.mask.shape[0]

    @property
    def L(self): return self.mask.shape[1]


def _record_layout(seed: int, N: int, prompt: int, max_resp: int):
    L = prompt + max_resp
    resp = _rng(seed).integers(1, max_resp + 1, size=N, dtype=np.int64)
    pos = np.arange(L)[None, :]
    mask = ((pos >= prompt) & (pos < prompt + resp[:, None])).astype(np.uint8)
    return L, resp, mask


def compare_case(N: int = 8, max_resp: int = 2048, prompt: int = 256,
                 seed: int = 0, B: np.ndarray | None = None) -> CompareCase:
    """Baseline record with A = B bitwise and C = B bitwise on the response.

    B defaults to logprob-shaped values log(U), U ~ uniform(0, 1]; a caller may
    pass its own [N, prompt + max_resp] float32 B (for example scores from the
    oracle). Prompt positions hold finite garbage in all three arrays, and C
    holds NaN after EOS, so that only masked-in tokens may affect results.
    """
    b = BASE_SEED + _OFF_CMP + 16 * seed
    L, resp, mask = _record_layout(b, N, prompt, max_resp)
    if B is None:
        u = 1.0 - _rng(b + 1).random((N, L))
        B = np.log(u).astype(np.float32)
    B = np.array(B, dtype=np.float32, copy=True)
    garbage = (normal_f32(b + 2, N * L, 30.0).reshape(N, L))
    outside = mask == 0
    B[outside] = garbage[outside]
    A = B.copy()
    C = B.copy()
    after_eos = np.arange(L)[None, :] >= (prompt + resp[:, None])
    C[after_eos] = np.nan
    return CompareCase("baseline", A, B, C, mask, prompt, resp)


def offset_scores(x: np.ndarray, mask: np.ndarray, offset: float,
                  first_pos: int = 0) -> np.ndarray:
    """Subtract `offset` nat (in fp64, rounded to fp32) from masked-in tokens at
    active index >= first_pos: the blog's injected score faults (Case 1: A at
    response positions >= 1; Case 2: C everywhere)."""
    y = x.copy()
    rank = np.cumsum(mask, axis=1) - 1
    sel = (mask != 0) & (rank >= first_pos)
    y[sel] = (x[sel].astype(np.float64) - offset).astype(np.float32)
    return y


def noise_scores(x: np.ndarray, mask: np.ndarray, std: float, seed: int) -> np.ndarray:
    """x + N(0, std) on masked-in tokens, rounded to fp32."""
    y = x.copy()
    z = normal_f32(BASE_SEED + _OFF_CMP + 7 + seed, x.size, std).reshape(x.shape)
    sel = mask != 0
    y[sel] = (x[sel].astype(np.float64) + z[sel].astype(np.float64)).astype(np.float32)
    return y


def shift_scores(x: np.ndarray, seq: int, k: int, fill: float = np.nan) -> np.ndarray:
    """Misalign one sequence by k positions: y[seq, i] = x[seq, i + k]."""
    y = x.copy()
    L = x.shape[1]
    row = np.full(L, fill, dtype=np.float32)
    if k >= 0:
        row[:L - k] = x[seq, k:]
    else:
        row[-k:] = x[seq, :L + k]
    y[seq] = row
    return y


def stale_inputs(N: int = 8, L: int = 2304, H: int = 256, V: int = 4096,
                 noise: float = 1e-3, seed: int = 0):
    """Rows and weights for the skipped-weight-sync fault: W' = bf16(W + N(0,
    noise)). Returns (x_bits [N*L, H], w_bits, w_stale_bits, ids [N*L])."""
    b = BASE_SEED + _OFF_STALE + 16 * seed
    x = _hidden_bits(b + _OFF_X, N * L, H, rms=True)
    w = _weight_bits(b + _OFF_W, V, H, 1.0 / np.sqrt(H))
    dw = normal_f32(b + 5, V * H, noise).reshape(V, H)
    w_stale = bf16_bits_from_f32(f32_from_bf16_bits(w) + dw)
    ids = zipf_ids(b + _OFF_IDS, N * L, V)
    return x, w, w_stale, ids


def stale_qwen_inputs(N: int = 8, L: int = 2304, H: int = 2048, V: int = 151936,
                      noise: float = 1e-3, seed: int = 0):
    """The skipped-weight-sync fault at the Qwen3-1.7B-shaped head: rms-scaled
    bf16 rows for every position of an N x L record, W = the Qwen-shaped
    bf16 N(0, 0.02) weight of qwen_weight(H, V), W' = bf16(W + N(0, noise)),
    Zipf(1.1) target ids. Returns (x_bits [N*L, H], w_bits, w_stale_bits,
    ids [N*L])."""
    b = BASE_SEED + _OFF_STALE + 16 * (seed + 1)
    x = _hidden_bits(b + _OFF_X, N * L, H, rms=True)
    w = qwen_weight(H, V)
    w_stale = bf16_bits_from_f32(f32_from_bf16_bits(w) + normal_f32(b + 5, V * H, noise).reshape(V, H))
    ids = zipf_ids(b + _OFF_IDS, N * L, V)
    return x, w, w_stale, ids


def compare_sweep_case(N: int, L: int = 2304, prompt: int = 256, seed: int = 0) -> CompareCase:
    """Large comparison batch for bandwidth measurement: A = B, C = B + N(0, 1e-3)."""
    c = compare_case(N=N, max_resp=L - prompt, prompt=prompt, seed=seed + 1)
    c.C = noise_scores(c.C, c.mask, 1e-3, seed)
    c.name = f"sweep N={N} L={L}"
    return c
