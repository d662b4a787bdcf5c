"""Seeded synthetic workloads: SID catalogs, per-step logits, hidden states and weights.

This module only *draws inputs*. It holds none of the method's arithmetic (no
masking, no log-softmax, no selection), so both the HIP path and the CPU oracle
can take their inputs from it.

The shapes follow the pages:
  * SIDs are short fixed-depth code tuples with 256 codes per level; OPQ gives
    L=4 x 256 (SPRINT summary, method paragraph), FlashRec decodes 3-5 steps
    (flashrec 0.1.0, intro).
  * beam widths 50-512+ (flashrec 0.1.0, intro) and catalogs from tens of
    thousands (SPRINT summary, "catalogs of roughly 12k-90k items") to millions.

No dataset the pages measure on (RecIF-Bench, Sohu traffic, Amazon/Yelp) is
available; these generators stand in for them.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

V_DEFAULT = 256
CHUNK = 1 << 20


# --------------------------------------------------------------------------- catalogs
def zipf_probs(V: int = V_DEFAULT, s: float = 1.1) -> np.ndarray:
    """Bounded Zipf over ranks 1..V: p_k proportional to k**-s; code = rank - 1."""
    w = np.arange(1, V + 1, dtype=np.float64) ** (-s)
    return w / w.sum()


def pack_sids(sids: np.ndarray) -> np.ndarray:
    """Pack [n, L] uint8 code tuples big-endian into uint64 (first code most significant)."""
    sids = np.asarray(sids, dtype=np.uint8)
    key = np.zeros(sids.shape[0], dtype=np.uint64)
    for j in range(sids.shape[1]):
        key = (key << np.uint64(8)) | sids[:, j].astype(np.uint64)
    return key


def catalog(n_distinct: int, L: int, level_dists, seed, V: int = V_DEFAULT) -> np.ndarray:
    """Draw ``n_distinct`` distinct SIDs, returned in first-occurrence order.

    ``level_dists`` is a sequence of L entries, each "uniform" or "zipf".
    Draws happen in chunks of 2**20 rows; each level uses ``integers(0, V)`` or
    ``choice(V, p=zipf)``; repeated tuples are rejected, keeping the first N
    distinct ones in draw order. Item id = row index of the result.
    """
    assert len(level_dists) == L
    if n_distinct > V ** L:
        raise ValueError(f"catalog: {n_distinct} distinct SIDs requested, only {V ** L} exist at L={L}, V={V}")
    rng = np.random.default_rng(seed)
    pz = zipf_probs(V)
    seen = np.zeros(0, dtype=np.uint64)          # sorted keys already kept
    kept = []                                     # chunks of kept rows in draw order
    n_kept = 0
    while n_kept < n_distinct:
        cols = []
        for d in level_dists:
            if d == "uniform":
                cols.append(rng.integers(0, V, size=CHUNK, dtype=np.int64))
            elif d == "zipf":
                cols.append(rng.choice(V, size=CHUNK, p=pz))
            else:
                raise ValueError(d)
        chunk = np.stack(cols, axis=1).astype(np.uint8)
        keys = pack_sids(chunk)
        _, first = np.unique(keys, return_index=True)
        first.sort()                               # first occurrences, in draw order
        keys_f = keys[first]
        if seen.size:
            pos = np.searchsorted(seen, keys_f)
            pos = np.minimum(pos, seen.size - 1)
            fresh = seen[pos] != keys_f
        else:
            fresh = np.ones(keys_f.size, dtype=bool)
        take = first[fresh][: n_distinct - n_kept]
        kept.append(chunk[take])
        n_kept += take.size
        seen = np.union1d(seen, keys[take])
    return np.concatenate(kept, axis=0)


# --------------------------------------------------------------------------- dtype helpers
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round-to-nearest-even); returns the uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# --------------------------------------------------------------------------- row-keyed logits
def logits_rowkeyed(workload_seed: int, step: int, req: int, rows: int, sigma: float,
                    V: int = V_DEFAULT, bf16: bool = False) -> np.ndarray:
    """Logits for request ``req`` at its step ``step``: N(0, sigma^2), shape [rows, V].

    Drawn by ``default_rng([workload_seed, 2, step, req])`` in float64 and rounded
    to float32 (then to bfloat16 bits when ``bf16``). Live row r of the request
    uses row r, independent of how many rows end up live.
    """
    rng = np.random.default_rng([workload_seed, 2, step, req])
    x = rng.normal(0.0, sigma, size=(rows, V)).astype(np.float32)
    return f32_to_bf16_bits(x) if bf16 else x


# --------------------------------------------------------------------------- prefix-keyed logits
_M64 = (1 << 64) - 1
_GOLD = np.uint64(0x9E3779B97F4A7C15)
_MIX1 = np.uint64(0xBF58476D1CE4E5B9)
_MIX2 = np.uint64(0x94D049BB133111EB)


def splitmix64(x):
    """SplitMix64 output function (Steele, Lea & Flood, OOPSLA 2014), vectorised on uint64."""
    with np.errstate(over="ignore"):
        z = np.asarray(x, dtype=np.uint64) + _GOLD
        z = (z ^ (z >> np.uint64(30))) * _MIX1
        z = (z ^ (z >> np.uint64(27))) * _MIX2
        return z ^ (z >> np.uint64(31))


def logits_prefixkeyed(seed: int, depth: int, prefixes_packed, sigma: float,
                       V: int = V_DEFAULT, bf16: bool = False) -> np.ndarray:
    """Logits that depend only on (seed, depth, prefix, code), shape [len(prefixes), V].

    For a prefix p (its codes packed big-endian) at depth d and code c:
      h = sm64(sm64(seed) ^ (d << 56) ^ p);  a = sm64(h + 2c);  b = sm64(h + 2c + 1)
      u1 = ((a >> 11) + 0.5) * 2**-53;  u2 = (b >> 11) * 2**-53
      x = sigma * sqrt(-2 ln u1) * cos(2 pi u2)     (Box-Muller, float64, then rounded)
    Any implementation that knows a row's prefix regenerates the same row.
    """
    p = np.asarray(prefixes_packed, dtype=np.uint64).reshape(-1, 1)
    with np.errstate(over="ignore"):
        h0 = splitmix64(np.uint64(seed & _M64)) ^ (np.uint64(depth) << np.uint64(56))
        h = splitmix64(h0 ^ p)
        c = np.arange(V, dtype=np.uint64).reshape(1, -1)
        a = splitmix64(h + np.uint64(2) * c)
        b = splitmix64(h + np.uint64(2) * c + np.uint64(1))
    u1 = ((a >> np.uint64(11)).astype(np.float64) + 0.5) * 2.0 ** -53
    u2 = (b >> np.uint64(11)).astype(np.float64) * 2.0 ** -53
    x = (sigma * np.sqrt(-2.0 * np.log(u1)) * np.cos(2.0 * math.pi * u2)).astype(np.float32)
    return f32_to_bf16_bits(x) if bf16 else x


# --------------------------------------------------------------------------- lm_head inputs
def hidden_states(workload_seed: int, step: int, rows: int, H: int) -> np.ndarray:
    """bf16 bits of hidden states N(0, 1), shape [rows, H], from ``default_rng([seed, 4, step])``."""
    rng = np.random.default_rng([workload_seed, 4, step])
    return f32_to_bf16_bits(rng.standard_normal((rows, H), dtype=np.float32))


def lmhead_weight(workload_seed: int, level: int, V: int, H: int, std: float = 0.02) -> np.ndarray:
    """bf16 bits of the SID-range lm_head of one level, shape [V, H], N(0, std^2)."""
    rng = np.random.default_rng([workload_seed, 5, level])
    return f32_to_bf16_bits((rng.standard_normal((V, H), dtype=np.float32) * np.float32(std)))


# --------------------------------------------------------------------------- scoring inputs
# Single-pass scoring (SPRINT summary, method paragraph): per user an L x V table of
# per-position token distributions and a user vector; per valid SID an embedding row.
def score_logits(seed, users: int, L: int, sigma: float = 2.0, V: int = V_DEFAULT) -> np.ndarray:
    """float32 [users, L, V] raw per-position logits N(0, sigma^2), ``default_rng([seed, 6])``."""
    rng = np.random.default_rng([seed, 6])
    return (rng.standard_normal((users, L, V), dtype=np.float32) * np.float32(sigma))


def score_logprobs(seed, users: int, L: int, alpha: float = 0.3, V: int = V_DEFAULT) -> np.ndarray:
    """float32 [users, L, V] log-probabilities of random per-position distributions:
    Dirichlet(alpha) draws (peaked for alpha < 1), floored at 1e-30 before the log."""
    rng = np.random.default_rng([seed, 7])
    p = rng.dirichlet(np.full(V, alpha), size=(users, L))
    return np.log(np.maximum(p, 1e-30)).astype(np.float32)


def user_vectors(seed, users: int, D: int) -> np.ndarray:
    """bf16 bits [users, D] of user vectors N(0, 1), ``default_rng([seed, 8])``."""
    rng = np.random.default_rng([seed, 8])
    return f32_to_bf16_bits(rng.standard_normal((users, D), dtype=np.float32))


def sid_embeddings(seed, n: int, D: int) -> np.ndarray:
    """bf16 bits [n, D] of SID-level embeddings N(0, 1/D) in leaf order, drawn in chunks
    of 2^20 rows from ``default_rng([seed, 9, chunk])``."""
    out = np.empty((n, D), dtype=np.uint16)
    scale = np.float32(1.0 / math.sqrt(D))
    for c0 in range(0, n, CHUNK):
        rows = min(CHUNK, n - c0)
        rng = np.random.default_rng([seed, 9, c0 // CHUNK])
        out[c0:c0 + rows] = f32_to_bf16_bits(rng.standard_normal((rows, D), dtype=np.float32) * scale)
    return out


# --------------------------------------------------------------------------- workloads
@dataclasses.dataclass(frozen=True)
class Workload:
    """One benchmark / parity workload, named by what it is."""
    name: str
    seed: int                  # first element of every seed list of this workload
    L: int
    n_catalog: int
    level_dists: tuple
    widths: tuple              # beam width per request
    sigma: float = 2.0
    bf16: bool = False
    slot_budget: int = 0       # >0: requests are admitted in FIFO waves under this many rows
    hidden: int = 0            # >0: fused lm_head with this hidden size (bf16 hidden + weights)

    @property
    def n_requests(self) -> int:
        return len(self.widths)

    def catalog(self) -> np.ndarray:
        return catalog(self.n_catalog, self.L, self.level_dists, [self.seed, 1])


def _mixed_widths() -> tuple:
    rng = np.random.default_rng([4, 3])
    return tuple(int(b) for b in rng.choice([50, 128, 256, 512], 256))


WORKLOADS = {
    # 1 request, L=3, 20k uniform SIDs, beam 50, fp32 logits N(0, 2^2)
    "b50x1_l3_20k_f32": Workload("b50x1_l3_20k_f32", 1, 3, 20_000, ("uniform",) * 3, (50,)),
    # 64 requests x beam 128, L=4, 1M Zipf(1.1) SIDs, fp32 N(0, 2^2)
    "b128x64_l4_1m_zipf_f32": Workload("b128x64_l4_1m_zipf_f32", 2, 4, 1_000_000,
                                       ("zipf",) * 4, (128,) * 64),
    # 32 requests x beam 512, L=4, 4M Zipf(1.1) SIDs, bf16 N(0, 3^2)
    "b512x32_l4_4m_zipf_bf16": Workload("b512x32_l4_4m_zipf_bf16", 3, 4, 4_000_000,
                                        ("zipf",) * 4, (512,) * 32, sigma=3.0, bf16=True),
    # mixed decode wave: 256 requests, widths from {50,128,256,512}, 32,768-row budget, L=5, 8M SIDs
    "mixed256_l5_8m_f32": Workload("mixed256_l5_8m_f32", 4, 5, 8_000_000,
                                   ("uniform",) + ("zipf",) * 4, _mixed_widths(),
                                   slot_budget=32_768),
    # fused SID-range lm_head: 8 requests x beam 512, hidden 2048, L=4, 1M uniform SIDs
    "lmhead_b512x8_l4_1m_h2048": Workload("lmhead_b512x8_l4_1m_h2048", 5, 4, 1_000_000,
                                          ("uniform",) * 4, (512,) * 8, hidden=2048),
}


@dataclasses.dataclass(frozen=True)
class ScoreWorkload:
    """A single-pass scoring workload: every valid SID of a catalog scored for a batch of
    users from raw per-position logits plus a SID-level term, best k kept."""
    name: str
    seed: int
    catalog_of: str            # the beam workload whose catalog is scored
    users: int
    dim: int
    k: int
    sigma: float = 2.0

    def catalog(self) -> np.ndarray:
        return WORKLOADS[self.catalog_of].catalog()


SCORE_WORKLOADS = {
    # the 4M-SID Zipf catalog of the beam line, 32 users, 64-dim SID embeddings, top 512
    "score_u32_k512_l4_4m_zipf_d64": ScoreWorkload("score_u32_k512_l4_4m_zipf_d64", 6,
                                                   "b512x32_l4_4m_zipf_bf16", 32, 64, 512),
}
