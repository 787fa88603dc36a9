"""Seeded synthetic workloads shaped like the settings the pages study.

The pages evaluate long contexts (16K to 128K tokens), sparsity up to 0.95 and
GQA models with 28-64 query heads over 4-16 KV heads (page "稀疏注意力的Trade-offs",
sections 1.2, 3.1 and 3.4).  No dataset is used: every tensor here is drawn from its own
PCG64 stream, seeded by numpy's SeedSequence(1000 + config id, spawn_key=(tensor, sequence)), so any sequence can be regenerated alone and in any order.

Values of bf16 workloads are drawn in float32 and rounded to bfloat16
round-to-nearest-even; they are returned as float32 arrays that hold exactly
bf16-representable numbers, so the CPU oracle and the GPU path see identical
inputs.

Structure planted so that block selection is well defined:
  * needles: every key of a needle block gets ``+3 * qhat`` where ``qhat`` is the
    unit vector of the mean of all query vectors that score that KV head (all
    query rows of the sequence times the group's query heads).  Needle blocks are
    drawn without replacement from the blocks strictly before the first query
    row's block (for a full prefill from 0 .. NB-2), the same blocks for every KV
    head of a sequence.
  * block offsets (prefill with gate): one vector o ~ N(0, sigma^2 I) per
    (sequence, KV head, block), added to every key of that block.
  * gist tokens (SSA-style decode): gist_k = chunk mean of K + N(0, 0.1^2),
    gist_v = chunk mean of V + N(0, 0.1^2), one per complete chunk.

This module is input synthesis only; it does not pool, score, select or attend.
"""
from __future__ import annotations

import functools
import math
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Tuple

import numpy as np

# query coordinate 0 of the near-tie plant (exact in bf16)
NEAR_TIE_Q0 = np.float32(2.0 ** -18)

# stream ids (second component of the seed sequence's spawn key)
_S_LENS, _S_Q, _S_K, _S_V, _S_NEEDLE, _S_OFFSET, _S_GK, _S_GV, _S_MK, _S_MV, _S_DO = range(11)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returns float32."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    r = (u + bias) & np.uint32(0xFFFF0000)
    return r.view(np.float32)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Bit pattern (uint16) of float32 values that are already bf16-representable."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    return (u >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _rng(seed: int, stream: int, index: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=(stream, index))))


# ---------------------------------------------------------------------------------------------
# The five workloads.  ``kind``: prefill | decode | gist_decode | mixed (prefill + decode halves).
# Budget: k_u = min(#candidates, k_fixed) when frac_den == 0, else
#         min(#candidates, ceil(frac_num * (c + count_current) / frac_den));
#         optional keys sqrt_num / sqrt_den (sqrt_den > 0) select the square-root rule
#         min(#candidates, ceil(sqrt_num * sqrt(c + count_current) / sqrt_den)).
# ---------------------------------------------------------------------------------------------
CONFIGS: Dict[int, dict] = {
    1: dict(name="tiny_causal_prefill_f32", kind="prefill", dtype="f32",
            batch=1, hq=1, hkv=1, d=64, block=64, seq_len=1024, tq=1024,
            sel="group", k_fixed=4, frac_num=0, frac_den=0, count_current=0,
            sink=False, gate=False, needles=2, offset_sigma=0.0),
    2: dict(name="decode_b8_h32x8_32k", kind="decode", dtype="bf16",
            batch=8, hq=32, hkv=8, d=128, block=64, seq_len=32768,
            sel="group", k_fixed=16, frac_num=0, frac_den=0, count_current=0,
            sink=False, gate=False, needles=4, offset_sigma=0.0),
    3: dict(name="prefill_h28x4_32k_sink_gate", kind="prefill", dtype="bf16",
            batch=1, hq=28, hkv=4, d=128, block=128, seq_len=32768, tq=32768,
            sel="group", k_fixed=0, frac_num=1, frac_den=8, count_current=0,
            sink=True, gate=True, needles=0, offset_sigma=0.5),
    4: dict(name="gist_decode_b4_h64x8_128k", kind="gist_decode", dtype="bf16",
            batch=4, hq=64, hkv=8, d=128, block=64, seq_len=131073,
            sel="group", k_fixed=104, frac_num=0, frac_den=0, count_current=0,
            sink=False, gate=False, needles=0, offset_sigma=0.0, gist_sigma=0.1),
    5: dict(name="mixed_varlen_16seq_h32x8_perhead_gate", kind="mixed", dtype="bf16",
            batch=16, hq=32, hkv=8, d=128, block=64, len_lo=4096, len_hi=131072,
            n_prefill=8, tq=4096,
            sel="head", k_fixed=0, frac_num=1, frac_den=20, count_current=1,
            sink=False, gate=True, needles_frac=0.01, offset_sigma=0.0),
    # The two-level (meta-gist) variant of configuration 4's shape: groups of 32 chunks, the 8
    # best of the 64 groups opened, then 104 of their chunks expanded as in configuration 4.
    6: dict(name="hssa_decode_b4_h64x8_128k_m32", kind="gist_decode", dtype="bf16",
            batch=4, hq=64, hkv=8, d=128, block=64, seq_len=131073,
            sel="group", k_fixed=104, frac_num=0, frac_den=0, count_current=0,
            sink=False, gate=False, needles=0, offset_sigma=0.0, gist_sigma=0.1,
            group_chunks=32, k_groups=8, meta_sigma=0.1),
}

# "mini" variants: same structure, lengths divided by 8 (budgets that are fixed counts are
# divided by 8 too, so that the sparsity stays close to the full configuration's).
_MINI = {
    1: {},
    2: dict(seq_len=4096, k_fixed=2),
    3: dict(seq_len=4096, tq=4096),
    4: dict(seq_len=16385, k_fixed=13),
    5: dict(len_lo=512, len_hi=16384, tq=512),
    6: dict(seq_len=16385, k_fixed=13, group_chunks=8, k_groups=4),
}


@dataclass(eq=False)
class Workload:
    cfg_id: int
    mini: bool = False
    overrides: Optional[dict] = None
    spec: dict = field(init=False)
    seed: int = field(init=False)

    def __post_init__(self):
        spec = dict(CONFIGS[self.cfg_id])
        if self.mini:
            spec.update(_MINI[self.cfg_id])
            spec["name"] = spec["name"] + "_mini"
        if self.overrides:
            spec.update(self.overrides)
            spec["name"] = spec["name"] + "_" + str(self.overrides.get("tag", "custom"))
        self.spec = spec
        self.seed = 1000 + self.cfg_id + int(spec.get("seed_offset", 0))
        s = spec
        self.name: str = s["name"]
        self.kind: str = s["kind"]
        self.dtype: str = s["dtype"]
        self.batch: int = s["batch"]
        self.hq: int = s["hq"]
        self.hkv: int = s["hkv"]
        self.group: int = self.hq // self.hkv
        self.d: int = s["d"]
        self.block: int = s["block"]
        self.sel: str = s["sel"]
        self.k_fixed: int = s["k_fixed"]
        self.frac_num: int = s["frac_num"]
        self.frac_den: int = s["frac_den"]
        self.count_current: int = s["count_current"]
        self.sqrt_num: int = int(s.get("sqrt_num", 0))
        self.sqrt_den: int = int(s.get("sqrt_den", 0))
        self.sink: bool = s["sink"]
        self.gate: bool = s["gate"]
        if self.kind == "mixed":
            r = _rng(self.seed, _S_LENS)
            self.seq_lens: List[int] = [int(x) for x in r.integers(s["len_lo"], s["len_hi"] + 1, size=self.batch)]
            npf = s["n_prefill"]
            self.seq_kind = ["prefill"] * npf + ["decode"] * (self.batch - npf)
            self.tq = s["tq"]
        else:
            self.seq_lens = list(s["seq_lens"]) if "seq_lens" in s else [s["seq_len"]] * self.batch
            self.seq_kind = ["prefill" if self.kind == "prefill" else "decode"] * self.batch
            self.tq = s.get("tq", 1)
        # first query row position per sequence
        self.q_start: List[int] = []
        self.rows: List[int] = []
        for b in range(self.batch):
            L = self.seq_lens[b]
            if self.seq_kind[b] == "prefill":
                self.q_start.append(L - self.tq)
                self.rows.append(self.tq)
            else:
                self.q_start.append(L - 1)
                self.rows.append(1)
        self.max_len = max(self.seq_lens)

    # ------------------------------------------------------------------ helpers
    def is_bf16(self) -> bool:
        return self.dtype == "bf16"

    def _finish(self, x: np.ndarray) -> np.ndarray:
        return round_bf16(x) if self.is_bf16() else np.ascontiguousarray(x, dtype=np.float32)

    def prefill_seqs(self) -> List[int]:
        return [b for b in range(self.batch) if self.seq_kind[b] == "prefill"]

    def decode_seqs(self) -> List[int]:
        return [b for b in range(self.batch) if self.seq_kind[b] == "decode"]

    # ------------------------------------------------------------------ queries
    @functools.lru_cache(maxsize=4)
    def q(self, b: int) -> np.ndarray:
        """Queries of sequence b: [hq, rows_b, d] (rows at positions q_start[b] + t)."""
        r = _rng(self.seed, _S_Q, b)
        x = r.standard_normal((self.hq, self.rows[b], self.d), dtype=np.float32)
        if self.spec.get("near_tie"):
            x[:, :, 0] = NEAR_TIE_Q0
        return self._finish(x)

    def grad_out(self, b: int) -> np.ndarray:
        """Output gradient dO of sequence b for a backward pass: [hq, rows_b, d], N(0, 1) entries
        in the workload dtype (its own stream, so the other inputs do not change)."""
        r = _rng(self.seed, _S_DO, b)
        x = r.standard_normal((self.hq, self.rows[b], self.d), dtype=np.float32)
        return self._finish(x)

    def needle_blocks(self, b: int) -> np.ndarray:
        s = self.spec
        L = self.seq_lens[b]
        nb = -(-L // self.block)
        first = self.q_start[b] // self.block
        pool = first if first > 0 else nb - 1
        if "needles_frac" in s:
            n = max(1, int(round(s["needles_frac"] * nb)))
        else:
            n = s.get("needles", 0)
        n = min(n, pool)
        if n <= 0:
            return np.zeros(0, dtype=np.int64)
        r = _rng(self.seed, _S_NEEDLE, b)
        return np.sort(r.choice(pool, size=n, replace=False)).astype(np.int64)

    def needle_dirs(self, b: int) -> np.ndarray:
        """Unit vector of the mean query of each KV head's query heads: [hkv, d] float64."""
        q = self.q(b).astype(np.float64)
        m = q.reshape(self.hkv, self.group, self.rows[b], self.d).mean(axis=(1, 2))
        n = np.linalg.norm(m, axis=1, keepdims=True)
        return m / np.maximum(n, 1e-30)

    # ------------------------------------------------------------------ keys / values
    @functools.lru_cache(maxsize=2)
    def kv(self, b: int) -> Tuple[np.ndarray, np.ndarray]:
        """(K, V) of sequence b: each [hkv, L_b, d]."""
        L = self.seq_lens[b]
        K = _rng(self.seed, _S_K, b).standard_normal((self.hkv, L, self.d), dtype=np.float32)
        V = _rng(self.seed, _S_V, b).standard_normal((self.hkv, L, self.d), dtype=np.float32)
        blk = self.block
        nb = -(-L // blk)
        sig = self.spec.get("offset_sigma", 0.0)
        if sig > 0.0:
            off = _rng(self.seed, _S_OFFSET, b).standard_normal((self.hkv, nb, self.d), dtype=np.float32) * np.float32(sig)
            full = (L // blk) * blk
            K[:, :full, :] += np.repeat(off[:, : L // blk, :], blk, axis=1)
            if full < L:
                K[:, full:, :] += off[:, nb - 1: nb, :]
        needles = self.needle_blocks(b)
        if needles.size:
            dirs = (3.0 * self.needle_dirs(b)).astype(np.float32)  # [hkv, d]
            for j in needles:
                lo, hi = int(j) * blk, min((int(j) + 1) * blk, L)
                K[:, lo:hi, :] += dirs[:, None, :]
        if self.spec.get("near_tie"):
            return self._near_tie(K, b), self._finish(V)
        return self._finish(K), self._finish(V)

    def near_tie_blocks(self, b: int) -> Tuple[int, int]:
        """The planted pair (A, B), A < B, complete blocks before the first query row's block."""
        pool = self.q_start[b] // self.block
        assert pool >= 2, "a near tie needs two complete blocks before the query"
        a, c = np.sort(_rng(self.seed, _S_NEEDLE, 10_000 + b).choice(pool, size=2, replace=False))
        return int(a), int(c)

    def _near_tie(self, K: np.ndarray, b: int) -> np.ndarray:
        """Plant two needle blocks A < B whose selector scores differ by far less than 1e-5 relative
        but are not equal: B is a copy of A (both get the needle offset 3 qhat) whose first key has
        its coordinate 0 raised by one bf16 step, and every query has coordinate 0 = 2^-18.  B's
        exact score then exceeds A's by about 1e-13 relative, below what fp32 sums resolve."""
        assert self.is_bf16(), "the near tie is planted in bf16 inputs"
        blk = self.block
        A, B = self.near_tie_blocks(b)
        dirs = (3.0 * self.needle_dirs(b)).astype(np.float32)
        K[:, A * blk:(A + 1) * blk, :] += dirs[:, None, :]
        K = self._finish(K)
        K[:, B * blk:(B + 1) * blk, :] = K[:, A * blk:(A + 1) * blk, :]
        v = np.ascontiguousarray(K[:, B * blk, 0], dtype=np.float32)
        bits = v.view(np.uint32).copy()
        up = np.where(v >= 0, bits + np.uint32(0x10000), bits - np.uint32(0x10000))   # next bf16 towards +inf
        K[:, B * blk, 0] = up.view(np.float32)
        return K

    def gist(self, b: int) -> Tuple[np.ndarray, np.ndarray]:
        """(gist_k, gist_v) of sequence b: each [hkv, NC, d], NC = number of complete chunks."""
        K, V = self.kv(b)
        L = self.seq_lens[b]
        nc = L // self.block
        sig = self.spec.get("gist_sigma", 0.1)
        out = []
        for X, stream in ((K, _S_GK), (V, _S_GV)):
            cm = X[:, : nc * self.block, :].astype(np.float64).reshape(self.hkv, nc, self.block, self.d).mean(axis=2)
            noise = _rng(self.seed, stream, b).standard_normal((self.hkv, nc, self.d), dtype=np.float32)
            out.append(self._finish((cm + sig * noise.astype(np.float64)).astype(np.float32)))
        return out[0], out[1]

    def meta(self, b: int) -> Tuple[np.ndarray, np.ndarray]:
        """(meta_k, meta_v) of sequence b: each [hkv, NM, d] for the NM complete groups of
        group_chunks consecutive chunks: the mean of the group's gists plus N(0, meta_sigma^2)
        noise, as the gists are the chunk means plus noise."""
        M = self.spec["group_chunks"]
        gk, gv = self.gist(b)
        nm = gk.shape[1] // M
        sig = self.spec.get("meta_sigma", 0.1)
        out = []
        for X, stream in ((gk, _S_MK), (gv, _S_MV)):
            gm = X[:, : nm * M, :].astype(np.float64).reshape(self.hkv, nm, M, self.d).mean(axis=2)
            noise = _rng(self.seed, stream, b).standard_normal((self.hkv, nm, self.d), dtype=np.float32)
            out.append(self._finish((gm + sig * noise.astype(np.float64)).astype(np.float32)))
        return out[0], out[1]

    # ------------------------------------------------------------------ budget description
    def budget(self) -> dict:
        return dict(k_fixed=self.k_fixed, frac_num=self.frac_num, frac_den=self.frac_den,
                    count_current=self.count_current, sqrt_num=self.sqrt_num, sqrt_den=self.sqrt_den,
                    sink=self.sink, gate=self.gate)

    def describe(self) -> dict:
        return dict(name=self.name, kind=self.kind, dtype=self.dtype, batch=self.batch, hq=self.hq,
                    hkv=self.hkv, d=self.d, block=self.block, seq_lens=self.seq_lens, q_start=self.q_start,
                    rows=self.rows, sel=self.sel, **self.budget())
