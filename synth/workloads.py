"""The five synthetic decode-attention workloads and their seeded generators.

Every input is a pure function of (config seed, what is drawn, physical page id), so
that a single page can be regenerated on its own and pages can be drawn in parallel
threads without changing any value.

Draw recipe (numpy PCG64, one SeedSequence per item):
  * per-channel scales        SeedSequence([seed, 40 + tensor])      tensor: 0 = K, 1 = V
  * outlier channels          SeedSequence([seed, 50])       (the workloads with outlier K channels)
  * page contents             SeedSequence([seed, 100 + tensor, page_id])
  * queries                   SeedSequence([seed, 10])
  * page-table permutation    SeedSequence([seed, 20])
  * sequence lengths          SeedSequence([seed, 30])       (the workload of uneven lengths)
FP32 samples are rounded to BF16 with round-to-nearest-even.

The workload shapes follow the serving setting of the ZipFusion summary (16-token pages,
head_dim 128, contexts of several thousand tokens: "A. Experimental Setup" and
"B. Attention Kernel Performance"); the value distributions are this repository's own.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

K_TENSOR, V_TENSOR = 0, 1

# name, batch, query heads, kv heads, head_dim, page size, context, distributions, appended
CONFIGS = {
    1: dict(name="tiny", B=1, Hq=2, Hkv=2, D=64, P=256, L=256, append=0,
            k_dist="chan_lognormal", v_dist="chan_lognormal"),
    2: dict(name="llama7b_b1_ctx4k", B=1, Hq=32, Hkv=32, D=128, P=16, L=4096, append=0,
            k_dist="outlier_normal", v_dist="normal"),
    3: dict(name="mha_ctx8k_b32", B=32, Hq=32, Hkv=32, D=128, P=16, L=8193, append=1,
            k_dist="chan_lognormal", v_dist="chan_lognormal"),
    4: dict(name="gqa28x4_b64", B=64, Hq=28, Hkv=4, D=128, P=16, L=None, append=0,
            k_dist="student_t3", v_dist="normal_half"),
    5: dict(name="escape_stress_ctx32k_b4", B=4, Hq=32, Hkv=32, D=128, P=16, L=32768, append=0,
            k_dist="log_uniform", v_dist="log_uniform"),
    # the attention-benchmark shape of the ZipFusion summary (§IV.B: 32 query / 8 KV heads,
    # head_dim 128, 16-token pages, 8192-token context, batch 64), K with outlier channels
    6: dict(name="gqa32x8_b64_ctx8k", B=64, Hq=32, Hkv=8, D=128, P=16, L=8192, append=0,
            k_dist="outlier_normal", v_dist="normal"),
}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round finite float32 values to BF16 (nearest, ties to even); returns uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen BF16 bit patterns to float32 exactly."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _rng(*key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(key))))


@dataclass
class Workload:
    cfg: int
    name: str
    B: int
    Hq: int
    Hkv: int
    D: int
    P: int
    seq_lens: np.ndarray          # int32 [B]  tokens in the cache when attention runs
    n_append: int                 # tokens of each request that arrive through the append step
    page_table: np.ndarray        # int32 [B, max_pages]; -1 past ceil(L/P)
    num_pages: int
    k_dist: str
    v_dist: str
    seed: int
    _scales: dict = field(default_factory=dict, repr=False)
    _outliers: np.ndarray | None = field(default=None, repr=False)

    @property
    def max_pages(self) -> int:
        return int(self.page_table.shape[1])

    @property
    def sm_scale(self) -> float:
        return 1.0 / math.sqrt(self.D)

    @property
    def group(self) -> int:
        return self.Hq // self.Hkv

    # ---- per-channel parameters, drawn once per config -------------------------------
    def _channel_scale(self, tensor: int) -> np.ndarray:
        if tensor not in self._scales:
            g = _rng(self.seed, 40 + tensor)
            lo, hi = math.log(0.1), math.log(10.0)
            self._scales[tensor] = np.exp(g.uniform(lo, hi, size=(self.Hkv, self.D))).astype(np.float32)
        return self._scales[tensor]

    def _outlier_mult(self) -> np.ndarray:
        if self._outliers is None:
            g = _rng(self.seed, 50)
            m = np.ones((self.Hkv, self.D), np.float32)
            for h in range(self.Hkv):
                m[h, g.choice(self.D, size=4, replace=False)] = 20.0
            self._outliers = m
        return self._outliers

    # ---- page contents ------------------------------------------------------------
    def page(self, page_id: int, tensor: int) -> np.ndarray:
        """BF16 bits of one physical page, uint16 [Hkv, P, D] (token-major rows)."""
        dist = self.k_dist if tensor == K_TENSOR else self.v_dist
        g = _rng(self.seed, 100 + tensor, int(page_id))
        shape = (self.Hkv, self.P, self.D)
        if dist == "chan_lognormal":
            x = g.standard_normal(shape, dtype=np.float32) * self._channel_scale(tensor)[:, None, :]
        elif dist == "outlier_normal":
            x = g.standard_normal(shape, dtype=np.float32) * self._outlier_mult()[:, None, :]
        elif dist == "normal":
            x = g.standard_normal(shape, dtype=np.float32)
        elif dist == "normal_half":
            x = g.standard_normal(shape, dtype=np.float32) * np.float32(0.5)
        elif dist == "student_t3":
            x = np.clip(g.standard_t(3, size=shape), -64.0, 64.0).astype(np.float32)
        elif dist == "log_uniform":
            return self._log_uniform_page(g, shape)
        else:
            raise ValueError(dist)
        return f32_to_bf16_bits(x)

    @staticmethod
    def _log_uniform_page(g: np.random.Generator, shape) -> np.ndarray:
        mag = np.exp2(g.uniform(-20.0, 20.0, size=shape).astype(np.float32))
        sign = g.integers(0, 2, size=shape, dtype=np.uint16) << np.uint16(15)
        bits = f32_to_bf16_bits(mag) | sign
        u = g.random(size=shape)
        zero = u < 0.01
        sub = (u >= 0.01) & (u < 0.011)
        bits[zero] = sign[zero]
        sub_mant = g.integers(1, 128, size=shape, dtype=np.uint16)
        bits[sub] = sign[sub] | sub_mant[sub]
        return bits

    def pages(self, tensor: int, page_ids=None, threads: int | None = None) -> np.ndarray:
        """Pages stacked as uint16 [n, Hkv, P, D]; all physical pages when page_ids is None."""
        ids = np.arange(self.num_pages) if page_ids is None else np.asarray(page_ids)
        out = np.empty((len(ids), self.Hkv, self.P, self.D), np.uint16)
        self._channel_scale(tensor)
        self._outlier_mult()

        def work(i):
            out[i] = self.page(int(ids[i]), tensor)

        nthreads = threads or min(16, os.cpu_count() or 1)
        if len(ids) < 64 or nthreads == 1:
            for i in range(len(ids)):
                work(i)
        else:
            with ThreadPoolExecutor(nthreads) as ex:
                list(ex.map(work, range(len(ids)), chunksize=64))
        return out

    def q(self) -> np.ndarray:
        """Query BF16 bits, uint16 [B, Hq, D], N(0, 1)."""
        g = _rng(self.seed, 10)
        return f32_to_bf16_bits(g.standard_normal((self.B, self.Hq, self.D), dtype=np.float32))

    def token(self, r: int, t: int, tensor: int) -> np.ndarray:
        """BF16 bits of token t of request r for every KV head, uint16 [Hkv, D]."""
        pid = int(self.page_table[r, t // self.P])
        return self.page(pid, tensor)[:, t % self.P, :]

    def appended(self, tensor: int) -> np.ndarray:
        """The token each request receives through the append step, uint16 [B, Hkv, D]."""
        assert self.n_append == 1
        return np.stack([self.token(r, int(self.seq_lens[r]) - 1, tensor) for r in range(self.B)])


def make_workload(cfg: int, *, B: int | None = None, L: int | None = None, seed: int | None = None,
                  Hq: int | None = None, Hkv: int | None = None, D: int | None = None,
                  P: int | None = None, lens=None, k_dist: str | None = None,
                  v_dist: str | None = None, n_append: int | None = None) -> Workload:
    """Build config `cfg` at its full shape, or a reduced variant when sizes are given.

    `lens` overrides the per-request lengths (an int array of length B).
    """
    c = dict(CONFIGS[cfg])
    B = c["B"] if B is None else B
    Hq = c["Hq"] if Hq is None else Hq
    Hkv = c["Hkv"] if Hkv is None else Hkv
    D = c["D"] if D is None else D
    P = c["P"] if P is None else P
    seed = cfg if seed is None else seed
    n_app = c["append"] if n_append is None else n_append
    if lens is not None:
        seq = np.asarray(lens, dtype=np.int32)
        assert seq.shape == (B,)
    elif L is not None:
        seq = np.full(B, L, np.int32)
    elif c["L"] is not None:
        seq = np.full(B, c["L"], np.int32)
    else:  # the uneven-length workload: lengths uniform in [1024, 8192]
        seq = _rng(seed, 30).integers(1024, 8193, size=B).astype(np.int32)
    npr = (seq + P - 1) // P
    num_pages = int(npr.sum())
    max_pages = max(1, int(npr.max()))
    perm = _rng(seed, 20).permutation(num_pages).astype(np.int32)
    table = np.full((B, max_pages), -1, np.int32)
    pos = 0
    for r in range(B):
        table[r, :npr[r]] = perm[pos:pos + npr[r]]
        pos += int(npr[r])
    return Workload(cfg=cfg, name=c["name"], B=B, Hq=Hq, Hkv=Hkv, D=D, P=P, seq_lens=seq,
                    n_append=n_app, page_table=table, num_pages=num_pages,
                    k_dist=k_dist or c["k_dist"], v_dist=v_dist or c["v_dist"], seed=seed)
