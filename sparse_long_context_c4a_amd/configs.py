"""Workload shapes of the compressed sparse attention layer.

Each workload is one layer step on synthetic data: a decode step (one new
token per sequence at position m = L-1) or a prefill chunk.  The shapes
follow the pages' description of DeepSeek V4 attention: c4a entries are
weighted sums of 8 raw tokens at stride 4, c128a of 128 at stride 128, k=512
for c4a and k=8192 for c128a, a 128-token raw window, a 512-dim latent
shared by 64 query heads, and a 16-head fp8 indexer of dim 128.
"""

from dataclasses import dataclass, replace


@dataclass(frozen=True)
class Workload:
    name: str
    mode: str            # "decode" or "prefill"
    B: int               # sequences
    L: int               # decode: context length, query at m = L-1
    D: int               # latent dim (K = V)
    r: int               # rotary dims (last r of D)
    H: int               # query heads
    Hi: int              # indexer heads (0: no indexer, selection = all visible)
    Di: int              # indexer dim
    k: int               # Top-k
    s: int               # compressor stride
    S: int               # compressor span
    W: int = 128         # window
    r_idx: int = 0       # rotary dims of the indexer keys
    base: float = 10000.0
    main_dtype: str = "bf16"   # main cache, window, q, out, raw tokens
    idx_dtype: str = "fp8"     # indexer cache and indexer query ("fp4": MXFP4
                               # cache, fp8 query)
    p0: int = 0          # prefill: first position of the chunk
    T: int = 1           # prefill: chunk length
    seed: int = 0
    w_cap: int = 0       # window ring slots (0: 2 W, so a decode step can
                         # insert token m before attention reads [m-W, m-1])
    main_cache_dtype: str = ""  # "fp8": token-wise fp8 main cache (decode); "": main_dtype
    cluster: int = 0     # > 0: that many consecutive cached entries of each sequence
                         # (seeded start) get 16x larger indexer key scales

    @property
    def E_cap(self):
        """Cache slots: one per stride of the context (ceil(L / s))."""
        end = self.L if self.mode == "decode" else self.p0 + self.T
        return -(-end // self.s)

    @property
    def W_cap(self):
        return self.w_cap if self.w_cap else 2 * self.W

    @property
    def m(self):
        return self.L - 1


TINY_C4A_F32 = Workload(
    name="tiny_c4a_decode_f32_L1024", mode="decode", B=1, L=1024, D=128, r=32,
    H=16, Hi=4, Di=64, k=64, s=4, S=8, main_dtype="f32", idx_dtype="f32",
    seed=20260)

C4A_DECODE_64K = Workload(
    name="c4a_decode_B32_L64K", mode="decode", B=32, L=65536, D=512, r=64,
    H=64, Hi=16, Di=128, k=512, s=4, S=8, seed=20261)

C4A_DECODE_1M = Workload(
    name="c4a_decode_B4_L1M", mode="decode", B=4, L=1048576, D=512, r=64,
    H=64, Hi=16, Di=128, k=512, s=4, S=8, seed=20262)

# The same step with the high scores clustered: the scores of 1024 consecutive
# entries per sequence (four 256-entry waves of the indexer) are 16x larger,
# so the positive ones among them (about a fifth) outrank the rest of the row
# and a few waves hold far more of the Top-k than a uniform spread would.
C4A_DECODE_1M_CLUSTERED = Workload(
    name="c4a_decode_B4_L1M_clustered", mode="decode", B=4, L=1048576, D=512, r=64,
    H=64, Hi=16, Di=128, k=512, s=4, S=8, seed=20265, cluster=1024)

C128A_DECODE_1M = Workload(
    name="c128a_decode_B16_L1M", mode="decode", B=16, L=1048576, D=512, r=64,
    H=64, Hi=0, Di=0, k=8192, s=128, S=128, seed=20263)

C4A_PREFILL_128K = Workload(
    name="c4a_prefill_T4096_at126976", mode="prefill", B=1, L=131072, D=512,
    r=64, H=64, Hi=16, Di=128, k=512, s=4, S=8, p0=126976, T=4096,
    seed=20264)

# The same step with the indexer cache stored in MXFP4 (64 bytes of E2M1 codes
# and 4 E8M0 block scales per entry instead of 128 fp8 bytes and an f32 scale):
# the pages keep the indexer in fp4 so that scanning the whole history is cheap.
C4A_DECODE_1M_FP4 = Workload(
    name="c4a_decode_B4_L1M_fp4idx", mode="decode", B=4, L=1048576, D=512, r=64,
    H=64, Hi=16, Di=128, k=512, s=4, S=8, seed=20266, idx_dtype="fp4")

ALL = [TINY_C4A_F32, C4A_DECODE_64K, C4A_DECODE_1M, C128A_DECODE_1M,
       C4A_PREFILL_128K, C4A_DECODE_1M_CLUSTERED, C4A_DECODE_1M_FP4]
BY_NAME = {w.name: w for w in ALL}


def shrink(w: Workload, **kw) -> Workload:
    """A smaller copy of a workload (same geometry, fewer tokens / rows)."""
    return replace(w, **kw)
