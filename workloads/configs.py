"""The five synthetic workloads of gist-token sparse attention, by name.

Each workload is a plain record of shapes and layout parameters.  Nothing here
computes any part of the method; the oracle and the HIP path both read these
records.

Layout parameters follow the pages' statement of the problem:
  * n_sink            -- leading sink tokens (UniGist summary, Approach and the
                         sink ablation; four sinks in the Study page, App. A)
  * chunk_len, gists  -- raw tokens per chunk and gist tokens after it; the
                         compression ratio is chunk_len / gists (Study page, §2)
  * window            -- local causal window in interleaved positions, self
                         included (UniGist summary, Approach, window ablation)
  * top_k             -- chunks unfolded per query, 0 = fixed layout
                         (Simplified Sparse Attention via Gist Tokens, abstract)
  * l2_chunks, l2_gists, l2_top_k -- the gist-of-gist level (Forget, Then
                         Recall ... Gist Sparse Attention, abstract); zero for a
                         single level.
"""
from __future__ import annotations

from dataclasses import dataclass, field, asdict


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str            # "prefill" or "decode"
    dtype: str           # "f32" or "bf16"
    batch: int
    hq: int
    hkv: int
    d: int
    n_sink: int
    chunk_len: int
    gists: int
    window: int
    top_k: int
    n_chunks: int = 0    # complete level-1 chunks (single level)
    l2_chunks: int = 0   # level-1 chunks per level-2 group
    l2_gists: int = 0
    l2_top_k: int = 0
    n_groups: int = 0    # complete level-2 groups (two levels)
    plant_chunks: int = 0   # decode: chunks per sequence given planted gist keys
    plant_groups: int = 0   # two levels: groups per sequence given planted keys
    note: str = ""

    # ---- derived sizes (plain bookkeeping of the layout, no method arithmetic)
    @property
    def period(self) -> int:
        return self.chunk_len + self.gists

    @property
    def group_period(self) -> int:
        return self.l2_chunks * self.period + self.l2_gists

    @property
    def hierarchical(self) -> bool:
        return self.l2_chunks > 0

    @property
    def seq_len(self) -> int:
        """Positions in the interleaved sequence; decode adds the query's own token."""
        if self.hierarchical:
            body = self.n_sink + self.n_groups * self.group_period
        else:
            body = self.n_sink + self.n_chunks * self.period
        return body + (1 if self.kind == "decode" else 0)

    @property
    def layout(self) -> dict:
        return dict(n_sink=self.n_sink, chunk_len=self.chunk_len, gists=self.gists,
                    window=self.window, top_k=self.top_k, l2_chunks=self.l2_chunks,
                    l2_gists=self.l2_gists, l2_top_k=self.l2_top_k)

    def as_dict(self) -> dict:
        d = asdict(self)
        d["seq_len"] = self.seq_len
        return d


TINY_PREFILL_F32 = Workload(
    name="tiny_prefill_f32", kind="prefill", dtype="f32", batch=1, hq=1, hkv=1, d=64,
    n_sink=4, chunk_len=16, gists=1, window=32, top_k=4, n_chunks=32,
    note="548 positions, per-query top-4 unfolding, fp32")

LLAMA3B_K0_PREFILL = Workload(
    name="llama3b_gqa24x8_ratio4_k0_prefill_32k", kind="prefill", dtype="bf16",
    batch=1, hq=24, hkv=8, d=128, n_sink=128, chunk_len=4, gists=1, window=128,
    top_k=0, n_chunks=8192,
    note="3B attention shape, 32768 raw tokens + 8192 gists + 128 sinks, fixed layout")

LLAMA8B_K0_PREFILL = Workload(
    name="llama8b_gqa32x8_ratio8_k0_prefill_32k", kind="prefill", dtype="bf16",
    batch=2, hq=32, hkv=8, d=128, n_sink=128, chunk_len=8, gists=1, window=128,
    top_k=0, n_chunks=4096,
    note="8B attention shape, 32768 raw tokens + 4096 gists + 128 sinks, fixed layout")

SELECTIVE_DECODE = Workload(
    name="selective_decode_b16_32x_k16", kind="decode", dtype="bf16",
    batch=16, hq=32, hkv=8, d=128, n_sink=128, chunk_len=32, gists=1, window=128,
    top_k=16, n_chunks=1024, plant_chunks=16,
    note="one query token per sequence; 16 planted chunks per sequence")

HIER_DECODE = Workload(
    name="hier_decode_b8_g8x8_k8_k16", kind="decode", dtype="bf16",
    batch=8, hq=32, hkv=8, d=128, n_sink=128, chunk_len=8, gists=1, window=128,
    top_k=16, l2_chunks=8, l2_gists=1, l2_top_k=8, n_groups=1024,
    plant_chunks=16, plant_groups=8,
    note="gist-of-gist decode: top-8 groups, then top-16 chunks inside them")

# Next-step workloads (built after the five above; see the design notes).
# Fixed-layout decode over a compacted cache (raw tokens outside the window
# removed): the UniGist setting of the 8B attention shape at ratio 4, 128 sinks,
# window 128, 32768 raw tokens before the query.
COMPACT_DECODE = Workload(
    name="unigist_compact_decode_b16_8b_ratio4_32k", kind="decode", dtype="bf16",
    batch=16, hq=32, hkv=8, d=128, n_sink=128, chunk_len=4, gists=1, window=128,
    top_k=0, n_chunks=8192,
    note="one query per sequence over a cache of sinks + gists + a 128-slot ring of raws")

# Selective unfolding at prefill scale: the 3B shape's 32K layout with every
# query unfolding its 16 best chunks.
LLAMA3B_K16_PREFILL = Workload(
    name="llama3b_gqa24x8_ratio4_k16_prefill_32k", kind="prefill", dtype="bf16",
    batch=1, hq=24, hkv=8, d=128, n_sink=128, chunk_len=4, gists=1, window=128,
    top_k=16, n_chunks=8192,
    note="3B attention shape, 32K raw tokens, per-query top-16 unfolding")

@dataclass(frozen=True)
class BlockMaskWorkload:
    """Prefill over byte positions under a gzip-guided block mask (Gzip-guided
    sparse attention page, Core equations): ``block`` bytes per mask block,
    local band of ``w`` blocks."""
    name: str
    dtype: str
    batch: int
    hq: int
    hkv: int
    d: int
    n_bytes: int
    block: int
    w: int
    note: str = ""
    kind: str = "blockmask"

    def as_dict(self):
        return asdict(self)


# 8K-byte contexts as in the page's long-context setting, the head shape of a
# ~100M-parameter byte model (12 heads of 64), blocks of 128 bytes (one MFMA
# query tile), a band of 2 blocks; bytes from workloads.inputs.mixed_bytes
GZIP_BLOCKMASK_PREFILL = BlockMaskWorkload(
    name="gzip_blockmask_prefill_b8_8k", dtype="bf16", batch=8, hq=12, hkv=12, d=64, n_bytes=8192, block=128,
    w=2, note="8 sequences of 8192 synthetic bytes of mixed compressibility")

ALL = [TINY_PREFILL_F32, LLAMA3B_K0_PREFILL, LLAMA8B_K0_PREFILL, SELECTIVE_DECODE, HIER_DECODE]
NEXT = [COMPACT_DECODE, LLAMA3B_K16_PREFILL, GZIP_BLOCKMASK_PREFILL]
BY_NAME = {w.name: w for w in ALL + NEXT}
