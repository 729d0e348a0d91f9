"""Seeded synthetic workloads shaped like the pages' reasoning-model decode.

This module only draws random inputs and schedules: segment lengths and
thought types, K/V rows, queries, sinks, pool permutations, and the lists of
append / evict calls that build a cache state.  It holds none of the method's
arithmetic (no quantization, attention, classification or allocation); both
the HIP path and the CPU oracle consume exactly the same arrays.

Workloads (sizes from the five configurations the measurements use):

1. tiny      B1, Hq=Hkv=4, D64, g32, 512 tokens; segments U{16..64}, types
             R/E/T .4/.4/.2; 30% of T+E tokens evicted by whole segments
             (the last partly) and half of them refilled by new tokens.
2. llama8b   B32, Hq32/Hkv8, D128, g64, 16k generated tokens per sequence,
             1638 retained (10% budget); segment lengths lognormal mean 48;
             R/E/T .35/.45/.20; K/V N(0,1) with 1% outlier channels x8.
3. qwen14b   B64, Hq40/Hkv8, D128, g64; lengths lognormal, median 24k, cap
             32k; 5% budget; pools 70% occupied after the build, block order
             a seeded permutation so block tables are scattered.
4. gptoss20b B128, Hq64/Hkv8, D64, g32, 32k context, 5% budget; one learned
             sink logit per query head; timed with a 128-token window and
             with full attention.
5. churn     B256, Hq32/Hkv8, D128, g64, starting lengths U{4k..32k}, 5%
             budget, 1024 decode steps of classify -> append -> evict ->
             attention with planted-temperature queries.

The thought types drawn here stand in for the pages' reasoning traces (the
math and coding benchmarks named on the pages are not used).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Iterator, List, Optional, Tuple

import numpy as np

R, E, T = 0, 1, 2
TYPE_BITS = {R: 8, E: 4, T: 2}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even fp32 -> bf16 bit patterns (input preparation)."""
    u = np.ascontiguousarray(x, np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32)


@dataclasses.dataclass
class Layout:
    num_kv_heads: int
    num_q_heads: int
    head_dim: int
    group_size: int
    pool_blocks: Tuple[int, int, int]
    max_seqs: int
    max_blocks_per_seq: int
    max_segments_per_seq: int
    max_tokens_per_call: int = 4096
    bits: Tuple[int, int, int] = (8, 4, 2)
    num_layers: int = 1                  # layers sharing block tables and eviction
    code_format: int = 0                 # 0 integer codes; 1 FP8 E4M3 / FP4 E2M1 / ternary


@dataclasses.dataclass
class AppendCall:
    seq_ids: np.ndarray
    positions: np.ndarray
    thought: np.ndarray
    kv_seed: Tuple[int, ...]


@dataclasses.dataclass
class EvictCall:
    seq_ids: np.ndarray
    seg_ids: np.ndarray
    keep_n: np.ndarray
    new_bits: np.ndarray


@dataclasses.dataclass
class Workload:
    name: str
    seed: int
    layout: Layout
    block_order: Optional[List[np.ndarray]]
    calls: list                      # AppendCall | EvictCall, in order
    seq_ids: np.ndarray              # batch -> sequence
    q_pos: np.ndarray
    q_bf16: np.ndarray               # uint16 [B, Hq, D]
    sinks: Optional[np.ndarray]
    windows: Tuple[int, ...]
    outlier_k: np.ndarray            # flat (head*D + dim) indices scaled x8 in K
    outlier_v: np.ndarray
    budget: Tuple[int, int]          # (num, den) token budget fraction
    retained: np.ndarray             # retained tokens per sequence after the build

    def kv(self, call: AppendCall):
        return draw_kv(call.kv_seed, call.seq_ids.size, self.layout, self.outlier_k, self.outlier_v)

    def attended_tokens(self, window: int = 0) -> int:
        return int(self.retained.sum()) if window == 0 else -1


def draw_kv(seed, n, layout: Layout, outlier_k, outlier_v):
    rng = np.random.default_rng(list(seed))
    H, D = layout.num_kv_heads * layout.num_layers, layout.head_dim     # every layer's rows
    k = rng.standard_normal((n, H * D), dtype=np.float32)
    v = rng.standard_normal((n, H * D), dtype=np.float32)
    if outlier_k is not None and outlier_k.size:
        k[:, outlier_k] *= np.float32(8.0)
        v[:, outlier_v] *= np.float32(8.0)
    return k.reshape(n, H, D), v.reshape(n, H, D)


# ---------------------------------------------------------------------------
# segment process
# ---------------------------------------------------------------------------
def lognormal_segments(rng, total, mean=48.0, sigma=0.5, probs=(0.35, 0.45, 0.20)):
    """Contiguous thought segments covering positions [0, total)."""
    mu = math.log(mean) - sigma * sigma / 2.0
    lens, types = [], []
    covered = 0
    while covered < total:
        ln = max(1, int(round(rng.lognormal(mu, sigma))))
        ln = min(ln, total - covered)
        lens.append(ln)
        types.append(int(rng.choice(3, p=probs)))
        covered += ln
    return np.array(lens, np.int64), np.array(types, np.int64)


def uniform_segments(rng, total, lo=16, hi=64, probs=(0.4, 0.4, 0.2)):
    lens, types = [], []
    covered = 0
    while covered < total:
        ln = min(int(rng.integers(lo, hi + 1)), total - covered)
        lens.append(ln)
        types.append(int(rng.choice(3, p=probs)))
        covered += ln
    return np.array(lens, np.int64), np.array(types, np.int64)


def method_segments(appended_types: np.ndarray):
    """Segment ids the cache assigns to a sequence's appended tokens: a new id
    whenever the thought type changes between consecutive appends."""
    if appended_types.size == 0:
        return np.zeros(0, np.int64)
    change = np.concatenate([[0], (appended_types[1:] != appended_types[:-1]).astype(np.int64)])
    return np.cumsum(change)


@dataclasses.dataclass
class SeqPlan:
    positions: np.ndarray   # appended positions, ascending
    types: np.ndarray       # appended types
    evict: List[Tuple[int, int]]   # (method segment id, keep_n)
    retained: int
    length: int


def plan_sequence(rng, L, n_keep, tail_min=128, over=1.15, seg_fn=lognormal_segments):
    """Retain the newest >= tail_min tokens (whole segments) plus random older
    whole segments until ceil(over * n_keep) tokens are appended; then evict
    whole older T/E method segments (the last one partly) down to n_keep."""
    lens, types = seg_fn(rng, L)
    starts = np.concatenate([[0], np.cumsum(lens)[:-1]])
    nseg = lens.size
    chosen = np.zeros(nseg, bool)
    tail = 0
    j = nseg - 1
    while j >= 0 and tail < tail_min:
        chosen[j] = True; tail += lens[j]; j -= 1
    n_tail_segs = nseg - 1 - j
    target = int(math.ceil(over * n_keep))
    total = tail
    order = rng.permutation(j + 1) if j >= 0 else np.zeros(0, np.int64)
    for s in order:
        if total >= target:
            break
        chosen[s] = True; total += lens[s]
    idx = np.nonzero(chosen)[0]
    positions = np.concatenate([np.arange(starts[s], starts[s] + lens[s]) for s in idx])
    tps = np.concatenate([np.full(lens[s], types[s]) for s in idx])
    mseg = method_segments(tps)
    # method segments entirely older than the tail segments
    tail_first_pos = starts[nseg - n_tail_segs] if n_tail_segs > 0 else L
    n_m = int(mseg[-1]) + 1 if mseg.size else 0
    cand = []
    for m in range(n_m):
        sel = mseg == m
        if tps[sel][0] == R:
            continue
        if positions[sel][-1] >= tail_first_pos:
            continue
        cand.append((m, int(sel.sum())))
    excess = total - n_keep
    evict = []
    removed = 0
    for ci in rng.permutation(len(cand)):
        if excess <= 0:
            break
        m, cnt = cand[ci]
        if cnt <= excess:
            evict.append((m, 0)); excess -= cnt; removed += cnt
        else:
            evict.append((m, cnt - excess)); removed += excess; excess = 0
    retained = total - removed
    return SeqPlan(positions.astype(np.int64), tps.astype(np.int64), evict, int(retained), int(L))


def interleave_appends(plans: List[SeqPlan], seq_base: int, max_call: int, seed, start_index=0):
    """Append calls that interleave sequences round-robin by token rank."""
    calls = []
    maxlen = max(p.positions.size for p in plans)
    buf_s, buf_p, buf_t = [], [], []
    ci = start_index

    def flush():
        nonlocal ci
        if buf_s:
            calls.append(AppendCall(np.array(buf_s, np.int32), np.array(buf_p, np.int32),
                                    np.array(buf_t, np.uint8), (seed, 100 + ci)))
            ci += 1
            buf_s.clear(); buf_p.clear(); buf_t.clear()

    for r in range(maxlen):
        for b, p in enumerate(plans):
            if r < p.positions.size:
                buf_s.append(seq_base + b); buf_p.append(int(p.positions[r])); buf_t.append(int(p.types[r]))
                if len(buf_s) == max_call:
                    flush()
    flush()
    return calls


def evict_calls(plans: List[SeqPlan], seq_base=0):
    s, g, k, nb = [], [], [], []
    for b, p in enumerate(plans):
        for m, keep in p.evict:
            s.append(seq_base + b); g.append(m); k.append(keep); nb.append(0)
    if not s:
        return []
    return [EvictCall(np.array(s, np.int32), np.array(g, np.int32), np.array(k, np.int32),
                      np.array(nb, np.uint8))]


def outlier_channels(rng, H, D):
    n = int(math.ceil(0.01 * H * D))
    return (np.sort(rng.choice(H * D, n, replace=False)).astype(np.int64),
            np.sort(rng.choice(H * D, n, replace=False)).astype(np.int64))


def blocks_needed(plans: List[SeqPlan]):
    """Blocks per class the build acquires: appends come before evictions, so
    no slot is reused during the build."""
    need = np.zeros((len(plans), 3), np.int64)
    for b, p in enumerate(plans):
        for y in range(3):
            c = {8: 0, 4: 1, 2: 2}[TYPE_BITS[y]]
            need[b, c] += int((p.types == y).sum())
    return -(-need // 16)


def queries(rng, B, Hq, D, beta=None):
    u = rng.standard_normal((B, Hq, D), dtype=np.float32)
    if beta is not None:
        u *= np.asarray(beta, np.float32)[:, None, None]
    return f32_to_bf16_bits(u).reshape(B, Hq, D)


# ---------------------------------------------------------------------------
# workloads
# ---------------------------------------------------------------------------
def tiny(seed=1001) -> Workload:
    rng = np.random.default_rng(seed)
    Hq = Hkv = 4; D = 64; g = 32; N = 512
    lens, types = uniform_segments(rng, N)
    tps = np.concatenate([np.full(l, t) for l, t in zip(lens, types)])
    mseg = method_segments(tps)
    n_m = int(mseg[-1]) + 1
    seg_type = np.array([tps[mseg == m][0] for m in range(n_m)])
    seg_cnt = np.array([(mseg == m).sum() for m in range(n_m)])
    n_te = int((tps != R).sum())
    target = int(math.floor(0.3 * n_te))
    ev = []; gone = 0; ev_cnt = {E: 0, T: 0}
    for m in rng.permutation(n_m):
        if gone >= target:
            break
        if seg_type[m] == R:
            continue
        take = min(int(seg_cnt[m]), target - gone)
        ev.append((int(m), int(seg_cnt[m]) - take))
        gone += take; ev_cnt[int(seg_type[m])] += take
    layout = Layout(Hkv, Hq, D, g, (64, 64, 64), 1, 64, 256, 1024)
    calls = [AppendCall(np.zeros(N, np.int32), np.arange(N, dtype=np.int32), tps.astype(np.uint8), (seed, 100))]
    calls.append(EvictCall(np.zeros(len(ev), np.int32), np.array([e[0] for e in ev], np.int32),
                           np.array([e[1] for e in ev], np.int32), np.zeros(len(ev), np.uint8)))
    n_e, n_t = ev_cnt[E] // 2, ev_cnt[T] // 2
    refill_t = np.array([E] * n_e + [T] * n_t, np.uint8)
    pos = np.arange(N, N + refill_t.size, dtype=np.int32)
    calls.append(AppendCall(np.zeros(refill_t.size, np.int32), pos, refill_t, (seed, 101)))
    q = queries(rng, 1, Hq, D)
    retained = np.array([N - gone + refill_t.size], np.int64)
    return Workload("tiny", seed, layout, None, calls, np.zeros(1, np.int32),
                    np.array([N + refill_t.size], np.int32), q, None, (0,),
                    np.zeros(0, np.int64), np.zeros(0, np.int64), (1, 10), retained)


def _static(name, seed, B, Hq, Hkv, D, g, lengths, n_keep, occupancy=None, permute=False, sinks=False,
            windows=(0,), max_call=4096, slack_blocks=8, segs=None) -> Workload:
    rng = np.random.default_rng(seed)
    plans = [plan_sequence(rng, int(lengths[b]), int(n_keep[b])) for b in range(B)]
    need = blocks_needed(plans)
    per_class = need.sum(axis=0)
    if occupancy is not None:
        pool = tuple(int(math.ceil(per_class[c] / occupancy)) + 1 for c in range(3))
    else:
        pool = tuple(int(per_class[c]) + slack_blocks * B for c in range(3))
    max_blocks = int(need.max()) + slack_blocks
    max_segs = max(int(method_segments(p.types)[-1]) + 1 for p in plans) + (segs or 64)
    layout = Layout(Hkv, Hq, D, g, pool, B, max_blocks, max_segs, max_call)
    order = [rng.permutation(pool[c]).astype(np.int32) for c in range(3)] if permute else None
    ok, ov = outlier_channels(rng, Hkv, D)
    calls = interleave_appends(plans, 0, max_call, seed) + evict_calls(plans)
    q = queries(rng, B, Hq, D)
    sk = rng.standard_normal(Hq, dtype=np.float32) if sinks else None
    retained = np.array([p.retained for p in plans], np.int64)
    return Workload(name, seed, layout, order, calls, np.arange(B, dtype=np.int32),
                    np.array([p.length for p in plans], np.int32), q, sk, windows, ok, ov,
                    (1, 10), retained)


def llama8b(seed=1002, B=32, L=16384) -> Workload:
    n = int(L * 0.1)
    return _static("llama8b", seed, B, 32, 8, 128, 64, [L] * B, [n] * B)


def qwen14b(seed=1003, B=64) -> Workload:
    rng = np.random.default_rng(seed + 50000)
    L = np.clip(np.round(np.exp(math.log(24576) + 0.3 * rng.standard_normal(B))), 4096, 32768).astype(np.int64)
    n = (L * 5) // 100
    w = _static("qwen14b", seed, B, 40, 8, 128, 64, L, n, occupancy=0.7, permute=True)
    w.budget = (1, 20)
    return w


def gptoss20b(seed=1004, B=128, L=32768) -> Workload:
    n = (L * 5) // 100
    w = _static("gptoss20b", seed, B, 64, 8, 64, 32, [L] * B, [n] * B, sinks=True, windows=(128, 0))
    w.budget = (1, 20)
    return w


def small_static(seed=77, B=3, Hq=8, Hkv=2, D=128, g=64, L=900, frac=0.3, sinks=False, permute=True,
                 windows=(0,)) -> Workload:
    """Parity-sized cache (several blocks and splits, ragged tails)."""
    rng = np.random.default_rng(seed + 7)
    lengths = rng.integers(L // 2, L + 1, B)
    n = (lengths * int(frac * 100)) // 100
    w = _static("small", seed, B, Hq, Hkv, D, g, lengths, n, permute=permute, sinks=sinks, windows=windows,
                max_call=256, slack_blocks=4)
    return w


def layered(w: Workload, num_layers: int) -> Workload:
    """The workload with num_layers layers sharing its block tables: the same
    appends, evictions and queries, K/V rows drawn for every layer, the
    outlier channels repeated in each layer."""
    H, D = w.layout.num_kv_heads, w.layout.head_dim
    w = dataclasses.replace(w, layout=dataclasses.replace(w.layout, num_layers=num_layers))
    if w.outlier_k is not None and w.outlier_k.size:
        w.outlier_k = np.concatenate([w.outlier_k + l * H * D for l in range(num_layers)])
        w.outlier_v = np.concatenate([w.outlier_v + l * H * D for l in range(num_layers)])
    return w


def page_formats(w: Workload) -> Workload:
    """The workload stored in the float / ternary code formats (FP8 E4M3 for
    the 8-bit class, FP4 E2M1 for the 4-bit class, ternary for the 2-bit
    class): the same calls and inputs."""
    return dataclasses.replace(w, layout=dataclasses.replace(w.layout, code_format=1))


def layer_queries(w: Workload, layer: int, beta=1.0) -> np.ndarray:
    """Seeded bf16 queries [B][Hq][D] of one layer (layer 0: the workload's own)."""
    if layer == 0:
        return w.q_bf16
    L = w.layout
    rng = np.random.default_rng([w.seed, 50000 + layer])
    return queries(rng, w.seq_ids.size, L.num_q_heads, L.head_dim,
                   np.full(w.seq_ids.size, beta, np.float32))


# ---------------------------------------------------------------------------
# decode-loop workloads (churn, and the bench step)
# ---------------------------------------------------------------------------
BETA = {E: 0.5, R: 1.75, T: 6.0}


@dataclasses.dataclass
class Churn:
    base: Workload
    steps: int
    target_types: np.ndarray     # [steps, B] planted type per step
    budget: Tuple[int, int]
    tau: Tuple[float, float] = (0.38, 0.85)

    def step_inputs(self, s: int):
        w = self.base
        Lh = w.layout
        B = w.seq_ids.size
        rng = np.random.default_rng([w.seed, 20000 + s])
        beta = np.array([BETA[int(t)] for t in self.target_types[s]], np.float32)
        q = queries(rng, B, Lh.num_q_heads, Lh.head_dim, beta)
        k, v = draw_kv((w.seed, 30000 + s), B, Lh, w.outlier_k, w.outlier_v)
        pos = (w.q_pos + s).astype(np.int32)
        return q, k, v, pos


def churn(seed=1005, B=256, steps=1024, lo=4096, hi=32768, frac=(1, 20), extra_blocks=None) -> Churn:
    rng = np.random.default_rng(seed + 60000)
    L0 = rng.integers(lo, hi + 1, B)
    n = (L0 * frac[0]) // frac[1]
    # room for every step's token to need a fresh block of any class
    grow = steps if extra_blocks is None else extra_blocks
    w = _static("churn", seed, B, 32, 8, 128, 64, L0, n, slack_blocks=grow // 16 + 4,
                segs=grow + 8)
    w.budget = frac
    tt = np.zeros((steps, B), np.int64)
    srng = np.random.default_rng(seed + 70000)
    for b in range(B):
        lens, types = lognormal_segments(srng, steps)
        tt[:, b] = np.concatenate([np.full(l, t) for l, t in zip(lens, types)])[:steps]
    return Churn(w, steps, tt, frac)


def bench_cycle(seed=1002, B=32, L=16384, steps=64) -> Churn:
    """Decode cycle on the llama8b-like cache: 10% budget, planted queries."""
    w = llama8b(seed, B, L)
    # pools and tables sized for `steps` more tokens per sequence
    lay = w.layout
    extra = steps // 16 + 4
    w.layout = dataclasses.replace(lay, pool_blocks=tuple(p + extra * B for p in lay.pool_blocks),
                                   max_blocks_per_seq=lay.max_blocks_per_seq + extra,
                                   max_segments_per_seq=lay.max_segments_per_seq + steps)
    srng = np.random.default_rng(seed + 70000)
    tt = np.zeros((steps, B), np.int64)
    for b in range(B):
        lens, types = lognormal_segments(srng, steps)
        tt[:, b] = np.concatenate([np.full(l, t) for l, t in zip(lens, types)])[:steps]
    return Churn(w, steps, tt, (1, 10))


def small_churn(seed=88, B=8, steps=96, lo=600, hi=1600, frac=(1, 10)) -> Churn:
    """Parity-sized decode loop (lockstep with the oracle every step)."""
    rng = np.random.default_rng(seed + 60000)
    L0 = rng.integers(lo, hi + 1, B)
    n = (L0 * frac[0]) // frac[1]
    w = _static("small_churn", seed, B, 8, 2, 128, 64, L0, n, slack_blocks=steps // 16 + 4, segs=steps + 8,
                permute=True, max_call=128)
    w.budget = frac
    tt = np.zeros((steps, B), np.int64)
    srng = np.random.default_rng(seed + 70000)
    for b in range(B):
        lens, types = lognormal_segments(srng, steps, mean=12.0)
        tt[:, b] = np.concatenate([np.full(l, t) for l, t in zip(lens, types)])[:steps]
    return Churn(w, steps, tt, frac)


WORKLOADS = {"tiny": tiny, "llama8b": llama8b, "qwen14b": qwen14b, "gptoss20b": gptoss20b}
