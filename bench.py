"""Benchmark of the ThinKV decode hot path on one MI355X.

One step = one pass of the whole path over one batch: paged decode attention
over the mixed-precision, hole-bearing cache (with the staged self token) ->
thought classification and kv_append_quant of the new token at its label's
precision (one call, kv_classify_append) -> kv_plan_budget (token budget
ladder) -> kv_evict_segment (the two in one call, kv_plan_budget_evict).

Default workload: the B256 eviction-churn decode loop (Hq32/Hkv8, D128, g64,
starting lengths U{4k..32k}, 5% token budget, R/E/T 8/4/2-bit codes,
planted-temperature queries), the largest configuration; --workload llama8b
runs the same step on the Llama-8B-like layer (B32, 16k generated tokens, 10%
budget).  Two decode batches are in flight by default (--streams 2): copy j of
the state is stepped on stream j with its own buffers, each attention launch
waits for the previous step's attention, and one copy's state calls run beside
the other copy's attention (--streams 1: every call in order on one stream).
Besides the step, the line carries:
  - `configs`: the attention call alone on each static workload -- tiny (B1,
    G1, D64), llama8b (B32, G4, D128), qwen14b (B64, G5, ragged lengths,
    scattered block tables), gptoss20b (B128, G8, D64, sinks) with a 128-token
    window and with full attention -- each timed as the median of 5
    repetitions of 50 back-to-back launches, with its algorithmic bytes,
    achieved GB/s and fraction of the 8 TB/s peak, and the oracle's rate on
    the same state;
  - `stream_read`: a plain 128-bit streaming read of a 2 GiB buffer in the
    same process (the HBM read ceiling of this machine);
  - `step_split_us`: per-call device time of the step (a second pass with
    events between the calls).
Options: --policy anneal (the TBE annealing schedule instead of the ladder),
--compact (the gather-compaction baseline after every eviction), --layers N,
--formats page (FP8 E4M3 / FP4 E2M1 / ternary codes).

Every state is replicated into enough copies to exceed the 256 MB Infinity
Cache and consecutive launches rotate through them, so each launch reads its
cache from HBM.  All inputs are resident in HBM before any timed region.
A device error reported by any cache (tkv_get_error) aborts the run with a
non-zero exit status and no result line.

Prints ONE JSON line.
"""
from __future__ import annotations

import argparse
import ctypes
import dataclasses
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode-attn KV tokens/s and achieved HBM GB/s (% of MI355X peak), 1 GPU"
HBM_PEAK_GBS = 8000.0
CLASS_BITS = (8, 4, 2)
ATTN_CONFIGS = ("tiny", "llama8b", "qwen14b", "gptoss20b")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class HipEvents:
    """Timing events of the HIP runtime torch has loaded, created with
    hipEventDisableSystemFence: recording one then costs no system-scope cache
    writeback / invalidation, which a default event performs and which would
    both slow the following work and inflate what the event pair measures."""

    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self, n, torch_events=False):
        C = ctypes
        self.C = C
        self.torch_events = torch_events
        if torch_events:
            import torch
            self.ev = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
            return
        self.hip = C.CDLL("libamdhip64.so.7")          # the runtime already in the process
        self.hip.hipEventCreateWithFlags.argtypes = [C.c_void_p, C.c_uint]
        self.hip.hipEventRecord.argtypes = [C.c_void_p, C.c_void_p]
        self.hip.hipEventElapsedTime.argtypes = [C.c_void_p, C.c_void_p, C.c_void_p]
        self.hip.hipEventDestroy.argtypes = [C.c_void_p]
        self.hip.hipStreamWaitEvent.argtypes = [C.c_void_p, C.c_void_p, C.c_uint]
        self.ev = []
        for _ in range(n):
            e = C.c_void_p()
            if self.hip.hipEventCreateWithFlags(C.byref(e), self.DISABLE_SYSTEM_FENCE) != 0:
                raise RuntimeError("hipEventCreateWithFlags failed")
            self.ev.append(e)

    def record(self, i, stream):
        if self.torch_events:
            self.ev[i].record()
        elif self.hip.hipEventRecord(self.ev[i], self.C.c_void_p(stream)) != 0:
            raise RuntimeError("hipEventRecord failed")

    def wait(self, i, stream):
        """Make `stream` wait for event i (recorded on another stream)."""
        if self.torch_events:
            raise RuntimeError("cross-stream waits need the HIP events")
        if self.hip.hipStreamWaitEvent(self.C.c_void_p(stream), self.ev[i], 0) != 0:
            raise RuntimeError("hipStreamWaitEvent failed")

    def elapsed_ms(self, i, j):
        if self.torch_events:
            return self.ev[i].elapsed_time(self.ev[j])
        ms = self.C.c_float()
        if self.hip.hipEventElapsedTime(self.C.byref(ms), self.ev[i], self.ev[j]) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def close(self):
        if not self.torch_events:
            for e in self.ev:
                self.hip.hipEventDestroy(e)
        self.ev = []


# ---------------------------------------------------------------------------
# algorithmic bytes of one attention call, from an exported state
# ---------------------------------------------------------------------------
_POP16 = np.array([bin(m).count("1") for m in range(1 << 16)], np.int64)


def attn_bytes(state, L, seq_ids, q_pos, window=0, self_token=False, sinks=False):
    """Bytes one paged_decode_attn call must move, per the byte model: codes +
    fp16 (scale, zero) of every attended cached token and KV head; per visited
    block its id and mask word (with a window also its largest position and
    the 16 slot positions); the queries, outputs, statistics, sinks and the
    staged self token.  Returns (bytes, KV-code bytes, attended cached tokens)."""
    D, g, Hkv, Hq = L.head_dim, L.group_size, L.num_kv_heads, L.num_q_heads
    NG = D // g
    per_tok = [Hkv * 2 * (D * b // 8 + NG * 4) for b in CLASS_BITS]
    seq = state["seq"].reshape(L.max_seqs, 16)
    bt = state["btab"].reshape(L.max_seqs, 3, L.max_blocks_per_seq)
    kv = 0
    meta = 0
    tokens = 0
    for c in range(3):
        blk = state[f"blk{c}"].reshape(-1, 4)
        pos = state[f"slot{c}"].reshape(-1, 16, 2)[:, :, 0]
        for i, s in enumerate(seq_ids):
            nb = int(seq[s, c])
            ids = bt[s, c, :nb]
            masks = blk[ids, 0].astype(np.int64) & 0xFFFF
            if window > 0:
                lo = int(q_pos[i]) - window + 1
                live = (masks != 0) & (blk[ids, 1] >= lo)
                bits = (masks[:, None] >> np.arange(16)[None, :]) & 1
                inw = bits.astype(bool) & (pos[ids] >= lo)
                n = int(inw[live].sum())
                meta += int(live.sum()) * (4 + 2 + 4 + 16 * 4)
            else:
                n = int(_POP16[masks].sum())
                meta += int((masks != 0).sum()) * (4 + 2)
            tokens += n
            kv += n * per_tok[c]
    B = len(seq_ids)
    io = B * Hq * D * 2 + B * Hq * D * 4 + B * Hq * 12 + (Hq * 4 if sinks else 0)
    if self_token:
        io += B * Hkv * D * 4 * 2
    return kv + meta + io, kv, tokens


# ---------------------------------------------------------------------------
# building and replicating states
# ---------------------------------------------------------------------------
def replicate(w, L=None, min_total=1 << 30, copies=0):
    """Build the workload's state through the C-ABI, then import it into
    enough further caches that all copies together exceed min_total bytes."""
    import torch
    from thought_adaptive_mixed_amd import binding, drive
    L = L or w.layout
    sizes = binding.buffer_sizes(drive.gpu_layout(L))
    R = copies or max(2, math.ceil(min_total / sum(sizes[:-1])))
    c0 = binding.Cache(drive.gpu_layout(L), w.block_order)
    drive.build_gpu(w, c0)
    torch.cuda.synchronize()
    check_errors([c0], f"build of {w.name}")
    state = c0.export()
    caches = [c0] + [binding.Cache(drive.gpu_layout(L), w.block_order) for _ in range(R - 1)]
    for c in caches[1:]:
        c.import_(state)
    return caches, state


def check_errors(caches, what):
    errs = [c.get_error() for c in caches]
    bad = [(i, e) for i, e in enumerate(errs) if e[0] or e[2]]
    if bad:
        log(f"[bench] device errors after {what}: (copy, (kinds, lowest seq, count)) {bad[:8]}")
        log("[bench] a result measured with skipped work is not reported")
        sys.exit(3)


# ---------------------------------------------------------------------------
# the oracle as it stands (CPU baseline)
# ---------------------------------------------------------------------------
def _oracle_cache(w, state):
    import oracle
    Lw = w.layout
    ol = oracle.OracleLayout(Lw.num_kv_heads, Lw.num_q_heads, Lw.head_dim, Lw.group_size, Lw.pool_blocks,
                             Lw.max_seqs, Lw.max_blocks_per_seq, Lw.max_segments_per_seq, Lw.bits, Lw.num_layers,
                             Lw.code_format)
    oc = oracle.OracleCache(ol, w.block_order)
    oc.import_(state)
    return oc


def _omp_threads(n):
    try:
        ctypes.CDLL("libgomp.so.1").omp_set_num_threads(int(n))
    except OSError:
        pass


def oracle_attention_rate(w, state, window, n_seq, threads, budget_s=3.0):
    """Attended cached KV tokens per second of the oracle's attention on the
    first n_seq sequences of a static state (repeated up to budget_s)."""
    oc = _oracle_cache(w, state)
    _omp_threads(threads)
    sel = w.seq_ids[:n_seq]
    tokens, reps, t0 = 0, 0, time.perf_counter()
    while True:
        _, _, na = oc.attention(sel, w.q_pos[:n_seq], w.q_bf16[:n_seq], window=window, sinks=w.sinks)
        tokens += int(na.sum()); reps += 1
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    return tokens / dt, reps, dt


def cpu_baseline(w, state, ch, n_seq, budget_s=12.0, max_reps=1000, policy="ladder", r0=64, compact=False):
    """The oracle as it stands, on a sample of n_seq sequences of the same
    workload: one full step (attention with the self token, classify, append,
    ladder or annealing plan, evict) per repetition, on all host cores the
    process may use."""
    import oracle
    cores = len(os.sched_getaffinity(0))
    _omp_threads(cores)
    oc = _oracle_cache(w, state)
    sel = w.seq_ids[:n_seq]
    q, k, v, pos = ch.step_inputs(0)
    tokens = 0
    t0 = time.perf_counter()
    reps = 0
    while True:
        p = (pos[:n_seq] + reps).astype(np.int32)
        out, st, na = oc.attention(sel, p, q[:n_seq], k_self=k[:n_seq], v_self=v[:n_seq])
        lab = oracle.classify(st.astype(np.float32), *ch.tau)
        oc.append(sel, p, lab, k[:n_seq], v[:n_seq])
        if policy == "anneal":
            ops = oc.plan_anneal(sel, r0, 256)
        else:
            ops = oc.plan_budget(sel, ch.budget[0], ch.budget[1], 256)
        if ops[0].size:
            oc.evict(*ops)
            if compact:
                oc.compact(ops[0])
        tokens += int(na.sum()) - sel.size            # cached tokens (the self token excluded)
        reps += 1
        if time.perf_counter() - t0 > budget_s or reps >= max_reps:
            break
    dt = time.perf_counter() - t0
    return {"value": tokens / dt, "unit": "KV tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"{reps} full steps (attention+classify+append+{policy}+evict"
                      f"{'+compact' if compact else ''}) on {sel.size} of "
                      f"{w.seq_ids.size} sequences of the same cache, fp64 attention, {dt:.1f} s"}


# ---------------------------------------------------------------------------
# the streaming-read ceiling
# ---------------------------------------------------------------------------
def stream_ceiling(nbytes=2 << 30, reps=5, passes=4):
    import torch
    from thought_adaptive_mixed_amd import binding
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    buf.fill_(1)
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    sh = torch.cuda.current_stream().cuda_stream
    f = binding.stream_read(buf, sink, stream=sh, prepare=True)
    f()
    torch.cuda.synchronize()
    ev = HipEvents(2 * reps)
    for r in range(reps):
        ev.record(2 * r, sh)
        for _ in range(passes):
            f()
        ev.record(2 * r + 1, sh)
    torch.cuda.synchronize()
    t = sorted(ev.elapsed_ms(2 * r, 2 * r + 1) / passes for r in range(reps))
    ev.close()
    del buf
    ms = t[len(t) // 2]
    return {"GB/s": nbytes / (ms * 1e-3) / 1e9, "bytes": nbytes, "ms_median": ms,
            "kernel": "k_stream_read (128-bit loads, grid stride, 2048 work-groups of 256 lanes)",
            "timing": f"median of {reps} repetitions of {passes} back-to-back reads"}


# ---------------------------------------------------------------------------
# the attention call alone on a static workload
# ---------------------------------------------------------------------------
def attention_config(name, reps=5, launches=50, oracle_s=3.0):
    """Median over `reps` repetitions of `launches` back-to-back attention
    launches rotating over state copies, per window of the workload."""
    import torch
    from thought_adaptive_mixed_amd import drive, synth
    t0 = time.time()
    w = synth.WORKLOADS[name]()
    caches, state = replicate(w)
    L = w.layout
    B, Hq, D = w.seq_ids.size, L.num_q_heads, L.head_dim
    dv = drive.dev
    seq_d, pos_d, q_d = dv(w.seq_ids, np.int32), dv(w.q_pos, np.int32), dv(w.q_bf16, np.uint16)
    sinks_d = dv(w.sinks, np.float32) if w.sinks is not None else None
    out = torch.empty(B, Hq, D, dtype=torch.float32, device="cuda")
    stats = torch.empty(B, Hq, 3, dtype=torch.float32, device="cuda")
    n_att = torch.zeros(B, dtype=torch.int32, device="cuda")
    ws = torch.empty(max(caches[0].workspace_bytes(B), 16), dtype=torch.uint8, device="cuda")
    sh = torch.cuda.current_stream().cuda_stream
    res = {}
    cores = len(os.sched_getaffinity(0))
    # the dispatch order of each copy (tkv_attn_order), made once: the state does not change here
    orders = [torch.zeros(1 + B, dtype=torch.int32, device="cuda") for _ in caches]
    for c, o in zip(caches, orders):
        c.attn_order(seq_d, o)
    def timed(window):
        calls = [c.attention(seq_d, pos_d, q_d, out, ws, stats=stats, n_attended=n_att, sinks=sinks_d,
                             window=window, order=o, stream=sh, prepare=True) for c, o in zip(caches, orders)]
        for i in range(2 * len(calls)):
            calls[i % len(calls)]()
        torch.cuda.synchronize()
        ev = HipEvents(2 * reps)
        for r in range(reps):
            ev.record(2 * r, sh)
            for i in range(launches):
                calls[(r * launches + i) % len(calls)]()
            ev.record(2 * r + 1, sh)
        torch.cuda.synchronize()
        per = sorted(ev.elapsed_ms(2 * r, 2 * r + 1) / launches for r in range(reps))
        ev.close()
        check_errors(caches, f"attention on {name}")
        _, _, toks = attn_bytes(state, L, w.seq_ids, w.q_pos, window, sinks=w.sinks is not None)
        got = int(n_att.sum().item())
        assert got == toks, (name, window, got, toks)
        return per
    for window in w.windows:
        per = timed(window)
        ms = per[len(per) // 2]
        nbytes, kvb, toks = attn_bytes(state, L, w.seq_ids, w.q_pos, window, sinks=w.sinks is not None)
        floor = {}
        if window > 0:
            # the latency floor of the windowed call: a window of one block's
            # positions (one step per work-group, the same launch shape)
            pf = timed(16)
            floor = {"floor_us_window16": pf[len(pf) // 2] * 1e3,
                     "floor_note": "same call with a 16-position window: launch, prologue, one step, epilogue"}
        gbs = nbytes / (ms * 1e-3) / 1e9
        key = name if len(w.windows) == 1 else f"{name}_{'full' if window == 0 else f'window{window}'}"
        ora = {}
        n_seq = min(B, 8)
        rate, orep, odt = oracle_attention_rate(w, state, window, n_seq, cores, oracle_s)
        ora["oracle_kv_tokens_per_s"] = rate
        ora["oracle_sample"] = f"{orep} calls on {n_seq} of {B} sequences, {cores} cores, {odt:.1f} s"
        if name in ("tiny", "llama8b"):
            rate1, orep1, odt1 = oracle_attention_rate(w, state, window, min(B, 2), 1, oracle_s)
            ora["oracle_1thread_kv_tokens_per_s"] = rate1
            ora["oracle_1thread_sample"] = f"{orep1} calls on {min(B, 2)} of {B} sequences, 1 thread, {odt1:.1f} s"
        res[key] = {"batch": B, "heads": f"Hq{Hq}/Hkv{L.num_kv_heads}", "head_dim": D, "group": L.group_size,
                    "window": window, "sinks": w.sinks is not None, "copies": len(caches),
                    "attended_tokens": toks, "bytes_per_launch": nbytes, "kv_code_bytes": kvb,
                    "us_per_launch": ms * 1e3, "us_per_launch_reps": [p * 1e3 for p in per],
                    "kv_tokens_per_s": toks / (ms * 1e-3), "achieved_GBs": gbs, "frac": gbs / HBM_PEAK_GBS,
                    **floor, **ora}
        log(f"[bench] {key}: {ms * 1e3:.2f} us/launch, {nbytes / 1e6:.2f} MB, {gbs:.0f} GB/s "
            f"({gbs / HBM_PEAK_GBS:.3f} of peak), {toks / (ms * 1e-3) / 1e9:.2f} G KV tokens/s")
    del caches
    torch.cuda.empty_cache()
    log(f"[bench] {name} done in {time.time() - t0:.1f} s")
    return res


# ---------------------------------------------------------------------------
# the decode step
# ---------------------------------------------------------------------------
def workload_name(args):
    if args.workload == "llama8b":
        head = "llama8b-like reasoning decode, one layer: B32, Hq32/Hkv8, D128, g64, 16k generated tokens/seq, "
        body = ("10% budget (1638 retained), " if args.policy == "ladder" else "")
    else:
        head = "B256 eviction-churn reasoning decode loop, one layer: Hq32/Hkv8, D128, g64, "
        body = ("starting lengths U{4k..32k}, " + ("5% budget, " if args.policy == "ladder" else ""))
    pol = "ladder" if args.policy == "ladder" else f"anneal (TBE annealing schedule, r0 {args.r0})"
    s = (head + body + "R/E/T 8/4/2-bit, planted-temperature queries; step = attention+classify+append+"
         + pol + "+evict" + ("+compact (gather-compaction baseline, dense start)" if args.compact else ""))
    if args.layers > 1:
        s += f"; {args.layers} layers per step sharing the block tables (each layer holds the one-layer state's records)"
    if args.formats == "page":
        s += "; page code formats (R FP8 E4M3, E FP4 E2M1, T ternary)"
    return s


ORDER_EVERY = 16       # decode steps of a copy between two dispatch orders


def n_copies(args, sizes):
    """State copies: enough for more than 1 GiB (beyond the Infinity Cache),
    a multiple of the streams (copy j always runs on stream j % streams)."""
    R = args.copies or max(2, math.ceil((1 << 30) / sum(sizes[:-1])))
    return -(-R // args.streams) * args.streams


def step_bench(args):
    import torch
    from thought_adaptive_mixed_amd import binding, drive, synth
    split_steps = 0 if args.attn_only else args.split_steps
    total = args.warmup + args.steps + 2 * split_steps     # timed steps, then the split, then per-kernel timing
    log(f"[bench] building the {args.workload} workload")
    t0 = time.time()
    # the decode sequence is generated for a fixed horizon of 128 steps (or
    # more when asked): the timed workload then does not depend on how many
    # extra steps follow it, and at the B256 loop it is the 128-step sequence
    # the full-shape GPU test checks against the oracle step by step
    horizon = max(total, 128)
    ch = synth.bench_cycle(steps=horizon) if args.workload == "llama8b" else synth.churn(steps=horizon)
    if args.formats == "page":
        ch.base = synth.page_formats(ch.base)
    w = ch.base
    if args.compact:
        # room to compact every sequence in one call: each class's pool doubled
        # (a compaction pops all its new blocks before it returns the old ones)
        Lw = w.layout
        grow = tuple(p + p + 16 for p in Lw.pool_blocks)
        if w.block_order is not None:
            w.block_order = [np.concatenate([o, np.arange(Lw.pool_blocks[c], grow[c], dtype=np.int32)])
                             for c, o in enumerate(w.block_order)]
        w.layout = dataclasses.replace(Lw, pool_blocks=grow)
    L = w.layout
    B = w.seq_ids.size
    NL = max(1, args.layers)
    c0 = binding.Cache(drive.gpu_layout(L), w.block_order)
    drive.build_gpu(w, c0)
    torch.cuda.synchronize()
    dv0 = lambda a: drive.dev(a, np.int32)
    if args.policy == "anneal":
        # the built state has never been annealed: apply the schedule until it plans nothing
        m_all = L.max_tokens_per_call
        t_ops = [torch.zeros(m_all, dtype=torch.int32, device="cuda") for _ in range(3)]
        t_bits = torch.zeros(m_all, dtype=torch.uint8, device="cuda")
        t_n = torch.zeros(1, dtype=torch.int32, device="cuda")
        for _ in range(1000):
            c0.plan_anneal(dv0(w.seq_ids), args.r0, m_all, t_n, *t_ops, t_bits)
            c0.evict(*t_ops, t_bits, n_ops_dev=t_n, n_ops=m_all)
            if int(t_n.item()) == 0:
                break
        torch.cuda.synchronize()
    if args.compact:
        c0.compact(dv0(w.seq_ids))                 # start dense
        torch.cuda.synchronize()
    check_errors([c0], "the build")
    state = c0.export()
    if NL > 1:
        # every layer of the layered cache holds the one-layer state's records (same bytes and work per layer)
        state1 = state
        state = dict(state1)
        for cc in range(3):
            P = L.pool_blocks[cc]
            state[f"pool{cc}"] = np.repeat(state1[f"pool{cc}"].reshape(P, 1, -1), NL, axis=1).ravel()
        del c0
        L = dataclasses.replace(L, num_layers=NL)
        sizes = binding.buffer_sizes(drive.gpu_layout(L))
        R = n_copies(args, sizes)
        caches = [binding.Cache(drive.gpu_layout(L), w.block_order) for _ in range(R)]
        for c in caches:
            c.import_(state)
        state = state1
    else:
        sizes = binding.buffer_sizes(drive.gpu_layout(L))
        R = n_copies(args, sizes)
        caches = [c0] + [binding.Cache(drive.gpu_layout(L), w.block_order) for _ in range(R - 1)]
        for c in caches[1:]:
            c.import_(state)
    L1 = dataclasses.replace(L, num_layers=1)
    q0, _, _, pos0 = ch.step_inputs(0)
    abytes, kvbytes, init_tokens = attn_bytes(state, L1, w.seq_ids, pos0, 0, self_token=True)
    log(f"[bench] state {sum(sizes[:-1]) / 1e6:.1f} MB x {R} copies, built in {time.time() - t0:.1f} s; "
        f"algorithmic bytes per attention call {abytes / 1e6:.2f} MB")

    # inputs for every step, resident on the device.  Step s runs on copy
    # s % R as that copy's (s // R)-th decode step: each copy replays the same
    # decode sequence (positions, planted thought types, new tokens), so every
    # copy sees the planted segment process as one cache would.
    dv = drive.dev
    seq_d = dv(w.seq_ids, np.int32)
    per_copy = []
    for i in range((total + R - 1) // R):
        q, k, v, pos = ch.step_inputs(i)
        kl, vl = np.tile(k, (1, NL, 1)), np.tile(v, (1, NL, 1))
        per_copy.append((dv(q, np.uint16), dv(k, np.float32), dv(v, np.float32), dv(pos, np.int32),
                         dv(kl, np.float32) if NL > 1 else None, dv(vl, np.float32) if NL > 1 else None))
    steps_in = [per_copy[s // R] for s in range(total)]
    Hq, D = L.num_q_heads, L.head_dim
    # Batches in flight: copy j runs on stream j % nst, each stream with its own
    # output, statistics, label, op-list and workspace buffers.  With two
    # streams, the state calls of one copy's step (latency-bound kernels of one
    # or a few work-groups) run while the other copy's attention streams the
    # cache; the attention launches themselves never overlap (each waits for
    # the previous step's attention to end), so every attention launch is
    # timed alone.
    nst = args.streams
    streams = [torch.cuda.current_stream()] + [torch.cuda.Stream() for _ in range(nst - 1)]
    sts = [x.cuda_stream for x in streams]
    sh = sts[0]
    n_att = torch.zeros(total, B, dtype=torch.int32, device="cuda")         # one row per step
    max_ops = 1024

    def buffers():
        return dict(out=torch.empty(B, Hq, D, dtype=torch.float32, device="cuda"),
                    stats=torch.empty(B, NL, Hq, 3, dtype=torch.float32, device="cuda"),  # every layer's rows
                    ws=torch.empty(max(caches[0].workspace_bytes(B), 16), dtype=torch.uint8, device="cuda"),
                    labels=torch.empty(B, dtype=torch.uint8, device="cuda"),
                    n_ops=torch.zeros(1, dtype=torch.int32, device="cuda"),
                    ops=[torch.zeros(max_ops, dtype=torch.int32, device="cuda") for _ in range(3)],
                    bits=torch.zeros(max_ops, dtype=torch.uint8, device="cuda"))
    bufs = [buffers() for _ in range(nst)]

    # the attention's dispatch order (tkv_attn_order: longest sequences first),
    # one per copy, made before the first step and again every ORDER_EVERY steps
    # of that copy inside the steps (lengths change slowly)
    orders = [torch.zeros(1 + B, dtype=torch.int32, device="cuda") for _ in range(R)]
    for c, o in zip(caches, orders):
        c.attn_order(seq_d, o)
    torch.cuda.synchronize()

    # every call's C arguments are converted once, before anything is timed;
    # the steps after the timed region (split and per-kernel timing) run on
    # one stream
    n_pipe = args.warmup + args.steps
    stream_of = lambda s: sts[s % nst] if s < n_pipe else sh
    calls_a, calls_b = [], []
    for s in range(total):
        c = caches[s % R]
        bf = bufs[s % nst]
        st_s = stream_of(s)
        q, k, v, pos, kl, vl = steps_in[s]
        stats = bf["stats"]
        renew = [c.attn_order(seq_d, orders[s % R], stream=st_s, prepare=True)] if (s // R) % ORDER_EVERY == 0 else []
        calls_a.append(renew + [c.attention(seq_d, pos, q, bf["out"], bf["ws"], stats=stats[:, l], n_attended=n_att[s],
                                            k_self=k, v_self=v, layer=l, stats_stride=NL * Hq * 3, order=orders[s % R],
                                            stream=st_s, prepare=True)
                                for l in range(NL)])
        o_seq, o_seg, o_keep = bf["ops"]
        calls_b.append([
            # classification of every layer's statistics rows, inside the append's allocation kernel
            ("classify+append", c.classify_append(seq_d, pos, stats.view(B, NL * Hq, 3), ch.tau[0], ch.tau[1],
                                                  kl if NL > 1 else k, vl if NL > 1 else v, labels_out=bf["labels"],
                                                  stream=st_s, prepare=True)),
            ("plan+evict",
             c.plan_anneal_evict(seq_d, args.r0, max_ops, bf["n_ops"], o_seq, o_seg, o_keep, bf["bits"], stream=st_s,
                                 prepare=True)
             if args.policy == "anneal" else
             c.plan_budget_evict(seq_d, ch.budget[0], ch.budget[1], max_ops, bf["n_ops"], o_seq, o_seg, o_keep,
                                 bf["bits"], stream=st_s, prepare=True)),
        ] + ([("compact", c.compact(o_seq, n_dev=bf["n_ops"], n=max_ops, stream=st_s, prepare=True))]
             if args.compact else []))

    # events: (before, after) each attention, the timed region's ends, and
    # one join event per further stream
    T0, T1 = 2 * total, 2 * total + 1
    ev = HipEvents(2 * total + 2 + nst, torch_events=args.torch_events)

    # Steps are launched eagerly (a replayed HIP graph per step measured slower
    # on this stack).  The attention launch is bracketed by events on its own
    # stream; with several streams it first waits for the previous step's
    # attention to end.
    def step(s):
        st_s = stream_of(s)
        if nst > 1 and s > 0:
            ev.wait(2 * (s - 1) + 1, st_s)
        ev.record(2 * s, st_s)
        for f in calls_a[s]:
            f()
        ev.record(2 * s + 1, st_s)
        if not args.attn_only:
            for _, f in calls_b[s]:
                f()

    if args.copy_calibration:
        nbytes = args.copy_calibration << 20
        src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] copy calibration: 3 x {nbytes} bytes read + written")
        del src, dst

    log("[bench] warmup")
    for s in range(args.warmup):
        step(s)
    torch.cuda.synchronize()
    log(f"[bench] timed ({nst} stream{'s' if nst > 1 else ''})")
    h0 = time.perf_counter()
    ev.record(T0, sh)
    for j in range(1, nst):
        ev.wait(T0, sts[j])
    for s in range(args.warmup, args.warmup + args.steps):
        step(s)
    for j in range(1, nst):                   # the region ends when every stream is done
        ev.record(T1 + j, sts[j])
        ev.wait(T1 + j, sh)
    ev.record(T1, sh)
    h1 = time.perf_counter()
    torch.cuda.synchronize()
    ms_total = ev.elapsed_ms(T0, T1)
    log(f"[bench] host enqueue {(h1 - h0) * 1e6 / args.steps:.1f} us/step, device {ms_total * 1e3 / args.steps:.1f} us/step")
    attn_ms = [ev.elapsed_ms(2 * s, 2 * s + 1) for s in range(args.warmup, args.warmup + args.steps)]
    check_errors(caches, "the timed steps")

    # per-call split: further steps with an event between every call
    split = {}
    kernels, kernels_launches = {}, {}
    if split_steps:
        names = ["attention"] + [n for n, _ in calls_b[0]]
        es = HipEvents((len(names) + 1) * split_steps)
        k = len(names) + 1
        s0 = args.warmup + args.steps
        for j, s in enumerate(range(s0, s0 + split_steps)):
            es.record(k * j, sh)
            for f in calls_a[s]:
                f()
            es.record(k * j + 1, sh)
            for i, (_, f) in enumerate(calls_b[s]):
                f()
                es.record(k * j + 2 + i, sh)
        torch.cuda.synchronize()
        for i, n in enumerate(names):
            t = sorted(es.elapsed_ms(k * j + i, k * j + i + 1) * 1e3 for j in range(split_steps))
            split[n] = t[len(t) // 2]
        es.close()
        # per kernel: as many further steps with every kernel launch bracketed
        # by events (tkv_kernel_timing), apart from the split above so that
        # their events do not enter it
        for c in caches:
            c.kernel_timing(True)
        for s in range(s0 + split_steps, total):
            for f in calls_a[s]:
                f()
            for _, f in calls_b[s]:
                f()
        torch.cuda.synchronize()
        tot = {}
        for c in caches:
            times, dropped = c.kernel_times()
            for name, (us, calls) in times.items():
                a = tot.setdefault(name, [0.0, 0])
                a[0] += us
                a[1] += calls
            c.kernel_timing(False)
        # mean duration of each kernel per step (HIP events around each launch)
        kernels = {name: round(us / split_steps, 2) for name, (us, calls) in tot.items()}
        kernels_launches = {name: calls / split_steps for name, (us, calls) in tot.items()}
        check_errors(caches, "the split steps")

    cached = n_att[args.warmup:args.warmup + args.steps].sum().item() - args.steps * B   # self token excluded
    tokens1 = int(cached)                                  # one layer's attended cached tokens
    tokens = tokens1 * NL
    ms_step = ms_total / args.steps
    attn_avg = float(np.mean(attn_ms))                     # every layer's attention of a step
    # the cache changes a little from step to step (appends, evictions): scale
    # the KV part of the byte count by the attended tokens actually seen
    abytes_step = abytes - kvbytes + kvbytes * (tokens1 / args.steps) / max(init_tokens, 1)
    achieved = abytes_step / (attn_avg / NL * 1e-3) / 1e9
    result = {
        "metric": METRIC,
        "value": tokens / (ms_total * 1e-3),
        "unit": "KV tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("f16 MFMA (int8/4/2 codes as exact fp16 subnormals), f32 accumulate" if args.formats == "int" else
                  "f16 MFMA (FP8 E4M3 / FP4 E2M1 codes converted exactly to fp16, ternary codes as fp16 "
                  "subnormals), f32 accumulate"),
        "data": "synthetic",
        "config": {"workload": workload_name(args), "batch": B, "copies": R,
                   "attended_cached_per_step": tokens / args.steps,
                   "launch": ("eager, one stream" if args.streams == 1 else
                              f"eager, {args.streams} streams: copy j on stream j % {args.streams}, the state calls "
                              f"of one copy's step beside the next copy's attention, attention launches never "
                              f"overlapping"),
                   **({"layers": NL} if NL > 1 else {})},
        "attn_ms": attn_avg,
        "attn_kv_tokens_per_s": (tokens / args.steps) / (attn_avg * 1e-3),
        "step_split_us": split,
        "step_kernels_us": kernels,
        "step_kernels_note": (f"per kernel, microseconds per step (launches per step: "
                              f"{ {k: round(v, 2) for k, v in kernels_launches.items()} }), from HIP events around "
                              f"every kernel launch of {split_steps} further steps (tkv_kernel_timing)")
        if kernels else None,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": None,
                     "kernel": "k_attn (paged_decode_attn; one launch per layer and step)",
                     "bytes_per_launch": abytes_step},
    }
    return result, (w, state, ch)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=6)
    ap.add_argument("--split-steps", type=int, default=16, help="extra steps timed call by call")
    ap.add_argument("--streams", type=int, choices=(1, 2, 3, 4), default=2,
                    help="decode batches in flight (state copies stepped on their own streams)")
    ap.add_argument("--copies", type=int, default=0, help="state copies (0 = enough for > 1 GiB)")
    ap.add_argument("--cpu-seqs", type=int, default=16)
    ap.add_argument("--workload", choices=("churn256", "llama8b", "none"), default="churn256",
                    help="the B256 churn decode loop (4k..32k, 5%% budget) or the llama8b-like layer (B32, 16k, 10%%); "
                         "'none' times only the --configs attention calls (diagnostic: no result line)")
    ap.add_argument("--policy", choices=("ladder", "anneal"), default="ladder",
                    help="eviction planner of the step: the token-budget ladder, or the TBE annealing schedule")
    ap.add_argument("--r0", type=int, default=64, help="first retention of the annealing schedule")
    ap.add_argument("--compact", action="store_true",
                    help="compact the sequences each step evicted from (gather-compaction baseline)")
    ap.add_argument("--layers", type=int, default=1,
                    help="layers per decode step sharing the block tables (the one-layer state replicated)")
    ap.add_argument("--formats", choices=("int", "page"), default="int",
                    help="code formats of the 8/4/2-bit classes: asymmetric integer, or FP8 E4M3 / FP4 E2M1 / ternary")
    ap.add_argument("--configs", default=",".join(ATTN_CONFIGS),
                    help="static workloads whose attention call is timed alone (comma list; 'none' for none)")
    ap.add_argument("--no-stream", action="store_true", help="skip the streaming-read ceiling")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--attn-only", action="store_true", help="time only the attention calls of the steps (diagnostic)")
    ap.add_argument("--torch-events", action="store_true", help="time with torch's default events (diagnostic)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="before the timed region, copy MIB MiB device-to-device 3 times (a plain copy kernel of "
                         "known size, to scale hardware byte counters by)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the hot path shards by "
              f"sequence with no exchange, so N GPUs would run N independent copies of this step.",
              file=sys.stderr)
        sys.exit(2)

    if args.torch_events and args.streams > 1:
        print("--torch-events times one stream only: add --streams 1", file=sys.stderr)
        sys.exit(2)
    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.workload == "none":
        names = [] if args.configs == "none" else [n for n in args.configs.split(",") if n]
        out = {}
        for n in names:
            log(f"[bench] attention alone: {n}")
            out.update(attention_config(n))
        print(json.dumps({"configs": out}), flush=True)
        return
    result, (w, state, ch) = step_bench(args)
    if not args.no_stream:
        log("[bench] streaming-read ceiling")
        sc = stream_ceiling()
        result["stream_read"] = sc
        result["roofline"]["frac_of_stream_read"] = result["roofline"]["achieved"] / sc["GB/s"]
        log(f"[bench] stream read {sc['GB/s']:.0f} GB/s")
    names = [] if args.configs == "none" else [n for n in args.configs.split(",") if n]
    if names:
        result["configs"] = {}
        for n in names:
            log(f"[bench] attention alone: {n}")
            result["configs"].update(attention_config(n))
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (oracle)")
        result["cpu_baseline"] = cpu_baseline(w, state, ch, min(args.cpu_seqs, w.seq_ids.size), policy=args.policy,
                                              r0=args.r0, compact=args.compact)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
