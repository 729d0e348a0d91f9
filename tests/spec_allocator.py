"""Logical specification of the cache's allocator, segment and eviction rules,
written with Python dicts and lists (no packed arrays, no codes).

It restates the rules the oracle documents -- LIFO free-slot stack per
(sequence, class), global LIFO block stack per class with blocks returned only
on reset, segments as maximal runs of one thought type, eviction of the oldest
tokens of a segment with slots pushed in ascending position order, downgrades
popping new slots in ascending position order before the old slots are pushed,
and the per-call failure rules -- in a different representation, so brute
force over short op sequences can catch indexing slips in the C oracle.
"""
from __future__ import annotations

BS = 16
CLASS = {8: 0, 4: 1, 2: 2}
CBITS = (8, 4, 2)
EINVAL, ENOMEM, ENOSEG = 1, 2, 3   # bit numbers in the error flag word


class Spec:
    def __init__(self, pool_blocks, max_seqs, max_blocks, max_segs, type_bits=(8, 4, 2), order=None):
        self.max_seqs, self.max_blocks, self.max_segs = max_seqs, max_blocks, max_segs
        self.type_bits = type_bits
        # pop order: first element popped first
        self.free = [list(order[c]) if order is not None else list(range(pool_blocks[c])) for c in range(3)]
        self.seqs = {}
        self.block = {}       # (c, blk) -> {"valid": set(), "maxpos": int, "owner": int}
        self.slot = {}        # (c, slot) -> (pos, seg)
        self.flags, self.minseq, self.count = 0, 0x7FFFFFFF, 0

    def _seq(self, s):
        if s not in self.seqs:
            self.seqs[s] = {"blocks": [[], [], []], "stack": [[], [], []], "segs": [],
                            "length": 0, "nret": 0, "napp": 0}
        return self.seqs[s]

    def _err(self, bit, s):
        self.flags |= 1 << bit
        self.minseq = min(self.minseq, s)
        self.count += 1

    def _pop(self, s, c):
        q = self._seq(s)
        if not q["stack"][c]:
            blk = self.free[c].pop(0)
            q["blocks"][c].append(blk)
            self.block[(c, blk)] = {"valid": set(), "maxpos": -1, "owner": s}
            q["stack"][c].extend(blk * BS + t for t in reversed(range(BS)))
        return q["stack"][c].pop()

    def _occupy(self, c, slot, pos, seg):
        b = self.block[(c, slot // BS)]
        b["valid"].add(slot % BS)
        b["maxpos"] = max(b["maxpos"], pos)
        self.slot[(c, slot)] = (pos, seg)

    def append(self, toks):
        """toks: list of (seq, pos, type).  Returns per-token (class, slot) or None."""
        failed, dry, out = set(), [False] * 3, []
        for s, pos, y in toks:
            out.append(None)
            if not (0 <= s < self.max_seqs):
                self._err(EINVAL, s if s >= 0 else 0x7FFFFFFF); continue
            if s in failed:
                continue
            q = self._seq(s)
            if y > 2 or pos < q["length"]:
                self._err(EINVAL, s); failed.add(s); continue
            c = CLASS[self.type_bits[y]]
            new_seg = not q["segs"] or q["segs"][-1]["type"] != y or q["segs"][-1]["bits"] != CBITS[c]
            if new_seg and len(q["segs"]) == self.max_segs:
                self._err(ENOMEM, s); failed.add(s); continue
            if not q["stack"][c]:
                if len(q["blocks"][c]) == self.max_blocks:
                    self._err(ENOMEM, s); failed.add(s); continue
                if dry[c] or not self.free[c]:
                    dry[c] = True; self._err(ENOMEM, s); failed.add(s); continue
            slot = self._pop(s, c)
            if new_seg:
                q["segs"].append({"type": y, "bits": CBITS[c], "first": pos, "last": pos, "ntot": 0, "nret": 0})
            seg = q["segs"][-1]
            seg["last"] = pos; seg["ntot"] += 1; seg["nret"] += 1
            self._occupy(c, slot, pos, len(q["segs"]) - 1)
            q["length"] = pos + 1; q["nret"] += 1; q["napp"] += 1
            out[-1] = (c, slot)
        return out

    def _seg_slots(self, s, k, c):
        q = self._seq(s)
        found = []
        for blk in q["blocks"][c]:
            for t in sorted(self.block[(c, blk)]["valid"]):
                sl = blk * BS + t
                if self.slot[(c, sl)][1] == k:
                    found.append(sl)
        return sorted(found, key=lambda sl: self.slot[(c, sl)][0])

    def evict(self, ops):
        failed, dry = set(), [False] * 3
        seen = []
        for s, k, keep_n, nb in ops:
            prior = list(seen)
            seen.append((s, k))
            if not (0 <= s < self.max_seqs):
                self._err(EINVAL, s if s >= 0 else 0x7FFFFFFF); continue
            if s in failed:
                continue
            q = self._seq(s)
            if not (0 <= k < len(q["segs"])):
                self._err(ENOSEG, s); failed.add(s); continue
            seg = q["segs"][k]
            if (s, k) in prior or keep_n < 0 or nb not in (0, 2, 4, 8) or (nb and nb > seg["bits"]):
                self._err(EINVAL, s); failed.add(s); continue
            if seg["nret"] == 0:
                self._err(ENOSEG, s); failed.add(s); continue
            c = CLASS[seg["bits"]]
            r = seg["nret"]
            keep = min(keep_n, r)
            down = nb and nb < seg["bits"] and keep > 0
            if down:
                c2 = CLASS[nb]
                have = len(q["stack"][c2])
                need = -(-(keep - have) // BS) if keep > have else 0
                if len(q["blocks"][c2]) + need > self.max_blocks:
                    self._err(ENOMEM, s); failed.add(s); continue
                if need > 0 and (dry[c2] or need > len(self.free[c2])):
                    dry[c2] = True; self._err(ENOMEM, s); failed.add(s); continue
            slots = self._seg_slots(s, k, c)
            ev = len(slots) - keep
            for sl in slots[:ev]:
                self.block[(c, sl // BS)]["valid"].discard(sl % BS)
                q["stack"][c].append(sl)
            if down:
                for sl in slots[ev:]:
                    pos = self.slot[(c, sl)][0]
                    ns = self._pop(s, c2)
                    self._occupy(c2, ns, pos, k)
                for sl in slots[ev:]:
                    self.block[(c, sl // BS)]["valid"].discard(sl % BS)
                    q["stack"][c].append(sl)
                seg["bits"] = nb
            seg["nret"] = keep
            q["nret"] -= ev

    def compact(self, seqs):
        """Gather compaction: for each sequence (its first listing only) and
        each class it holds blocks of, its retained tokens, oldest first, are
        placed 16 to a block in blocks taken from the class's free list; the
        tail of the last such block is the new free-slot stack.  The old blocks
        are released only after every listed sequence has taken its blocks."""
        dry = [False] * 3
        done, plans = set(), []
        for s in seqs:
            if not (0 <= s < self.max_seqs):
                self._err(EINVAL, s if s >= 0 else 0x7FFFFFFF); continue
            if s in done:
                continue
            done.add(s)
            q = self._seq(s)
            toks = [sorted(self.slot[(c, b * BS + t)] for b in q["blocks"][c] for t in self.block[(c, b)]["valid"])
                    for c in range(3)]
            need = [-(-len(toks[c]) // BS) for c in range(3)]
            short = [c for c in range(3) if need[c] and (dry[c] or need[c] > len(self.free[c]))]
            for c in short:
                dry[c] = True
            if short:
                self._err(ENOMEM, s); continue
            plans.append((s, toks, [[self.free[c].pop(0) for _ in range(need[c])] for c in range(3)]))
        released = []
        for s, toks, fresh in plans:
            q = self._seq(s)
            for c in range(3):
                if not q["blocks"][c]:
                    continue
                released.append((c, q["blocks"][c]))
                for j, blk in enumerate(fresh[c]):
                    part = toks[c][BS * j:BS * (j + 1)]
                    self.block[(c, blk)] = {"valid": set(range(len(part))), "maxpos": max(p for p, _ in part),
                                            "owner": s}
                    for t, rec in enumerate(part):
                        self.slot[(c, blk * BS + t)] = rec
                q["blocks"][c] = list(fresh[c])
                used = len(toks[c]) % BS
                q["stack"][c] = [fresh[c][-1] * BS + t for t in range(BS - 1, used - 1, -1)] if used else []
        for c, blocks in released:
            for blk in blocks:
                del self.block[(c, blk)]
                self.free[c].insert(0, blk)

    def reset(self, seqs):
        for s in seqs:
            if not (0 <= s < self.max_seqs):
                self._err(EINVAL, s if s >= 0 else 0x7FFFFFFF); continue
            q = self._seq(s)
            for c in range(3):
                for blk in q["blocks"][c]:
                    del self.block[(c, blk)]
                    self.free[c].insert(0, blk)
            del self.seqs[s]

    def anneal(self, seq_list, r0, max_ops):
        """TBE annealing: walking a sequence's segments from the newest back,
        every T segment passed is one more event for the older segments; an R
        or E segment seen after e >= 1 events keeps r0 // 2**(e-1) tokens."""
        ops = []
        for s in seq_list:
            if not (0 <= s < self.max_seqs):
                continue
            segs = self._seq(s)["segs"]
            found, events = [], 0
            for k in reversed(range(len(segs))):
                g = segs[k]
                if g["type"] == 2:
                    events += 1
                elif events and g["nret"] > r0 // 2 ** (events - 1):
                    found.append((s, k, r0 // 2 ** (events - 1), 0))
            ops.extend(reversed(found))
        return ops[:max_ops]

    def plan(self, seq_list, num, den, max_ops):
        ops = []
        for s in seq_list:
            if not (0 <= s < self.max_seqs):
                continue
            q = self._seq(s)
            segs = q["segs"]
            budget = q["length"] * num // den
            nr = q["nret"]
            if nr <= budget:
                continue
            ts = [k for k, g in enumerate(segs) if g["type"] == 2 and g["nret"] > 0]
            newest = ts[-1] if ts else -1
            for k in range(len(segs) - 1):
                if nr <= budget:
                    break
                g = segs[k]
                if g["type"] == 2 and g["nret"] > 0 and k != newest:
                    ops.append((s, k, 0, 0)); nr -= g["nret"]
            if nr > budget:
                for k in range(len(segs) - 1):
                    g = segs[k]
                    if g["type"] == 1 and g["bits"] > 2 and g["nret"] > 0:
                        ops.append((s, k, g["nret"], 2)); break
        return ops[:max_ops]
