"""Plain model of the paged-KV block manager (host bookkeeping, no GPU).

TEST INFRASTRUCTURE ONLY, like the rest of ``oracle/``: the tests compare the
library's native manager with this model operation by operation.  It shares
no code with the library.

What it models, and where the pages state it:

* a fixed pool of physical blocks and a virtual-to-physical block table per
  request (mini-infer docs, "Systems Architecture" figure, box "Paged
  KV-Cache Memory Manager"; "Core Capabilities at a Glance" table, row
  "Memory Allocation": 16-token blocks with virtual block tables);
* prefix reuse keyed per block, with least-recently-used eviction of the
  cached blocks (zingnex.cn mini-infer thread, feature list item 4: prefix KV
  reuse by block-level hash and LRU eviction; the docs' "Prompt Caching" row:
  no recompute on shared prefixes);
* preemption of the lowest-priority sequence when the pool is exhausted (the
  docs' "OOM Resilience (v0.2.1)" row: lowest-priority sequences go back to
  WAITING).

The pages leave the policy details open; the readings taken (also listed in
the design notes): a new block is the smallest free id, else the cached block
released longest ago; a full block is identified by its token ids and the
identity of the block before it (identities are never reused); the block of
a prompt's last token is never taken from the cache; a sequence's full blocks
become shareable at its next append or at its release; among the
lowest-priority sequences the most recently admitted is preempted; rolling
back into a block shared with another sequence is refused.
"""
from __future__ import annotations

OK, NULL, SHAPE, NO_BLOCKS, STATE = 0, -1, -2, -7, -8


class BlockManager:
    def __init__(self, num_blocks: int, block_size: int, max_blocks_per_seq: int,
                 prefix_cache: bool):
        self.nb, self.bs, self.maxb, self.prefix = num_blocks, block_size, max_blocks_per_seq, \
            bool(prefix_cache)
        self.free = set(range(num_blocks))
        self.lru = []                      # cached blocks, least recently released first
        self.ref = [0] * num_blocks
        self.content = [None] * num_blocks  # (identity, parent identity, tokens) when shareable
        self.by_key = {}                   # (parent identity, tokens) -> block
        self.seqs = {}
        self.next_identity = 1
        self.next_order = 1

    # -- pool -------------------------------------------------------------
    def available(self):
        return len(self.free) + len(self.lru)

    def _forget(self, b):
        if self.content[b] is not None:
            _, parent, toks = self.content[b]
            del self.by_key[(parent, toks)]
            self.content[b] = None

    def _new_block(self):
        if self.free:
            b = min(self.free)
            self.free.remove(b)
        else:
            b = self.lru.pop(0)
            self._forget(b)
        self.ref[b] = 1
        return b

    def _share(self, b):
        if b in self.lru:
            self.lru.remove(b)
        self.ref[b] += 1

    def _release_block(self, b):
        self.ref[b] -= 1
        if self.ref[b] == 0:
            if self.content[b] is not None:
                self.lru.append(b)
            else:
                self.free.add(b)

    def _make_shareable(self, s):
        """Full blocks behind the sequence's end, in order, until one whose
        content is already shareable elsewhere."""
        if not self.prefix:
            return
        while s["keyed"] < s["len"] // self.bs and s["chain_ok"]:
            i = s["keyed"]
            b = s["blocks"][i]
            toks = tuple(s["tokens"][i * self.bs:(i + 1) * self.bs])
            if self.content[b] is None:
                if (s["last"], toks) in self.by_key:
                    s["chain_ok"] = False
                    break
                self.content[b] = (self.next_identity, s["last"], toks)
                self.by_key[(s["last"], toks)] = b
                self.next_identity += 1
            s["last"] = self.content[b][0]
            s["keyed"] += 1

    # -- operations (each returns (status, outputs...)) ------------------------
    def admit(self, seq_id, priority, tokens):
        n = len(tokens)
        if n < 1:
            return SHAPE, None, None
        nblk = -(-n // self.bs)
        if nblk > self.maxb:
            return SHAPE, None, None
        if seq_id in self.seqs:
            return STATE, None, None
        hits, parent = [], 0
        if self.prefix:
            for i in range((n - 1) // self.bs):
                key = (parent, tuple(tokens[i * self.bs:(i + 1) * self.bs]))
                if key not in self.by_key:
                    break
                b = self.by_key[key]
                hits.append(b)
                parent = self.content[b][0]
        in_lru = sum(1 for b in hits if b in self.lru)
        if nblk - len(hits) > self.available() - in_lru:
            return NO_BLOCKS, None, None
        for b in hits:
            self._share(b)
        blocks = hits + [self._new_block() for _ in range(nblk - len(hits))]
        s = {"blocks": blocks, "tokens": list(tokens) if self.prefix else [], "len": n,
             "prio": priority, "order": self.next_order, "keyed": len(hits),
             "last": self.content[hits[-1]][0] if hits else 0, "chain_ok": True}
        self.next_order += 1
        self.seqs[seq_id] = s
        cached = len(hits) * self.bs
        slots = [blocks[t // self.bs] * self.bs + t % self.bs for t in range(cached, n)]
        return OK, cached, slots

    def append(self, seq_id, tokens):
        n = len(tokens)
        if n < 1:
            return SHAPE, None
        if seq_id not in self.seqs:
            return STATE, None
        s = self.seqs[seq_id]
        new_len = s["len"] + n
        nblk = -(-new_len // self.bs)
        if nblk > self.maxb:
            return SHAPE, None
        if nblk - len(s["blocks"]) > self.available():
            return NO_BLOCKS, None
        self._make_shareable(s)
        while len(s["blocks"]) < nblk:
            s["blocks"].append(self._new_block())
        if self.prefix:
            s["tokens"] += list(tokens)
        slots = [s["blocks"][t // self.bs] * self.bs + t % self.bs
                 for t in range(s["len"], new_len)]
        s["len"] = new_len
        return OK, slots

    def decode_step(self, seq_ids, tokens):
        """One token for each listed sequence, all or nothing."""
        if len(set(seq_ids)) != len(seq_ids) or any(k not in self.seqs for k in seq_ids):
            return STATE, None
        need = 0
        for k in seq_ids:
            s = self.seqs[k]
            if s["len"] % self.bs == 0:
                if len(s["blocks"]) + 1 > self.maxb:
                    return SHAPE, None
                need += 1
        if need > self.available():
            return NO_BLOCKS, None
        slots = []
        for k, t in zip(seq_ids, tokens):
            st, sl = self.append(k, [t])
            assert st == OK
            slots += sl
        return OK, slots

    def truncate(self, seq_id, new_len):
        if seq_id not in self.seqs:
            return STATE
        s = self.seqs[seq_id]
        if new_len < 1 or new_len > s["len"]:
            return SHAPE
        keep = -(-new_len // self.bs)
        partial = new_len % self.bs != 0
        if partial and self.ref[s["blocks"][keep - 1]] > 1:
            return STATE
        for b in s["blocks"][keep:]:
            self._release_block(b)
        del s["blocks"][keep:]
        if partial:
            self._forget(s["blocks"][keep - 1])
        if self.prefix:
            del s["tokens"][new_len:]
        s["len"] = new_len
        s["keyed"] = min(s["keyed"], new_len // self.bs)
        s["last"] = self.content[s["blocks"][s["keyed"] - 1]][0] if s["keyed"] else 0
        s["chain_ok"] = True
        return OK

    def release(self, seq_id):
        if seq_id not in self.seqs:
            return STATE
        s = self.seqs.pop(seq_id)
        self._make_shareable(s)
        for b in s["blocks"]:
            self._release_block(b)
        return OK

    def preempt(self):
        if not self.seqs:
            return STATE, None
        victim = min(self.seqs, key=lambda k: (self.seqs[k]["prio"], -self.seqs[k]["order"]))
        self.release(victim)
        return OK, victim

    def block_tables(self, seq_ids):
        if any(k not in self.seqs for k in seq_ids):
            return STATE, None, None
        tables = [self.seqs[k]["blocks"] + [0] * (self.maxb - len(self.seqs[k]["blocks"]))
                  for k in seq_ids]
        return OK, tables, [self.seqs[k]["len"] for k in seq_ids]

    def stats(self):
        used = sum(1 for r in self.ref if r > 0)
        return len(self.free), len(self.lru), used, len(self.seqs)
