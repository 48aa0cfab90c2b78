"""Reference model of the host block pool (oracle; test infrastructure only).

Citation keys are listed in ``oracle/__init__.py``.

* Paged blocks with reference counts, sharing by fork, copy-on-write when a
  partly filled shared last block is appended to ([DQ] 08 PagedAttention:
  fixed-size pages, freed pages reused at once, copy-on-write sharing of a
  prefix; [LC] 2.3: parallel samples and beam candidates share prompt blocks
  through reference counts and copy-on-write).
* Chained block keys ([SW] 知识点三): h_j = H(encode(h_{j-1}, X_j, E)); the
  key of a block carries its whole prefix and the compatibility identity E,
  so equal last blocks under different prefixes get different keys.  The
  byte encoding is the library's own (documented in its header); the hash is
  SHA-256 (hashlib).
* [SW] 源码导读: counts say how many users hold a block, keys say what it
  holds; a block whose count reaches zero can still be matched until its
  memory is reused.  Physical use is counted over unique blocks.

The model mirrors the library's policy (blocks never keyed are reused
first, then keyed ones in release order), so tests can compare block ids
exactly.  That comparison is not independent of the policy; the pin that is
simulates the pool's memory contents (copy pairs applied, new tokens written
through the tables) and checks that every sequence reads back exactly its
own tokens, that written blocks are held by one sequence, that counts equal
table occurrences and that use equals the unique blocks in the tables.
"""

import hashlib
import struct

TAG = b"kvd-block-v1"


def block_hashes(tokens, block_size, identity=b""):
    """32-byte chained keys of the full blocks of ``tokens``."""
    if block_size < 1:
        raise ValueError("block_size must be >= 1")
    tokens = [int(t) for t in tokens]
    full = len(tokens) // block_size
    if any(t < 0 for t in tokens[:full * block_size]):
        raise ValueError("tokens must be >= 0")
    out = []
    parent = None
    for j in range(full):
        h = hashlib.sha256()
        h.update(TAG)
        if parent is None:
            h.update(struct.pack("<I", 0))
        else:
            h.update(struct.pack("<I", 32))
            h.update(parent)
        h.update(struct.pack("<I", len(identity)))
        h.update(identity)
        h.update(struct.pack("<I", block_size))
        h.update(struct.pack(f"<{block_size}I", *tokens[j * block_size:(j + 1) * block_size]))
        parent = h.digest()
        out.append(parent)
    return out


class PoolExhausted(Exception):
    pass


class BlockPool:
    def __init__(self, num_blocks, block_size):
        self.bs = block_size
        self.ref = [0] * num_blocks
        self.key = [None] * num_blocks
        self.never = list(range(num_blocks))   # free, never keyed (FIFO)
        self.evictable = []                    # keyed, count 0, release order
        self.by_key = {}
        self.seqs = {}
        self.next_seq = 0

    # -- blocks
    def available(self):
        return len(self.never) + len(self.evictable)

    def used(self):
        return len(self.ref) - self.available()

    def _take(self):
        if self.never:
            b = self.never.pop(0)
        else:
            b = self.evictable.pop(0)
            del self.by_key[self.key[b]]
            self.key[b] = None
        self.ref[b] = 1
        return b

    def _hold(self, b):
        if self.ref[b] == 0 and self.key[b] is not None:
            self.evictable.remove(b)
        self.ref[b] += 1

    def _drop(self, b):
        self.ref[b] -= 1
        if self.ref[b] == 0:
            (self.evictable if self.key[b] is not None else self.never).append(b)

    # -- sequences
    def _new_seq(self):
        free = [s for s in range(self.next_seq) if s not in self.seqs]
        s = free[0] if free else self.next_seq
        if not free:
            self.next_seq += 1
        self.seqs[s] = {"len": 0, "blocks": []}
        return s

    def create(self):
        return self._new_seq()

    def fork(self, s):
        src = self.seqs[s]
        c = self._new_seq()
        self.seqs[c] = {"len": src["len"], "blocks": list(src["blocks"])}
        for b in src["blocks"]:
            self._hold(b)
        return c

    def release(self, s):
        for b in self.seqs.pop(s)["blocks"]:
            self._drop(b)

    def append(self, s, n):
        """Returns the copy pairs [(old, new)] the caller must perform."""
        q = self.seqs[s]
        fill = q["len"] % self.bs
        cow = fill != 0 and self.ref[q["blocks"][-1]] > 1
        need = -(-(q["len"] + n) // self.bs) - len(q["blocks"]) + (1 if cow else 0)
        if n and need > self.available():
            raise PoolExhausted
        copies = []
        if n and cow:
            old = q["blocks"][-1]
            new = self._take()
            copies.append((old, new))
            self._drop(old)
            q["blocks"][-1] = new
        while len(q["blocks"]) * self.bs < q["len"] + n:
            q["blocks"].append(self._take())
        q["len"] += n
        return copies

    def commit(self, s, keys):
        q = self.seqs[s]
        if len(keys) > q["len"] // self.bs:
            raise ValueError("more keys than full blocks")
        for j, k in enumerate(keys):
            b = q["blocks"][j]
            if self.key[b] is not None or k in self.by_key:
                continue
            self.by_key[k] = b
            self.key[b] = k

    def create_with_prefix(self, keys):
        s = self._new_seq()
        q = self.seqs[s]
        for k in keys:
            b = self.by_key.get(k)
            if b is None:
                break
            q["blocks"].append(b)
            self._hold(b)
        q["len"] = len(q["blocks"]) * self.bs
        return s, len(q["blocks"])
