"""Host block manager of a paged KV cache, as plain Python.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

"How does paged attention work (in detail)", sections 2-4: the cache is a
pool of fixed-size physical blocks; each sequence has a block table (its
logical blocks in order); a block manager hands out free blocks, counts the
references to each block, returns a block to the free pool when its count
drops to zero, gives a sequence that must write into a shared block a copy
of it (copy-on-write, section 3.3), allocates a new block only when a new
token starts a logical block that is not mapped yet (section 4.1), and under
memory pressure moves a sequence's blocks to CPU memory and back (section
4.3; the vLLM paper summary, section 5, names the CPU block allocator).

Policy (the page's example manager keeps its free ids in a queue): blocks
are taken from the front of the free list and freed blocks go to its back,
in table order.  Every operation either succeeds completely or raises and
changes nothing.
"""
from __future__ import annotations


class NoFreeBlocks(Exception):
    pass


class _Pool:
    def __init__(self, n: int, order=None):
        self.free = list(range(n)) if order is None else [int(b) for b in order]
        assert sorted(self.free) == list(range(n))
        self.refs = {}

    def take(self, k: int):
        if len(self.free) < k:
            raise NoFreeBlocks()
        got, self.free = self.free[:k], self.free[k:]
        for b in got:
            self.refs[b] = 1
        return got

    def release(self, b: int):
        self.refs[b] -= 1
        if self.refs[b] == 0:
            del self.refs[b]
            self.free.append(b)


class BlockManager:
    def __init__(self, num_gpu_blocks: int, num_cpu_blocks: int, block_size: int,
                 gpu_free_order=None):
        self.bs = int(block_size)
        self.gpu = _Pool(num_gpu_blocks, gpu_free_order)
        self.cpu = _Pool(num_cpu_blocks)
        self.seqs = {}   # id -> {"blocks": [...], "len": int, "on_gpu": bool}

    # -- queries ---------------------------------------------------------
    def table(self, sid):
        return list(self.seqs[sid]["blocks"])

    def length(self, sid) -> int:
        return self.seqs[sid]["len"]

    def num_free(self, on_gpu: bool = True) -> int:
        return len((self.gpu if on_gpu else self.cpu).free)

    def ref_count(self, block: int, on_gpu: bool = True) -> int:
        return (self.gpu if on_gpu else self.cpu).refs.get(block, 0)

    # -- operations ------------------------------------------------------
    def add_sequence(self, sid, num_tokens: int):
        """A new sequence holding num_tokens tokens (its prompt)."""
        if sid in self.seqs:
            raise KeyError(f"sequence {sid} exists")
        need = -(-int(num_tokens) // self.bs)
        self.seqs[sid] = {"blocks": self.gpu.take(need), "len": int(num_tokens), "on_gpu": True}

    def fork(self, parent, child):
        """child shares every block of parent (parallel sampling, beam search)."""
        p = self.seqs[parent]
        if child in self.seqs:
            raise KeyError(f"sequence {child} exists")
        if not p["on_gpu"]:
            raise ValueError("fork of a swapped-out sequence")
        for b in p["blocks"]:
            self.gpu.refs[b] += 1
        self.seqs[child] = {"blocks": list(p["blocks"]), "len": p["len"], "on_gpu": True}

    def append_slot(self, sid):
        """Slot of the sequence's next token, and the (src, dst) copy the
        caller must perform first when that token lands in a shared block
        (else None)."""
        st = self.seqs[sid]
        if not st["on_gpu"]:
            raise ValueError("append to a swapped-out sequence")
        pos = st["len"]
        j = pos // self.bs
        pair = None
        if j == len(st["blocks"]):
            st["blocks"].append(self.gpu.take(1)[0])
        elif self.gpu.refs[st["blocks"][j]] > 1:
            new = self.gpu.take(1)[0]
            old = st["blocks"][j]
            self.gpu.release(old)
            st["blocks"][j] = new
            pair = (old, new)
        st["len"] = pos + 1
        return st["blocks"][j] * self.bs + pos % self.bs, pair

    def free(self, sid):
        st = self.seqs.pop(sid)
        pool = self.gpu if st["on_gpu"] else self.cpu
        for b in st["blocks"]:
            pool.release(b)

    def swap_out(self, sid):
        """Move the sequence's blocks to the CPU pool; returns the (gpu, cpu)
        copies to perform.  A shared GPU block stays for its other users."""
        st = self.seqs[sid]
        if not st["on_gpu"]:
            raise ValueError("already swapped out")
        dst = self.cpu.take(len(st["blocks"]))
        pairs = list(zip(st["blocks"], dst))
        for b in st["blocks"]:
            self.gpu.release(b)
        st["blocks"], st["on_gpu"] = dst, False
        return pairs

    def swap_in(self, sid):
        """Bring a swapped-out sequence back; returns the (cpu, gpu) copies."""
        st = self.seqs[sid]
        if st["on_gpu"]:
            raise ValueError("not swapped out")
        dst = self.gpu.take(len(st["blocks"]))
        pairs = list(zip(st["blocks"], dst))
        for b in st["blocks"]:
            self.cpu.release(b)
        st["blocks"], st["on_gpu"] = dst, True
        return pairs
