"""Pure-Python brute force for tiny block-paged inputs.

TEST INFRASTRUCTURE (see ``oracle/__init__.py``). This is a second, independent
formulation of the same definition, used to pin the C oracle on tiny inputs:
instead of dividing a position by the page size ([Hurray] Element Lookup) it
expands each sequence's block-table slice into the list of (page, slot) pairs
the slice covers, in order, and reads the live prefix of that list. The pool
is treated as a nested Python list [num_pages][page_size][num_heads][head_dim].
"""
import math


def slot_list(block_table, seq_ptr, s, page_size):
    """(physical page, slot) of every reserved position of sequence s, in
    logical order: the slice's pages one after another, each slot 0..P-1."""
    slots = []
    for k in range(seq_ptr[s], seq_ptr[s + 1]):
        for slot in range(page_size):
            slots.append((block_table[k], slot))
    return slots


def gather(pool4, block_table, seq_ptr, seq_lens):
    """Logical rows (each a [H][D] nested list) in sequence order."""
    rows = []
    for s in range(len(seq_lens)):
        slots = slot_list(block_table, seq_ptr, s, len(pool4[0]) if pool4 else 1)
        for page, slot in slots[: seq_lens[s]]:
            rows.append([list(head) for head in pool4[page][slot]])
    return rows


def scatter(pool4, src_rows, block_table, seq_ptr, seq_lens, seq_start=None,
            zero_tail=False, zero=0):
    """Writes src_rows into a deep copy of pool4 and returns it."""
    page_size = len(pool4[0])
    pool = [[[list(head) for head in slot] for slot in page] for page in pool4]
    row = 0
    for s in range(len(seq_lens)):
        start = 0 if seq_start is None else seq_start[s]
        slots = slot_list(block_table, seq_ptr, s, page_size)
        for i in range(seq_lens[s]):
            page, slot = slots[start + i]
            pool[page][slot] = [list(head) for head in src_rows[row]]
            row += 1
        if zero_tail and seq_lens[s] > 0:
            end = start + seq_lens[s]
            last_page, last_slot = slots[end - 1]
            for slot in range(last_slot + 1, page_size):
                pool[last_page][slot] = [[zero] * len(head) for head in pool[last_page][slot]]
    return pool


def validate(rank, paged_axis, num_pages, page_size, block_table, seq_ptr, seq_lens,
             total_tokens, seq_start=None):
    """All failing checks as a list of (name, index), in check order then
    index order; the first entry is what a validator must report."""
    fails = []
    if rank != 3:
        return [("rank", 0)]
    if paged_axis != 0:
        return [("paged_axis", 0)]
    num_seqs = len(seq_lens)
    if seq_ptr[0] != 0:
        fails.append(("seq_ptr_first", 0))
    if seq_ptr[num_seqs] != len(block_table):
        fails.append(("seq_ptr_last", num_seqs))
    fails += [("seq_ptr_order", s) for s in range(num_seqs) if seq_ptr[s] > seq_ptr[s + 1]]
    fails += [("page_range", k) for k, p in enumerate(block_table) if not 0 <= p < num_pages]
    for s in range(num_seqs):
        start = 0 if seq_start is None else seq_start[s]
        if start + seq_lens[s] > (seq_ptr[s + 1] - seq_ptr[s]) * page_size:
            fails.append(("seq_len", s))
    if sum(seq_lens) != total_tokens:
        fails.append(("total_tokens", 0))
    return fails


def disjoint_writes(page_size, block_table, seq_ptr, seq_lens, seq_start=None,
                    zero_tail=False):
    """None if a scatter's written slots are pairwise distinct, else the
    smallest sequence that writes a slot some write repeats (tokens' slots and,
    with zero_tail, the rest of the last token's page)."""
    writes = []
    for s in range(len(seq_lens)):
        start = 0 if seq_start is None else seq_start[s]
        mine = [block_table[seq_ptr[s] + t // page_size] * page_size + t % page_size
                for t in range(start, start + seq_lens[s])]
        if zero_tail and seq_lens[s]:
            last = start + seq_lens[s] - 1
            page = block_table[seq_ptr[s] + last // page_size]
            mine += [page * page_size + r for r in range(last % page_size + 1, page_size)]
        writes.append(mine)
    seen = {}
    for mine in writes:
        for slot in mine:
            seen[slot] = seen.get(slot, 0) + 1
    for s, mine in enumerate(writes):
        if any(seen[slot] > 1 for slot in mine):
            return s
    return None


def copy_pages(pool4, scales, src_pages, dst_pages):
    """Deep copy of pool4 (and of the flat scales list) with page dst_pages[i]
    replaced by page src_pages[i], applied in order."""
    page_size = len(pool4[0])
    pool = [[[list(head) for head in slot] for slot in page] for page in pool4]
    sc = None if scales is None else list(scales)
    for src, dst in zip(src_pages, dst_pages):
        pool[dst] = [[list(head) for head in slot] for slot in pool[src]]
        if sc is not None:
            sc[dst * page_size:(dst + 1) * page_size] = sc[src * page_size:(src + 1) * page_size]
    return pool, sc


def attention(q, k_pool4, v_pool4, block_table, seq_ptr, seq_lens, scale):
    """Decode attention with plain Python floats: q is [S][Hq][D], the pools
    [N][P][Hkv][D]. Query head hq reads kv head hq // (Hq // Hkv); scores
    are scale * q.k, weights exp(score - max), output the weighted mean of
    the values; a sequence without tokens gives zeros."""
    page_size = len(k_pool4[0])
    out = []
    for s in range(len(seq_lens)):
        slots = slot_list(block_table, seq_ptr, s, page_size)[: seq_lens[s]]
        heads = []
        for hq, qv in enumerate(q[s]):
            hkv = hq // (len(q[s]) // len(k_pool4[0][0]))
            if not slots:
                heads.append([0.0] * len(qv))
                continue
            scores = [scale * math.fsum(a * b for a, b in zip(qv, k_pool4[p][i][hkv]))
                      for p, i in slots]
            top = max(scores)
            w = [math.exp(x - top) for x in scores]
            total = math.fsum(w)
            heads.append([math.fsum(wt * v_pool4[p][i][hkv][d] for wt, (p, i) in zip(w, slots))
                          / total for d in range(len(qv))])
        out.append(heads)
    return out
