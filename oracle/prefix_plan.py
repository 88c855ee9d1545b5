"""Plain-Python definition of the shared-prefix decode plan.

TEST INFRASTRUCTURE ONLY (see the package docstring): the product path never
imports this module.

What the pages fix.  The nano-vllm architecture page, "Hash-basiertes Prefix
Caching" and "Kern-Designentscheidungen" item 2: sequences whose prompts
begin with the same full blocks of tokens are given the SAME physical blocks
(a chained hash per full block finds the cached block), so equal leading
entries of two block tables mean equal K/V rows.  A decode step may therefore
attend over such a shared run once for all the sequences that hold it and
merge the result with each sequence's private remainder (the split-K merge of
the decode kernel); the output is the same attention.

What is this library's own choice (the pages describe no such plan), written
out here step by step:

1. S is the decode split length (keys per split).  Only whole splits are
   shared: split s covers keys s*S .. (s+1)*S - 1.
2. A sequence b is eligible when ctx[b] - 1 >= S (at least one whole split
   lies before its last position ctx[b] - 1, the row the decode step stores).
3. Eligible sequences are put in classes by their first block id; classes are
   taken in the order of their first member in the batch.  A class with one
   member shares nothing.
4. Within a class the members are ordered by their table row over the blocks
   that hold keys 0 .. ctx[b] - 2 (ceil((ctx[b] - 1) / B) entries), compared
   lexicographically (a row that is a prefix of another comes first), ties
   by batch index; so sequences sharing longer runs sit next to each other.
5. The ordered class is cut into runs of R = 16 // G consecutive members
   (G = num_q_heads / num_kv_heads: one run's query heads of one kv head fill
   at most 16 columns); a run of one member is dropped.
6. For a run: lcp = the number of leading table entries (within each member's
   entries of step 4) that all members have in common, T = min(lcp * B,
   min over members of ctx[b] - 1), k = T // S.  If k >= 1 the run becomes
   subgroup p (the next index) with items (p, 0) .. (p, k - 1), and skip[b] = k
   for each member (those splits are computed by the subgroup).

Plan words (int32), in this order:
  S, number of items, batch, G, number of subgroups P;
  skip[0 .. batch - 1];
  per subgroup: member count, then 16 member ids (unused: -1);
  per item: subgroup index, split index.
"""

from __future__ import annotations

from typing import List, Sequence

MEMBER_SLOTS = 16  # query columns of one subgroup's tile
HEADER_WORDS = 5


def plan_words_bound(batch: int, max_context_len: int, split_tokens: int) -> int:
    """Largest plan (in int32 words) the rule can produce for these sizes:
    at most batch // 2 subgroups, each with at most (max_ctx - 1) // S items."""
    p = batch // 2
    k = max(max_context_len - 1, 0) // split_tokens
    return HEADER_WORDS + batch + (1 + MEMBER_SLOTS) * p + 2 * p * k


def needed_blocks(ctx: int, block_size: int) -> int:
    """Blocks holding keys 0 .. ctx - 2, the keys before the last position
    (step 4)."""
    return -(-(ctx - 1) // block_size) if ctx > 1 else 0


def common_prefix(rows: Sequence[Sequence[int]]) -> int:
    """Number of leading entries all rows have in common (step 6)."""
    lcp = 0
    while all(lcp < len(r) for r in rows) and all(r[lcp] == rows[0][lcp] for r in rows):
        lcp += 1
    return lcp


def shared_splits(lcp: int, block_size: int, ctxs: Sequence[int], split_tokens: int) -> int:
    """k of step 6: whole splits inside the common blocks and before every
    member's last position."""
    T = min(lcp * block_size, min(c - 1 for c in ctxs))
    return T // split_tokens


def prefix_plan(block_tables: Sequence[Sequence[int]], context_lens: Sequence[int],
                block_size: int, group: int, split_tokens: int) -> List[int]:
    """The plan words for one decode batch (steps 1-6 of the module docstring).

    block_tables: per sequence, its table row (python ints; entries past the
    blocks it uses are not read); context_lens: keys per sequence (including
    the token stored this step); group: query heads per kv head;
    split_tokens: S > 0."""
    batch = len(context_lens)
    S = split_tokens
    B = block_size
    R = MEMBER_SLOTS // group
    skip = [0] * batch
    subgroups: List[List[int]] = []
    items: List[List[int]] = []

    def row(b):
        return tuple(int(x) for x in block_tables[b][:needed_blocks(context_lens[b], B)])

    if R >= 2:
        classes = {}  # first block id -> members, in batch order
        order = []
        for b in range(batch):
            if context_lens[b] - 1 < S:
                continue
            first = int(block_tables[b][0])
            if first not in classes:
                classes[first] = []
                order.append(first)
            classes[first].append(b)
        for first in order:
            members = classes[first]
            if len(members) < 2:
                continue
            members = sorted(members, key=lambda b: (row(b), b))
            for i in range(0, len(members), R):
                run = members[i:i + R]
                if len(run) < 2:
                    continue
                k = shared_splits(common_prefix([row(b) for b in run]), B,
                                  [context_lens[b] for b in run], S)
                if k < 1:
                    continue
                p = len(subgroups)
                subgroups.append(run)
                for b in run:
                    skip[b] = k
                items.extend([p, s] for s in range(k))
    words = [S, len(items), batch, group, len(subgroups)]
    words += skip
    for run in subgroups:
        words += [len(run)] + run + [-1] * (MEMBER_SLOTS - len(run))
    for it in items:
        words += it
    return words


def decode_plan(words: Sequence[int]):
    """The plan's parts: (S, batch, skip, subgroups, items)."""
    S, n_items, batch, _group, n_sub = words[:HEADER_WORDS]
    o = HEADER_WORDS
    skip = list(words[o:o + batch])
    o += batch
    subgroups = []
    for _ in range(n_sub):
        cnt = words[o]
        subgroups.append(list(words[o + 1:o + 1 + cnt]))
        o += 1 + MEMBER_SLOTS
    items = [(words[o + 2 * i], words[o + 2 * i + 1]) for i in range(n_items)]
    assert o + 2 * n_items == len(words)
    return S, batch, skip, subgroups, items
