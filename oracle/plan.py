"""Split-KV work plan of the decode scheduler, in plain Python loops.

Test infrastructure only.  The pages ask for a scheduler that splits long or
variable-length sequences across compute units and merges the split partials
with a log-sum-exp reduction ([MLA-FA3 article], "online softmax scaling and
partial reduction" stage of the fused dataflow figure).  They do not fix the
plan, so this is the library's own definition, restated here independently
of the device planner so that the device's plan can be compared bit for bit.

Definition (all quantities integers):
  n_b      = ceil(len_b / tile)                      tiles of sequence b
  mode "whole" (num_splits == 1): one part per sequence,
           t = max_b n_b + c0 (at least 1), start_b = b*t + c0.
  mode "line"  (num_splits >= 2): sequences laid end to end on a cost line,
           cost_b = n_b + c0 if n_b > 0 else 0   (c0 = fixed cost of
           loading a query block and writing its output, in tile units),
           A_b = sum_{b' < b} cost_b',  start_b = A_b + c0,  C = sum_b cost_b,
           t = max(ceil(C / parts), ceil(max_n / (num_splits - 1)), t_min, 1).
  Part p owns cost-line positions [p*t, (p+1)*t); tile k of sequence b sits
  at position start_b + k.  Hence
    first_b  = floor(start_b / t),  last_b = floor((start_b + n_b - 1) / t),
    nsplit_b = last_b - first_b + 1  (0 when n_b = 0)   <= num_splits,
    part_first_seq[p] = smallest b with n_b > 0 and first_b <= p <= last_b
                        (B when part p holds no tile),
    parts_used = ceil(C / t) in line mode, B in whole mode.
  A split sequence is always the first or the last piece of a part, so its
  partial result for part p goes to slot 2p (first piece) or 2p+1.

Pinned by (tests/test_oracle_plan.py): exact-cover of every tile, the
per-sequence split bound, the balance bound, and brute-force enumeration of
the cost line on small cases.
"""

__all__ = ["plan_ref", "plan_pieces_ref", "plan_slot_ref"]


def _cdiv(a, b):
    return -(-a // b)


def plan_ref(seqlens, tile, parts, num_splits, c0, t_min):
    """Return the plan as a dict of plain ints and lists (see module doc)."""
    seqlens = [int(x) for x in seqlens]
    B = len(seqlens)
    n = [_cdiv(L, tile) for L in seqlens]
    max_n = max(n) if n else 0
    start = [0] * B
    if num_splits == 1:
        mode = "whole"
        t = max(max_n + c0, 1)
        for b in range(B):
            start[b] = b * t + c0
        C = B * t
        parts_used = B
    else:
        mode = "line"
        A = 0
        for b in range(B):
            start[b] = A + c0
            A += (n[b] + c0) if n[b] > 0 else 0
        C = A
        t = max(_cdiv(C, parts) if parts > 0 else 0, _cdiv(max_n, num_splits - 1), t_min, 1)
        parts_used = _cdiv(C, t)
    first = [0] * B
    nsplit = [0] * B
    for b in range(B):
        if n[b] > 0:
            first[b] = start[b] // t
            nsplit[b] = (start[b] + n[b] - 1) // t - first[b] + 1
    n_parts = B if mode == "whole" else parts
    part_first_seq = [B] * n_parts
    for b in range(B - 1, -1, -1):
        for p in range(first[b], first[b] + nsplit[b]):
            part_first_seq[p] = b
    return {
        "mode": mode, "tile": tile, "t": t, "C": C, "c0": c0, "parts": n_parts,
        "parts_used": parts_used, "max_n": max_n, "n": n, "start": start,
        "first": first, "nsplit": nsplit, "part_first_seq": part_first_seq,
    }


def plan_pieces_ref(plan, p):
    """Pieces of part p as (b, tile_lo, tile_hi) with tiles relative to b."""
    t = plan["t"]
    B = len(plan["n"])
    out = []
    b = plan["part_first_seq"][p]
    lo_pos, hi_pos = p * t, (p + 1) * t
    while b < B:
        nb, sb = plan["n"][b], plan["start"][b]
        if nb > 0:
            if sb >= hi_pos:
                break
            lo, hi = max(sb, lo_pos), min(sb + nb, hi_pos)
            if lo < hi:
                out.append((b, lo - sb, hi - sb))
        if plan["mode"] == "whole":
            break
        b += 1
    return out


def plan_slot_ref(plan, p, b):
    """Partial-result slot of sequence b's piece in part p (split pieces only)."""
    return 2 * p + (0 if plan["part_first_seq"][p] == b else 1)
