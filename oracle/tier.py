"""Capacity-limited hot tier of expert records -- TEST INFRASTRUCTURE ONLY.

Plain Python over small integer and float arrays; shares no code with the HIP
library.  What it follows:
  * "为什么 Strata 在小显存显卡上这么快", section "一台电脑就是一组水管": the
    engine ships a usage profile that ranks all 24,576 experts; every card
    fills its expert slots in that order; an adaptive tier then swaps in at
    most 96 experts every four rounds, moving the cached set towards the
    experts the conversation actually uses.
  * "Strata：12GB 显卡跑 125B 模型，MoE 专家热缓存打破 VRAM 限制", section
    "工作原理": what gets evicted is decided by an exponentially decayed usage
    score (the scores of usage_update).
Readings where the pages are silent:
  * the pool holds n_hot hot slots plus every expert's record at its home
    slot; an expert is resident when one hot slot holds a copy of its record,
    and the slot table then points at that copy, else at its home record;
  * ranking is by (score descending, flat index l*E+e ascending), the order
    usage_update's re-rank returns;
  * fill: the n_hot first experts of that ranking become resident, hot slot i
    holding the i-th of them in flat-index order;
  * rebalance: the experts that are not resident, in rank order, are the
    candidates; the hot slots are the victims, empty slots first (lower slot
    first), then by the held expert's score ascending, ties to the higher flat
    index; candidate i replaces victim i while the slot is empty or the
    candidate's score is strictly higher (equal scores never swap), at most
    max_swaps times (96 on the pages);
  * the shared expert (column E of the slot table) is never part of the tier.
"""
import numpy as np

__all__ = ["tier_fill", "tier_rebalance", "tier_rank"]


def tier_rank(scores):
    """Flat indices of all experts in rank order (score desc, index asc)."""
    flat = np.asarray(scores, dtype=np.float64).reshape(-1)
    return [int(i) for i in np.lexsort((np.arange(flat.size), -flat))]


def _home_slot(home, E, f):
    return int(home[f // E][f % E])


def tier_fill(scores, n_hot, home):
    """Returns (slot_table [L][E+1], owner [n_hot], swaps) for an empty tier
    filled from the profile `scores` [L][E].  swaps: (expert, -1, hot slot,
    home slot) per copied record, in hot-slot order."""
    s = np.asarray(scores)
    L, E = s.shape
    assert 0 <= n_hot <= L * E
    chosen = sorted(tier_rank(s)[:n_hot])
    slot = np.array(home, dtype=np.int32, copy=True)
    owner = np.full(n_hot, -1, dtype=np.int32)
    swaps = []
    for i, f in enumerate(chosen):
        slot[f // E][f % E] = i
        owner[i] = f
        swaps.append((f, -1, i, _home_slot(home, E, f)))
    return slot, owner, swaps


def tier_rebalance(scores, n_hot, max_swaps, home, slot_table, owner):
    """One adaptive step.  Returns (slot_table, owner, swaps); swaps:
    (expert swapped in, expert evicted or -1, hot slot, the new expert's home
    slot), in candidate order."""
    s = np.asarray(scores, dtype=np.float32)
    L, E = s.shape
    flat = s.reshape(-1)
    slot = np.array(slot_table, dtype=np.int32, copy=True)
    own = np.array(owner, dtype=np.int32, copy=True)
    resident = set(int(f) for f in own if f >= 0)
    candidates = [f for f in tier_rank(s) if f not in resident]

    def victim_order(i):
        f = int(own[i])
        if f < 0:
            return (0, 0.0, 0, i)              # empty slots first, lower slot first
        return (1, float(flat[f]), -f, i)      # then score ascending, higher index first

    victims = sorted(range(n_hot), key=victim_order)
    swaps = []
    for c, v in zip(candidates, victims):
        if len(swaps) >= max_swaps:
            break
        old = int(own[v])
        if old >= 0 and not float(flat[c]) > float(flat[old]):
            break
        if old >= 0:
            slot[old // E][old % E] = _home_slot(home, E, old)
        slot[c // E][c % E] = v
        own[v] = c
        swaps.append((c, old, v, _home_slot(home, E, c)))
    return slot, own, swaps
