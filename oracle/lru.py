"""The global LRU expert-slot table as a deterministic state machine (test
infrastructure).

The pages keep the whole expert pool in host memory and use free device
memory as one least-recently-used expert cache shared by all MoE layers
(FreeToken explainer page, "how" section); LRU evicts, at capacity, the
entry unreferenced for longest (same page, glossary).  A call looks up the
experts one layer selected for a batch of tokens; the rule for several keys
in one call is this reading:

  key = (layer, expert); S slots; state: key_slot[L][E] (-1 = absent),
  slot_key[S] (-1 = free), last_use[S] (0 = never), tick.
  One call with ids (any order, repeats allowed):
    U = the distinct ids, ascending; hits = those already resident.
    If the misses outnumber the S - |hits| slots not touched by this call,
    report exhaustion and change nothing (not even the tick).
    tick += 1; every hit gets last_use = tick.
    The i-th miss (ascending expert id) takes the i-th slot of the order
    (last_use ascending, slot ascending) among slots with last_use < tick;
    the key it held (if any) is evicted; the slot is stamped with tick.
    The call returns slot_ids per input id, a miss flag per input id (set on
    every occurrence of a missed id), and the (expert, slot) list of misses.
With one key per call this is textbook LRU with free slots taken lowest first.
"""
import numpy as np


class LruSim:
    def __init__(self, n_layers: int, n_experts: int, n_slots: int):
        self.L, self.E, self.S = n_layers, n_experts, n_slots
        self.key_slot = np.full((n_layers, n_experts), -1, dtype=np.int32)
        self.slot_key = np.full(n_slots, -1, dtype=np.int32)
        self.last_use = np.zeros(n_slots, dtype=np.int64)
        self.tick = 0

    def lookup(self, layer: int, ids):
        ids = np.asarray(ids, dtype=np.int64).ravel()
        U = sorted(set(int(e) for e in ids))
        hits = [e for e in U if self.key_slot[layer, e] >= 0]
        misses = [e for e in U if self.key_slot[layer, e] < 0]
        if len(misses) > self.S - len(hits):
            return None  # exhaustion: no state change
        self.tick += 1
        tau = self.tick
        for e in hits:
            self.last_use[self.key_slot[layer, e]] = tau
        miss_list = []
        if misses:
            # order (last_use asc, slot asc) over slots not stamped by this call,
            # as one integer key last_use * S + slot
            key = self.last_use * self.S + np.arange(self.S, dtype=np.int64)
            key = np.where(self.last_use < tau, key, np.iinfo(np.int64).max)
            victims = np.argsort(key, kind="stable")[: len(misses)]
        for i, e in enumerate(misses):
            s = int(victims[i])
            old = int(self.slot_key[s])
            if old >= 0:
                self.key_slot[old // self.E, old % self.E] = -1
            self.slot_key[s] = layer * self.E + e
            self.key_slot[layer, e] = s
            self.last_use[s] = tau
            miss_list.append((e, s))
        missed = set(misses)
        slot_ids = np.array([self.key_slot[layer, int(e)] for e in ids], dtype=np.int32)
        miss_flags = np.array([1 if int(e) in missed else 0 for e in ids], dtype=np.uint8)
        return slot_ids, miss_flags, miss_list

    def snapshot(self):
        return (self.key_slot.copy(), self.slot_key.copy(), self.last_use.copy(), self.tick)

    def restore(self, snap):
        ks, sk, lu, tick = snap
        self.key_slot, self.slot_key, self.last_use, self.tick = ks.copy(), sk.copy(), lu.copy(), tick
