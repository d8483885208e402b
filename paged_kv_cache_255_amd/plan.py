"""Runs a list of pool operations through the library's block pool.

A plan is a list of tuples: ("create",), ("fork", parent), ("free", seq),
("prefill", seq, ntokens) -- sequences named by their position in creation
order.  Returns the library's id for each plan sequence and the slots of all
prefill tokens in plan order (the slot_mapping for one cache-append call).
"""
import numpy as np

from . import (pa_seq_append_slots, pa_seq_create, pa_seq_fork, pa_seq_free)


def execute_plan(pool, ops):
    ids = []
    slots = []
    for op in ops:
        if op[0] == "create":
            ids.append(pa_seq_create(pool))
        elif op[0] == "fork":
            ids.append(pa_seq_fork(pool, ids[op[1]]))
        elif op[0] == "free":
            pa_seq_free(pool, ids[op[1]])
        elif op[0] == "prefill":
            slots.append(pa_seq_append_slots(pool, ids[op[1]], op[2]))
        else:
            raise ValueError(op)
    flat = np.concatenate(slots) if slots else np.zeros(0, np.int32)
    return ids, flat.astype(np.int32)
