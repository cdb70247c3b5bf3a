"""Oracle for ring-KV slot/position arithmetic (integers only).

TEST INFRASTRUCTURE ONLY -- see the package docstring.

Source: "PersonaPlex native LM audit" (Clockless Inkling), section 6 "Three distinct
caches": a ring of `capacity` slots receives absolute position p in slot p mod capacity;
the declared temporal mask admits keys with 0 <= query - key < context.

Two labellings are provided:
  * stated_positions: each slot carries the latest absolute position written to it --
    the reading the library implements (all `capacity` slots usable once the ring is full);
  * compat_positions: the mapping the audit reproduced from the released ring cache,
    where slots are labelled relative to the write cursor and the slot under the cursor
    is labelled with the (future) end offset. The audit's integer examples pin it.
"""


def slot_of(pos, capacity):
    return pos % capacity


def stated_positions(capacity, end_offset):
    """Absolute position held by each slot after positions 0 .. end_offset-1 were written
    (None for a slot never written)."""
    out = []
    for s in range(capacity):
        if s >= end_offset:
            out.append(None)
        else:
            # latest p < end_offset with p mod capacity == s
            out.append(s + ((end_offset - 1 - s) // capacity) * capacity)
    return out


def compat_positions(capacity, end_offset):
    """Labels from cursor-relative arithmetic: with cursor = end_offset mod capacity and
    delta = slot - cursor, a slot gets end_offset + delta when delta <= 0 and
    end_offset + delta - capacity otherwise (a full ring is assumed)."""
    cursor = end_offset % capacity
    out = []
    for s in range(capacity):
        delta = s - cursor
        out.append(end_offset + delta if delta <= 0 else end_offset + delta - capacity)
    return out


def visible(labels, query, context):
    """Labels admitted for `query` by the declared mask 0 <= query - label < context."""
    return [p for p in labels if p is not None and 0 <= query - p < context]
