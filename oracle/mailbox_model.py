"""Host model of the three-generation Lamport mailbox and its stage state.

TEST INFRASTRUCTURE, NOT THE PRODUCT (see ``oracle/__init__.py``).

Follows the publish / consume protocol of the pages:
  vllm.models.glm5next.nvidia.specialized_decode.all_reduce_mhc,
    AllReduceMhcBoundary.__init__ (every slot starts as BF16 negative zero,
    stage state zeroed), _PublishDeviceKernel.kernel (read NEXT, store the
    sanitized fragment into generation NEXT, then ACTIVE = NEXT);
  vllm.models.deepseek_v41.nvidia.ops.cute_dsl.all_reduce_mhc,
    _LamportMHCDeviceKernel.kernel (read ACTIVE, wait until no fragment holds
    the sentinel, NEXT = (ACTIVE + 1) % 3, reset the consumed slots).
The GPU's mailbox bytes and stage words are compared with this model after
every call.
"""
from __future__ import annotations

import numpy as np

SENTINEL = 0x8000
GENERATIONS = 3
ACTIVE, NEXT = 0, 1


class MailboxModel:
    """slots [3, tp, capacity, H] BF16 bits; stage [ACTIVE, NEXT] int32."""

    def __init__(self, tp: int, capacity: int, hidden: int):
        self.tp, self.capacity, self.hidden = tp, capacity, hidden
        self.slots = np.full((GENERATIONS, tp, capacity, hidden), SENTINEL, np.uint16)
        self.stage = np.zeros(2, np.int32)

    def publish(self, partials: np.ndarray) -> None:
        """All tp ranks publish their [M, H] partials (stacked [tp, M, H])."""
        partials = np.asarray(partials, np.uint16)
        m = partials.shape[1]
        g = int(self.stage[NEXT])
        self.slots[g, :, :m] = np.where(partials == SENTINEL, 0, partials)
        self.stage[ACTIVE] = g

    def consume(self, m: int) -> np.ndarray:
        """The consumer of M tokens: returns the [tp, M, H] values it reads and
        resets them to the sentinel.  A slot still holding the sentinel would
        keep the consumer waiting: the model raises instead."""
        g = int(self.stage[ACTIVE])
        data = self.slots[g, :, :m].copy()
        if (data == SENTINEL).any():
            raise RuntimeError("consumer would wait: a slot still holds the sentinel")
        self.stage[NEXT] = (g + 1) % GENERATIONS
        self.slots[g, :, :m] = SENTINEL
        return data
