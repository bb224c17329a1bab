"""Ring-buffer pointer state machine of the replay state -- TEST INFRASTRUCTURE ONLY.

Model of what the pages describe: the state is a checkpoint plus a buffer of recent inputs
(deskofai.com, "ReplaySSM: Rethinking State Storage for Faster Hybrid-Model Decoding", para 2);
the buffer is folded into the checkpoint when it fills, and speculative drafts are appended and
rejected by moving a pointer, with no per-token state snapshot (same page, para 3).

Per sequence: the ring has `cap` slots; `start` is the slot of the oldest buffered entry, `count`
the number of committed entries after the checkpoint, `pending` the drafts appended after them.
  decode       append one entry at slot (start + count) % cap and commit it (count += 1)
  spec_append  write S drafts at slots (start + count + j) % cap, j < S; pending = S
  rollback(a)  commit the first a drafts: count += a, pending = 0 (rejected drafts stay in their
               slots as garbage and are overwritten later)
  flush_if_full  if count >= L: fold the oldest L committed entries, start += L, count -= L
  flush_all    fold every committed entry: start += count, count = 0
The checkpoint position (tokens folded so far) advances by the folded count.
Readings (the pages fix no policy): drafts are never folded; a flush folds exactly L entries
when the committed count has reached L.
"""
from __future__ import annotations

import dataclasses
from typing import List, Tuple


@dataclasses.dataclass
class Ring:
    cap: int
    L: int
    start: int = 0
    count: int = 0
    pending: int = 0
    position: int = 0          # tokens folded into the checkpoint
    committed: int = 0         # tokens committed in total (position + count)
    flushes: List[Tuple[int, int]] = dataclasses.field(default_factory=list)  # (pos_before, n)

    def slots(self) -> List[int]:
        """Slots of the committed entries, oldest first."""
        return [(self.start + i) % self.cap for i in range(self.count)]

    def decode(self) -> int:
        if self.pending:
            raise RuntimeError("decode while drafts are pending")
        if self.count + 1 > self.cap:
            raise RuntimeError("ring full")
        slot = (self.start + self.count) % self.cap
        self.count += 1
        self.committed += 1
        return slot

    def spec_append(self, S: int) -> List[int]:
        if self.pending:
            raise RuntimeError("drafts already pending")
        if self.count + S > self.cap:
            raise RuntimeError("ring full")
        self.pending = S
        return [(self.start + self.count + j) % self.cap for j in range(S)]

    def rollback(self, accepted: int) -> None:
        if not 0 <= accepted <= self.pending:
            raise RuntimeError("accepted count out of range")
        self.count += accepted
        self.committed += accepted
        self.pending = 0

    def _fold(self, n: int) -> None:
        self.flushes.append((self.position, n))
        self.start = (self.start + n) % self.cap
        self.count -= n
        self.position += n

    def flush_if_full(self) -> bool:
        if self.pending:
            raise RuntimeError("flush while drafts are pending")
        if self.count >= self.L:
            self._fold(self.L)
            return True
        return False

    def flush_all(self) -> None:
        if self.pending:
            raise RuntimeError("flush while drafts are pending")
        if self.count:
            self._fold(self.count)
