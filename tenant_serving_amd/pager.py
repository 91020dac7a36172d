"""Residency of users' deltas: a pool of device slots for one module (a list of
matrices, e.g. one layer's projections), fed from a store of every user's packed module
in pinned host memory, the least recently used slot given up when a request needs room
([P2] "Systems Mechanics" 3: deltas cached in spare GPU memory or streamed from host
memory per request; [P1] "Production Serving": the base model stays on the GPU and
the deltas in host memory; [P5] "Key Contributions" 4: a module's packed delta moves
in one transfer).

A slot holds one user's module in the layout of banks.module_layout, so filling it is
one host-to-device copy; the banks of matrix j are then strided through the pool
(slot k's signs at pool + k * slot_bytes + signs offset of j) and bd_apply_paged reads
them through a device table user -> slot.  Copies and table updates are enqueued on
the caller's stream, in order with the applies: a slot is overwritten only after the
applies enqueued before it on that stream."""
from collections import OrderedDict
from typing import Dict, Iterable, List, Optional, Sequence, Tuple

import numpy as np
import torch

from . import banks
from . import bitdelta as B


class SlotLRU:
    """The slot bookkeeping of a pager: which user holds which of n_slots slots, least
    recently used first.  ensure(users) makes every listed user resident and returns
    the (user, slot) loads it needs and the users it evicted for them; a user listed in
    the request is never evicted by it."""

    def __init__(self, n_slots: int):
        if n_slots < 1:
            raise ValueError("a pager needs at least one slot")
        self.n_slots = n_slots
        self.slot: "OrderedDict[int, int]" = OrderedDict()  # user -> slot, oldest first
        self.free: List[int] = list(range(n_slots - 1, -1, -1))

    def resident(self, user: int) -> bool:
        return user in self.slot

    def ensure(self, users: Iterable[int]) -> Tuple[List[Tuple[int, int]], List[int]]:
        want = list(dict.fromkeys(int(u) for u in users if int(u) >= 0))
        if len(want) > self.n_slots:
            raise ValueError(f"a request for {len(want)} users does not fit {self.n_slots} slots")
        for u in want:
            if u in self.slot:
                self.slot.move_to_end(u)
        wanted = set(want)
        loads, evicted = [], []
        for u in want:
            if u in self.slot:
                continue
            if self.free:
                k = self.free.pop()
            else:
                victim = next(v for v in self.slot if v not in wanted)
                k = self.slot.pop(victim)
                evicted.append(victim)
            self.slot[u] = k
            loads.append((u, k))
        return loads, evicted

    def drop(self, user: int) -> None:
        k = self.slot.pop(user, None)
        if k is not None:
            self.free.append(k)


class BankPager:
    """n_slots device slots of one module for n_users users.

    shapes: (d_out, d_in) of each matrix of the module; scale_counts: scales per user of
    each (bd_scales_count); scale_dtype: torch.float32 or torch.float16 for all of
    them.  Users enter the host store with pack() (or put() of an already packed
    module); ensure() makes a request's users resident; apply() runs bd_apply_paged on
    one matrix."""

    def __init__(self, shapes: Sequence[Tuple[int, int]], scale_counts: Sequence[int],
                 scale_dtype, n_slots: int, n_users: int, device):
        self.shapes = [tuple(s) for s in shapes]
        self.scale_counts = list(scale_counts)
        self.scale_dtype = scale_dtype
        esz = torch.tensor([], dtype=scale_dtype).element_size()
        self.offs, self.slot_bytes = banks.module_layout(self.shapes, self.scale_counts, esz)
        self.n_slots, self.n_users = n_slots, n_users
        self.device = torch.device(device)
        self.pool = torch.empty(n_slots * self.slot_bytes, dtype=torch.uint8, device=self.device)
        self.table = torch.full((n_users,), -1, dtype=torch.int32, device=self.device)
        self.lru = SlotLRU(n_slots)
        self.store: Dict[int, torch.Tensor] = {}
        # two pinned mirrors of the table, used in turn: a mirror is rewritten only after
        # its previous copy to the device has completed
        self._mirror = [torch.full((n_users,), -1, dtype=torch.int32).pin_memory() for _ in range(2)]
        self._mirror_ev: List[Optional[torch.cuda.Event]] = [None, None]
        self._turn = 0
        self._host_table = np.full(n_users, -1, dtype=np.int32)
        self.loads = 0
        self.bytes_loaded = 0

    # ---------------------------------------------------------------- host store
    def put(self, user: int, module: torch.Tensor) -> None:
        """Stores a packed module (uint8[slot_bytes], any device) for `user`, in pinned
        host memory; a resident copy of an older module is dropped."""
        if not 0 <= user < self.n_users:
            raise ValueError(f"user {user} outside [0, {self.n_users})")
        if module.dtype != torch.uint8 or module.numel() != self.slot_bytes:
            raise ValueError(f"a module is uint8[{self.slot_bytes}]")
        buf = self.store.get(user)
        if buf is None:
            buf = torch.empty(self.slot_bytes, dtype=torch.uint8, pin_memory=True)
            self.store[user] = buf
        buf.copy_(module)
        if self.lru.resident(user):
            self.lru.drop(user)
            self._host_table[user] = -1
            self._push_table(torch.cuda.current_stream(self.device))

    def pack(self, user: int, signs_list, scales_list) -> None:
        """Packs one user's banks of every matrix (signs int64[d_out][d_in/64] and
        scales, any device) into the host store."""
        buf = torch.zeros(self.slot_bytes, dtype=torch.uint8, device=signs_list[0].device)
        banks.pack_module(buf, self.shapes, signs_list, scales_list)
        self.put(user, buf)

    # ---------------------------------------------------------------- residency
    def _push_table(self, stream) -> None:
        i = self._turn
        self._turn ^= 1
        if self._mirror_ev[i] is not None:
            self._mirror_ev[i].synchronize()
        self._mirror[i].copy_(torch.from_numpy(self._host_table))
        with torch.cuda.stream(stream):
            self.table.copy_(self._mirror[i], non_blocking=True)
            ev = torch.cuda.Event()
            ev.record(stream)
        self._mirror_ev[i] = ev

    def ensure(self, users, stream=None) -> int:
        """Makes every user in `users` (ids; -1 entries ignored) resident, evicting the
        least recently used others; one host-to-device copy per missing user's module.
        Returns the number of modules loaded."""
        ids = users.tolist() if isinstance(users, (torch.Tensor, np.ndarray)) else list(users)
        want = [int(u) for u in ids if int(u) >= 0]
        for u in set(want):
            if u >= self.n_users or u not in self.store:
                raise KeyError(f"user {u} has no module in the host store")
        loads, evicted = self.lru.ensure(want)
        if not loads:
            return 0
        st = stream if stream is not None else torch.cuda.current_stream(self.device)
        for v in evicted:
            self._host_table[v] = -1
        with torch.cuda.stream(st):
            for u, k in loads:
                self.pool[k * self.slot_bytes:(k + 1) * self.slot_bytes].copy_(
                    self.store[u], non_blocking=True)
                self._host_table[u] = k
        self._push_table(st)
        self.loads += len(loads)
        self.bytes_loaded += len(loads) * self.slot_bytes
        return len(loads)

    def slot_of(self, user: int) -> int:
        return int(self._host_table[user])

    # ---------------------------------------------------------------- apply
    def views(self, j: int) -> Tuple[torch.Tensor, torch.Tensor]:
        """uint8 views of the pool from slot 0's signs and scales of matrix j."""
        s_off, c_off = self.offs[j]
        return self.pool[s_off:], self.pool[c_off:]

    def apply(self, j: int, x: torch.Tensor, w_base: torch.Tensor, p, user_ids: torch.Tensor,
              y: Optional[torch.Tensor] = None, y_dtype=torch.float32, ws=None, stream=None,
              check: bool = False) -> torch.Tensor:
        """y = x w_base^T + each token's user's delta of matrix j, read from its slot."""
        T, d_in = x.shape
        d_out = w_base.shape[0]
        if (d_out, d_in) != self.shapes[j]:
            raise ValueError(f"matrix {j} is {self.shapes[j]}, got ({d_out}, {d_in})")
        if y is None:
            y = torch.empty((T, d_out), dtype=y_dtype, device=x.device)
        if ws is None:
            ws = B.workspace(B.bd_apply_paged_workspace_bytes(
                p, T, self.n_slots, d_out, d_in, B._dtype_code(x), B._dtype_code(y)), x.device)
        sv, cv = self.views(j)
        B._check(B.bd_apply_paged(x, w_base, sv, cv, self.slot_bytes, self.slot_bytes,
                                  self.n_slots, p, self.table, user_ids, y, ws, stream),
                 "bd_apply_paged")
        if check:
            B._check(B.bd_device_status(ws, stream), "bd_apply_paged (device)")
        return y
