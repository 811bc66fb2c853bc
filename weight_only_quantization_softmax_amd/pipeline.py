"""EWQ tier dispatch over the five entry points (host orchestration only).

[EWQ] "Giai ma EWQ & FastEWQ" (2kvn.com), section "EWQ hoat dong nhu the
nao?", step 2: the lowest-entropy blocks (H <= T) are quantised
aggressively, the middle ones (T < H < mu) moderately, the rest are kept.
What each tier does is a parameter of the pass:

  "sinq"     SINQ Sinkhorn balancing, then group RTN at (bits, group)
  "int8row"  8-bit RTN with one group per row, no balancing
  "ternary"  ternary {-1, 0, +1} with a per-row scale
  "keep"     left as is (optionally stored with the lossless exponent code of
             [DF11] "DFloat11: Nen suy luan GPU khong mat du lieu ..."
             (vi.news.hada.io) by :meth:`QuantPass.compress_kept`)

With a storage budget, the tiers' choices are then moved along the ladder
ACTIONS (ascending storage: ternary < Sinkhorn + low-bit < int8 per row <
kept) by EWQ's budgeted placement (same page, step 3): spare room promotes
the highest-entropy quantised blocks, a shortfall demotes the lowest-entropy
ones (ewq_budget_levels, host-side in the library).

A :class:`QuantPass` is prepared once for a fixed set of device-resident
matrices: every output buffer and workspace is allocated up front (per tier
assignment), so :meth:`QuantPass.run` only launches library calls and reads
the tiers back (the one host synchronisation of the pass).
"""
from __future__ import annotations

import ctypes
from typing import Dict, List, Optional, Sequence

import torch

from . import _lib
from . import _check_mats, _device

ACTIONS = ("ternary", "sinq", "int8row", "keep")   # ascending storage per weight


def _mat_arr(ts):
    return _lib.mat_array((t.data_ptr(), _lib.WOQ_BF16 if t.dtype == torch.bfloat16 else _lib.WOQ_F32,
                           t.shape[0], t.shape[1]) for t in ts)


def _ws(op, mats, group, dev):
    lib = _lib.load()
    out = ctypes.c_size_t(0)
    _lib.check("woq_workspace_size", lib.woq_workspace_size(op, _mat_arr(mats), len(mats), group,
                                                             ctypes.byref(out)))
    return torch.empty(max(out.value, 256), dtype=torch.uint8, device=dev)


class _Call:
    """One prepared library call: name, bound ctypes arguments, kept-alive objects."""

    def __init__(self, name: str, fn, args, keep, kind: str, nbytes: int):
        self.name, self.fn, self.args, self.keep, self.kind, self.nbytes = name, fn, args, keep, kind, nbytes

    def __call__(self, stream_handle, stream=None):
        _lib.check(self.name, self.fn(*self.args, stream_handle))


def _wave_form(m: torch.Tensor) -> bool:
    """Rows the library's Sinkhorn sweep holds in one wave (at most 4096 bf16
    or 1536 fp32 columns); wider rows take a workgroup per row strip."""
    return m.shape[1] <= (4096 if m.dtype == torch.bfloat16 else 1536)


class _SplitSinq:
    """The Sinkhorn step of one tier as two concurrent sinq_balance calls on
    two streams (the second at default priority), so that their kernels
    share the GPU instead of running one after the other.  The split (chosen
    by :meth:`QuantPass._sinq_split`, measured on the stacks' shapes):

    - wave-form and wider matrices: the wider ones carry WOQ_SINQ_SHARED
      and are planned for half of the GPU, so every CU holds a barrier-bound
      workgroup of the wide rows beside a bandwidth-bound one of the narrow
      rows (8B stack's low tier: 10.9 ms one after the other, 10.4-10.7 ms
      side by side);
    - otherwise several row widths: the width with the most bytes in one
      call, the others in the other, neither flagged (their reductions and
      tails overlap: MoE layers 70.3 -> 67.3 ms, 70B blocks 103.5 -> 102.3).

    The first call, the longer one, runs on the caller's stream and is
    enqueued first; the second stream starts after, and the caller's stream
    continues after, everything the other holds."""

    kind = "sinq"

    def __init__(self, first: _Call, second: _Call, side: torch.cuda.Stream):
        self.first, self.second, self.side = first, second, side
        self.nbytes = first.nbytes + second.nbytes
        self.name = "sinq_balance x2"
        self._fork = torch.cuda.Event()
        self._join = torch.cuda.Event()

    def __call__(self, stream_handle, stream=None):
        if stream is None:
            raise ValueError("the split Sinkhorn call needs the caller's torch stream")
        self._fork.record(stream)
        self.first(stream_handle)
        self.side.wait_event(self._fork)
        self.second(self.side.cuda_stream)
        self._join.record(self.side)
        stream.wait_event(self._join)


class QuantPass:
    def __init__(self, mats: Sequence[torch.Tensor], block_id: Sequence[int], n_blocks: int, *,
                 iters: int, bits: int, group: int, x: float = 1.0, tiered: bool = True,
                 actions: Sequence[str] = ("sinq", "int8row", "keep"),
                 sinq_batch_bytes: int = 0, budget_bytes: Optional[int] = None):
        for a in actions:
            if a not in ACTIONS:
                raise ValueError(a)
        self.lib = _lib.load()
        self.mats = list(mats)
        _check_mats(self.mats)
        _device(self.mats)
        self.block_id = [int(b) for b in block_id]
        if len(self.block_id) != len(self.mats):
            raise ValueError(f"block_id: {len(self.block_id)} ids for {len(self.mats)} matrices")
        self.n_blocks = n_blocks
        self.iters, self.bits, self.group, self.x = iters, bits, group, x
        self.tiered = tiered
        self.actions = tuple(actions)
        self.sinq_batch_bytes = sinq_batch_bytes
        dev = self.mats[0].device
        self.device = dev
        n = len(self.mats)
        self.h_mat = torch.empty(n, dtype=torch.float64, device=dev)
        self.h_block = torch.empty(n_blocks, dtype=torch.float64, device=dev)
        self.stats = torch.empty(3, dtype=torch.float64, device=dev)
        self.tier = torch.empty(n_blocks, dtype=torch.int32, device=dev)
        self.order = torch.empty(n_blocks, dtype=torch.int32, device=dev)
        # each bf16 matrix's exponent histogram, from the entropy pass (the
        # input of the lossless code of the kept blocks)
        self.exp_hist = torch.empty(n, 256, dtype=torch.int32, device=dev)
        self._ent_ws = _ws(_lib.OP_ENTROPY, self.mats, 0, dev)
        self._ent_mats = _mat_arr(self.mats)
        self._bid = (ctypes.c_int32 * n)(*self.block_id)
        self._plans: Dict[tuple, tuple] = {}
        self.outputs: Dict[int, dict] = {}
        self.bytes_in = sum(m.numel() * m.element_size() for m in self.mats)
        self.budget_bytes = budget_bytes
        self._side: Optional[torch.cuda.Stream] = None   # second stream of the split Sinkhorn step
        self.last_actions: Optional[List[str]] = None
        self.last_budget: Optional[tuple] = None   # (total bytes, fits)

    # ------------------------------------------------------------ planning
    def _entropy_call(self) -> _Call:
        args = (self._ent_mats, len(self.mats), self._bid, self.n_blocks, float(self.x),
                self.h_mat.data_ptr(), self.h_block.data_ptr(), self.stats.data_ptr(),
                self.tier.data_ptr(), self.order.data_ptr(), self.exp_hist.data_ptr(),
                self._ent_ws.data_ptr(), self._ent_ws.numel())
        return _Call("ewq_block_entropy_ex", self.lib.ewq_block_entropy_ex, args, None, "entropy",
                     self.bytes_in)

    def _sinq_calls(self, idx: List[int]) -> List[_Call]:
        dev = self.device
        mats = [self.mats[i] for i in idx]
        s = [torch.empty(m.shape[0], dtype=torch.float32, device=dev) for m in mats]
        t = [torch.empty(m.shape[1], dtype=torch.float32, device=dev) for m in mats]
        codes = [torch.empty(m.shape[0], m.shape[1] * self.bits // 8, dtype=torch.uint8, device=dev)
                 for m in mats]
        g = self.group
        scales = [torch.empty(m.shape[0], m.shape[1] // g, dtype=torch.float32, device=dev) for m in mats]
        zeros = [torch.empty(m.shape[0], m.shape[1] // g, dtype=torch.uint8, device=dev) for m in mats]
        for k, i in enumerate(idx):
            self.outputs[i] = {"action": "sinq", "s": s[k], "t": t[k], "codes": codes[k],
                               "scales": scales[k], "zeros": zeros[k]}
        calls = []
        # optional batching of the Sinkhorn step (bytes per call)
        batches, cur, cur_b = [], [], 0
        for k, m in enumerate(mats):
            b = m.numel() * m.element_size()
            if cur and self.sinq_batch_bytes and cur_b + b > self.sinq_batch_bytes:
                batches.append(cur)
                cur, cur_b = [], 0
            cur.append(k)
            cur_b += b
        if cur:
            batches.append(cur)
        def sinq_call(ks, flags):
            bm = [mats[k] for k in ks]
            arr = _mat_arr(bm)
            sp = _lib.ptr_array(s[k].data_ptr() for k in ks)
            tp = _lib.ptr_array(t[k].data_ptr() for k in ks)
            ws = _ws(_lib.OP_SINQ, bm, 0, dev)
            nb = sum(m.numel() * m.element_size() for m in bm)
            return _Call("sinq_balance_ex", self.lib.sinq_balance_ex,
                         (arr, len(bm), self.iters, flags, sp, tp, ws.data_ptr(), ws.numel()),
                         (arr, sp, tp, ws), "sinq", nb)

        for bk in batches:
            bm = [mats[k] for k in bk]
            arr = _mat_arr(bm)
            sp = _lib.ptr_array(s[k].data_ptr() for k in bk)
            tp = _lib.ptr_array(t[k].data_ptr() for k in bk)
            nb = sum(m.numel() * m.element_size() for m in bm)
            split = self._sinq_split([mats[k] for k in bk])
            if split is None:
                calls.append(sinq_call(bk, 0))
            else:
                first, second, flags = split
                if self._side is None:
                    self._side = torch.cuda.Stream(device=dev)
                calls.append(_SplitSinq(sinq_call([bk[j] for j in first], 0),
                                        sinq_call([bk[j] for j in second], flags), self._side))
            cp = _lib.ptr_array(codes[k].data_ptr() for k in bk)
            scp = _lib.ptr_array(scales[k].data_ptr() for k in bk)
            zp = _lib.ptr_array(zeros[k].data_ptr() for k in bk)
            wsq = _ws(_lib.OP_QUANT, bm, g, dev)
            calls.append(_Call("quant_pack_groupwise", self.lib.quant_pack_groupwise,
                               (arr, len(bm), sp, tp, self.bits, g, cp, scp, zp, wsq.data_ptr(),
                                wsq.numel()),
                               (arr, sp, tp, cp, scp, zp, wsq), "quant", nb))
        return calls

    @staticmethod
    def _sinq_split(mats: Sequence[torch.Tensor]):
        """(first, second, flags of the second call) as positions in ``mats``
        for the two concurrent Sinkhorn calls (see _SplitSinq), or None for
        one call (a single row width)."""
        narrow = [j for j, m in enumerate(mats) if _wave_form(m)]
        wide = [j for j, m in enumerate(mats) if not _wave_form(m)]
        if narrow and wide:
            return narrow, wide, _lib.WOQ_SINQ_SHARED
        width_bytes: Dict[tuple, int] = {}
        for m in mats:
            key = (m.dtype, m.shape[1])
            width_bytes[key] = width_bytes.get(key, 0) + m.numel() * m.element_size()
        if len(width_bytes) < 2:
            return None
        top = max(width_bytes, key=lambda k: width_bytes[k])
        first = [j for j, m in enumerate(mats) if (m.dtype, m.shape[1]) == top]
        second = [j for j, m in enumerate(mats) if (m.dtype, m.shape[1]) != top]
        return first, second, 0

    def _int8_calls(self, idx: List[int]) -> List[_Call]:
        dev = self.device
        mats = [self.mats[i] for i in idx]
        codes = [torch.empty(m.shape[0], m.shape[1], dtype=torch.uint8, device=dev) for m in mats]
        scales = [torch.empty(m.shape[0], 1, dtype=torch.float32, device=dev) for m in mats]
        zeros = [torch.empty(m.shape[0], 1, dtype=torch.uint8, device=dev) for m in mats]
        for k, i in enumerate(idx):
            self.outputs[i] = {"action": "int8row", "codes": codes[k], "scales": scales[k],
                               "zeros": zeros[k]}
        arr = _mat_arr(mats)
        cp = _lib.ptr_array(c.data_ptr() for c in codes)
        scp = _lib.ptr_array(c.data_ptr() for c in scales)
        zp = _lib.ptr_array(c.data_ptr() for c in zeros)
        ws = _ws(_lib.OP_QUANT, mats, 0, dev)
        nb = sum(m.numel() * m.element_size() for m in mats)
        return [_Call("quant_pack_groupwise", self.lib.quant_pack_groupwise,
                      (arr, len(mats), None, None, 8, 0, cp, scp, zp, ws.data_ptr(), ws.numel()),
                      (arr, cp, scp, zp, ws), "int8row", nb)]

    def _ternary_calls(self, idx: List[int]) -> List[_Call]:
        dev = self.device
        mats = [self.mats[i] for i in idx]
        codes = [torch.empty(m.shape[0], m.shape[1] // 4, dtype=torch.uint8, device=dev) for m in mats]
        beta = [torch.empty(m.shape[0], dtype=torch.float32, device=dev) for m in mats]
        for k, i in enumerate(idx):
            self.outputs[i] = {"action": "ternary", "codes": codes[k], "beta": beta[k]}
        arr = _mat_arr(mats)
        cp = _lib.ptr_array(c.data_ptr() for c in codes)
        bp = _lib.ptr_array(c.data_ptr() for c in beta)
        ws = _ws(_lib.OP_TERNARY, mats, 0, dev)
        nb = sum(m.numel() * m.element_size() for m in mats)
        return [_Call("ternary_pack", self.lib.ternary_pack,
                      (arr, len(mats), cp, bp, ws.data_ptr(), ws.numel()),
                      (arr, cp, bp, ws), "ternary", nb)]

    def action_bytes(self, action: str, m: torch.Tensor) -> int:
        """Storage of one matrix under an action (codes and per-group /
        per-row / per-column metadata)."""
        r, c = m.shape
        if action == "ternary":
            return r * c // 4 + 4 * r
        if action == "sinq":
            return r * c * self.bits // 8 + r * (c // self.group) * 5 + 4 * (r + c)
        if action == "int8row":
            return r * c + 5 * r
        return m.numel() * m.element_size()

    def level_bytes(self) -> List[List[int]]:
        """Per block, its storage at each rung of ACTIONS."""
        out = [[0] * len(ACTIONS) for _ in range(self.n_blocks)]
        for m, b in zip(self.mats, self.block_id):
            for lvl, a in enumerate(ACTIONS):
                out[b][lvl] += self.action_bytes(a, m)
        return out

    def action_of_block(self, tiers) -> List[str]:
        """The action of every block: the first action for an untiered pass
        (``tiers`` unused), else the action of each block's tier."""
        if not self.tiered:
            return [self.actions[0]] * self.n_blocks
        return [self.actions[int(t) - 1] for t in tiers]

    def budgeted_actions(self, tiers, h_block) -> List[str]:
        """EWQ step 3: the tiers' actions moved along ACTIONS to the budget."""
        from . import ewq_budget_levels
        level0 = [ACTIONS.index(a) for a in self.action_of_block(tiers)]
        levels, total, fits = ewq_budget_levels(h_block, self.level_bytes(), level0,
                                                self.budget_bytes)
        self.last_budget = (total, fits)
        return [ACTIONS[lv] for lv in levels]

    def plan(self, tiers) -> List[_Call]:
        return self.plan_actions(self.action_of_block(tuple(int(t) for t in tiers)))

    def plan_actions(self, acts) -> List[_Call]:
        """Calls (and output buffers) for one action per block; cached per
        assignment, and ``outputs`` always describes the latest plan used."""
        key = tuple(acts)
        if key in self._plans:
            calls, outputs = self._plans[key]
            self.outputs = outputs
            return calls
        self.outputs = {}
        by_action: Dict[str, List[int]] = {a: [] for a in ACTIONS}
        for i, b in enumerate(self.block_id):
            by_action[acts[b]].append(i)
        calls: List[_Call] = []
        if by_action["sinq"]:
            calls += self._sinq_calls(by_action["sinq"])
        if by_action["int8row"]:
            calls += self._int8_calls(by_action["int8row"])
        if by_action["ternary"]:
            calls += self._ternary_calls(by_action["ternary"])
        for i in by_action["keep"]:
            self.outputs[i] = {"action": "keep"}
        self._plans[key] = (calls, self.outputs)
        return calls

    # ------------------------------------------------------------ running
    def run(self, stream: Optional[torch.cuda.Stream] = None, timers: Optional[dict] = None,
            read_tiers: bool = True):
        """One whole pass; returns the tiers (host list).  ``timers`` collects
        (kind -> list of (start_event, end_event, bytes)) around each call.
        When the tiers decide nothing (an untiered pass without a budget) the
        pass enqueues everything without waiting for the GPU; with
        ``read_tiers=False`` it then returns None and never synchronises (as
        needed to capture it into a graph)."""
        stream = stream or torch.cuda.current_stream(self.device)
        h = stream.cuda_stream
        calls = [self._entropy_call()]
        self._run_calls(calls, stream, h, timers)
        fixed = not self.tiered and self.budget_bytes is None
        tiers = None
        if fixed:
            acts = self.action_of_block(None)
        else:
            tiers = self.tier.cpu().tolist()   # the one host synchronisation
            if self.budget_bytes is None:
                acts = self.action_of_block(tiers)
            else:
                acts = self.budgeted_actions(tiers, self.h_block.cpu().tolist())
        self.last_actions = acts
        self._run_calls(self.plan_actions(acts), stream, h, timers)
        if tiers is None and read_tiers:
            tiers = self.tier.cpu().tolist()
        return tiers

    def graph(self, stream: Optional[torch.cuda.Stream] = None) -> "torch.cuda.CUDAGraph":
        """The whole pass captured into a HIP graph (untiered passes without a
        budget only: a tiered pass reads the tiers back on the host).  One
        eager pass first prepares every buffer; the graph's replay then runs
        the same kernels on the same buffers, with no host work per kernel."""
        if self.tiered or self.budget_bytes is not None:
            raise ValueError("only an untiered pass without a budget can be captured")
        stream = stream or torch.cuda.current_stream(self.device)
        self.run(stream=stream)
        torch.cuda.synchronize(self.device)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=torch.cuda.Stream(device=self.device)):
            self.run(read_tiers=False)
        torch.cuda.synchronize(self.device)
        return g

    def compress_kept(self, stream: Optional[torch.cuda.Stream] = None) -> int:
        """Lossless exponent code for the matrices the last run kept in bf16:
        one df11_compress over all of them, from the exponent histograms the
        entropy pass already counted (no second read of the kept weights
        before encoding; each matrix gets its own code, which comes from the
        data, so this step synchronises once).  Sets outputs[i]["df11"];
        returns the stored bytes of the kept matrices."""
        from . import df11_compress
        if self.last_actions is None:
            raise RuntimeError("run() first")
        idx = [i for i, b in enumerate(self.block_id) if self.last_actions[b] == "keep"]
        if not idx:
            return 0
        stored = 0
        hist = self.exp_hist[idx]
        for i, e in zip(idx, df11_compress([self.mats[i] for i in idx], hist=hist, stream=stream)):
            self.outputs[i]["df11"] = e
            stored += (e["enc"].numel() + e["sm"].numel() + e["gaps"].numel()
                       + 4 * e["block_pos"].numel() + e["tables"].numel() + 256)
        return stored

    @staticmethod
    def _run_calls(calls, stream, h, timers):
        for c in calls:
            if timers is not None:
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                c(h, stream)
                e1.record(stream)
                timers.setdefault(c.kind, []).append((e0, e1, c.nbytes))
            else:
                c(h, stream)
