"""A whole data-parallel step on one GPU through the C ABI.

``DPStep`` allocates the state in HBM with torch (memory only), binds it to a
plan and issues one step as:

* fused (default): ``dp_accumulate_all`` for micro-steps 1 .. a-1 (every
  replica in one launch), then ``dp_accumulate_reduce`` for micro-step a (the
  last accumulation fused with the replica average); with a = 1 or incoming
  partials only the latter;
* per replica: ``dp_accumulate`` for every (micro-step, replica), then
  ``dp_reduce_replicas`` (with n = 1 the last accumulation writes the
  statistics instead);

then ``dp_grad_stats`` and one ``dp_adam_step`` per shard range.  Both
sequences give the same bits.  With ``single_pass`` (runs without clipping)
the last micro-step, the replica average, the statistics and the update are
one ``dp_reduce_adam_step`` over two state banks; again the same bits.
Gradients come from a caller-supplied producer, standing in for the backward
pass; the fused sequence needs the n replicas' gradients of one micro-step at
once.  ``step_overlapped`` issues the same step bucket by bucket
(``dp_accumulate_reduce_range``, or ``dp_reduce_adam_range`` and
``dp_reduce_adam_finish`` for the single pass, and with ``micro_buckets`` also
``dp_accumulate_all_range`` for the earlier micro-steps), on a second stream
as the producer writes each bucket; again the same bits.

HBM layout (flat parameter space of P elements, tensors in list order; see
``layout`` for where the arrays sit relative to each other):
master, exp_avg, exp_avg_sq: binary32 [P] (two banks of each with
``single_pass``; in pinned host memory with ``state_location="host"``); param: bf16/fp16 [P]; acc[r]: binary32 [P] per replica
(absent for partials; with n = 1, acc[0] is also g_bar); gbar: binary32 [P]
when n > 1 or with partials, and not with ``single_pass``; gradients: the
producer's buffers, bound per call.
"""
from __future__ import annotations

from typing import Callable, List, Optional, Sequence, Tuple

import torch

from . import DP_ROLE_EXP_AVG, DP_ROLE_EXP_AVG_SQ, DP_ROLE_GRAD, DP_ROLE_MASTER, Plan, dp_plan_bind_flat

TORCH_DTYPES = {"bf16": torch.bfloat16, "f16": torch.float16}

# producer(step, replica, micro, loss_scale) -> device address of that gradient
GradProducer = Callable[[int, int, int, float], int]


# producer(step, micro, lo, hi, stream): writes every replica's gradient of
# elements [lo, hi) for that micro-step into its flat gradient buffer, on stream
RangeProducer = Callable[[int, int, int, int, int], None]


def backward_buckets(numel: Sequence[int], bucket_bytes: int, elem_bytes: int = 2,
                     split: bool = False) -> List[Tuple[int, int]]:
    """Buckets for a reduction that overlaps the backward pass: runs of whole
    tensors taken from the last tensor back to the first (the order in which
    a backward pass finishes them), each closed once it holds at least
    bucket_bytes of gradients.  Returned in that order.  With split, a tensor
    larger than one bucket is cut into buckets of bucket_bytes rounded down to
    a multiple of 256 elements, counted from its start (the buckets of a flat
    shard whose gradients arrive from the exchange in pieces)."""
    offs = [0]
    for x in numel:
        offs.append(offs[-1] + int(x))
    out: List[Tuple[int, int]] = []
    hi = offs[-1]
    acc = 0
    step = max(256, (bucket_bytes // elem_bytes) // 256 * 256)
    for t in range(len(numel) - 1, -1, -1):
        if split and int(numel[t]) * elem_bytes > bucket_bytes:
            if offs[t + 1] < hi:  # close the run of smaller tensors after it
                out.append((offs[t + 1], hi))
            starts = list(range(offs[t], offs[t + 1], step))
            out.extend(reversed(list(zip(starts, starts[1:] + [offs[t + 1]]))))
            hi, acc = offs[t], 0
            continue
        acc += int(numel[t]) * elem_bytes
        if acc >= bucket_bytes or t == 0:
            if offs[t] < hi:
                out.append((offs[t], hi))
            hi, acc = offs[t], 0
    return out


def even_shards(P: int, shards: int) -> List[Tuple[int, int]]:
    cuts = [P * i // shards for i in range(shards + 1)]
    return [(cuts[i], cuts[i + 1]) for i in range(shards)]


class StepGraph:
    """A step captured into a HIP graph.  ``replay`` launches it on the step's
    own stream, so a replay is ordered after the work issued there before it
    (new gradients written on that stream) and before the work issued after
    it (``read_state``, the next gradients).  torch's own ``replay`` launches
    on the current stream, which is not ordered with the step's stream."""

    def __init__(self, graph: "torch.cuda.CUDAGraph", stream: "torch.cuda.Stream"):
        self.graph = graph
        self.stream = stream

    def replay(self) -> None:
        with torch.cuda.stream(self.stream):
            self.graph.replay()


class DPStep:
    def __init__(self, numel: Sequence[int], n: int, a: int, grad_dtype: str, param_dtype: str, *,
                 lr: float = 1e-3, eps: float = 1e-8, weight_decay: float = 0.01, beta1: float = 0.9,
                 beta2: float = 0.999, max_norm: float = 0.0, scaler: str = "none", init_scale: float = 1.0,
                 backoff: float = 0.5, growth: float = 2.0, growth_interval: int = 2000, partials: bool = False,
                 shards: Optional[Sequence[Tuple[int, int]]] = None, chunk_elems: int = 0,
                 device: str = "cuda:0", stream: Optional[torch.cuda.Stream] = None, fused: bool = True,
                 single_pass: bool = False, state_location: str = "hbm", offload: str = "direct",
                 stage_elems: int = 1 << 24, layout: str = "auto"):
        if partials and a != 1:
            raise ValueError("incoming partials are reduced directly: a must be 1")
        if single_pass and max_norm > 0.0:
            raise ValueError("the single pass updates before the global norm is known: it needs max_norm = 0")
        if single_pass and not (fused or partials):
            raise ValueError("the single pass reads every replica's last micro-step at once: it needs fused = True")
        if single_pass and shards is not None and list(shards) != [(0, sum(numel))]:
            raise ValueError("the single pass updates the whole range in one call")
        if state_location not in ("hbm", "host"):
            raise ValueError("state_location is 'hbm' or 'host'")
        if offload not in ("direct", "staged"):
            raise ValueError("offload is 'direct' or 'staged'")
        if offload == "staged" and (state_location != "host" or single_pass):
            raise ValueError("the staged offload moves a host-resident state for the two-pass update")
        self.offload = offload
        self.n, self.a, self.partials, self.fused, self.single_pass = n, a, partials, fused, single_pass
        self.state_location = state_location
        self.lr, self.eps, self.weight_decay, self.max_norm = lr, eps, weight_decay, max_norm
        self.scaler = scaler
        self.plan = Plan(numel, n, grad_dtype, param_dtype, chunk_elems)
        P = self.P = self.plan.P
        self.device = torch.device(device)
        self.stream = stream if stream is not None else torch.cuda.current_stream(self.device)
        f32 = dict(dtype=torch.float32, device=self.device)
        pdt = TORCH_DTYPES[param_dtype]
        own_gbar = not (n == 1 and not partials) and not single_pass
        nbanks = 2 if single_pass else 1
        # The arrays one update streams together: g_bar (two passes), master, m
        # and v of every bank, and the parameters.
        update = ([("gbar", torch.float32)] if own_gbar else []) + \
            [(f"{r}{b}", torch.float32) for b in range(nbanks) for r in ("master", "exp_avg", "exp_avg_sq")] + \
            [("param", pdt)]
        self.layout = self._choose_layout(layout, state_location, update, P, 0 if partials else n)
        arrays = {}
        if self.layout == "spread":
            arrays = self._spread_arrays(update, P, 0 if partials else n)
        else:
            # optimizer state (master, m, v): in HBM, or offloaded to pinned
            # host memory that the update kernels read and write across PCIe
            st32 = f32 if state_location == "hbm" else dict(dtype=torch.float32, pin_memory=True)
            for name, dt in update:
                host = name.startswith(("master", "exp_avg")) and state_location == "host"
                arrays[name] = torch.zeros(P, **(st32 if host else dict(dtype=dt, device=self.device)))
            # the n accumulators are rows of one allocation: the micro-step
            # launch over all replicas then streams one contiguous region
            if not partials:
                arrays["acc"] = torch.zeros((n, P), **f32)
        self.master, self.exp_avg, self.exp_avg_sq = arrays["master0"], arrays["exp_avg0"], arrays["exp_avg_sq0"]
        self.param = arrays["param"]
        self.acc: List[torch.Tensor] = list(arrays["acc"].unbind(0)) if not partials else []
        if n == 1 and not partials:
            self.gbar = self.acc[0]
        else:
            self.gbar = arrays.get("gbar")
        # state banks: (master, exp_avg, exp_avg_sq); bank 1 only for the single pass
        self.banks = [tuple(arrays[f"{r}{b}"] for r in ("master", "exp_avg", "exp_avg_sq")) for b in range(nbanks)]
        pl = self.plan
        for b, (w_, m_, v_) in enumerate(self.banks):
            pl.bind("master", w_, b)
            pl.bind("exp_avg", m_, b)
            pl.bind("exp_avg_sq", v_, b)
        pl.bind("param", self.param)
        for r, t in enumerate(self.acc):
            pl.bind("acc", t, r)
        if self.gbar is not None and self.gbar is not (self.acc[0] if self.acc else None):
            pl.bind("gbar", self.gbar)
        self.shards = list(shards) if shards is not None else [(0, P)]
        for b, e in self.shards:
            pl.prepare_range(b, e)
        if offload == "staged":
            # three device slots of stage_elems elements of master, m, v, and
            # the pieces of every shard that pass through them
            self.stage_elems = int(stage_elems)
            self.stage = [tuple(torch.empty(self.stage_elems, **f32) for _ in range(3)) for _ in range(3)]
            self.stage_pieces = [(lo, min(e, lo + self.stage_elems)) for b, e in self.shards
                                 for lo in range(b, e, self.stage_elems)]
            for lo, hi in self.stage_pieces:
                pl.prepare_range(lo, hi)
            self.copy_in, self.copy_out = torch.cuda.Stream(self.device), torch.cuda.Stream(self.device)
        pl.state_init(beta1, beta2, scaler, init_scale, backoff, growth, growth_interval, stream=self.stream)
        self.scale = 1.0 if scaler == "none" else float(init_scale)
        self.steps_done = 0

    # -- HBM layout ---------------------------------------------------------
    # Where the arrays of one kernel sit relative to each other changes its
    # bandwidth on MI355X by up to 8%, and not by a rule that held across the
    # workloads measured (16 GiB slot offsets sped up the update of some and
    # slowed others).  "packed" (the default, also what "auto" picks) lets
    # torch place each array; "spread" carves the update's arrays from one
    # allocation at slot offsets that are multiples of 16 GiB, with the
    # accumulators after them, holding the gaps between slots allocated too.
    SLOT = 16 << 30
    ALIGN = 2 << 20

    def _spread_plan(self, update, P: int, nacc: int):
        nbytes = [P * torch.tensor([], dtype=dt).element_size() for _, dt in update]
        slot = self.SLOT * max(1, -(-max(nbytes) // self.SLOT))
        offs = [k * slot for k in range(len(update))]
        acc_off = -(-(offs[-1] + nbytes[-1]) // self.ALIGN) * self.ALIGN
        total = acc_off + nacc * P * 4
        return slot, offs, nbytes, acc_off, total

    def _choose_layout(self, layout: str, state_location: str, update, P: int, nacc: int) -> str:
        if layout not in ("auto", "packed", "spread"):
            raise ValueError("layout is 'auto', 'packed' or 'spread'")
        if layout == "packed" or state_location != "hbm" or P == 0:
            return "packed"
        if layout == "spread":
            total = self._spread_plan(update, P, nacc)[-1]
            free, _ = torch.cuda.mem_get_info(self.device)
            if total > free:
                raise MemoryError(f"the spread layout needs {total} bytes of HBM, {free} are free")
            return "spread"
        return "packed"

    def _spread_arrays(self, update, P: int, nacc: int) -> dict:
        _, offs, nbytes, acc_off, total = self._spread_plan(update, P, nacc)
        self.arena = torch.empty(total, dtype=torch.uint8, device=self.device)
        out = {}
        for (name, dt), off, nb in zip(update, offs, nbytes):
            out[name] = self.arena[off:off + nb].view(dt).zero_()
        if nacc:
            out["acc"] = self.arena[acc_off:acc_off + nacc * P * 4].view(torch.float32).view(nacc, P).zero_()
        return out

    # -- setup ------------------------------------------------------------
    def set_master(self, fill: Callable[[int], None]) -> None:
        """fill(address) writes the initial binary32 master weights into device
        memory; the low-precision copy starts as their round-to-nearest-even
        image."""
        dev = self.master if self.state_location == "hbm" else torch.empty(self.P, dtype=torch.float32,
                                                                            device=self.device)
        fill(dev.data_ptr())
        cur = torch.cuda.current_stream(self.device)
        cur.wait_stream(self.stream)
        self.param.copy_(dev.to(self.param.dtype))
        if dev is not self.master:
            self.master.copy_(dev)
            torch.cuda.synchronize(self.device)
        self.stream.wait_stream(cur)  # the step's launches come after these copies

    # -- one step ---------------------------------------------------------
    def issue_gradients(self, produce: GradProducer, step: int) -> None:
        """The accumulation (or partial) part of a step, up to g_bar."""
        pl, st, h = self.plan, self.stream.cuda_stream, self.plan.handle
        if self.partials or self.fused:
            last = 1 if self.partials else self.a
            for k in range(1, last):
                for r in range(self.n):
                    dp_plan_bind_flat(h, DP_ROLE_GRAD, r, produce(step, r, k, self.scale))
                pl.accumulate_all(first=(k == 1), stream=st)
            for r in range(self.n):
                dp_plan_bind_flat(h, DP_ROLE_GRAD, r, produce(step, r, last, self.scale))
            if not self.single_pass:  # else the reduction is part of finish()
                pl.accumulate_reduce(stream=st)
            return
        for k in range(1, self.a + 1):
            for r in range(self.n):
                dp_plan_bind_flat(h, DP_ROLE_GRAD, r, produce(step, r, k, self.scale))
                pl.accumulate(r, first=(k == 1), emit_stats=(self.n == 1 and k == self.a), stream=st)
        if self.n > 1:
            pl.reduce_replicas("acc", stream=st)

    def finish(self) -> None:
        """Statistics, scalars and the update on every shard range."""
        pl, st = self.plan, self.stream.cuda_stream
        if self.single_pass:
            pl.reduce_adam_step(self.lr, self.eps, self.weight_decay, stream=st)
            return
        pl.grad_stats(scan=False, max_norm=self.max_norm, stream=st)
        if self.offload == "staged":
            self.staged_update()
            return
        for b, e in self.shards:
            pl.adam_step(self.lr, self.eps, self.weight_decay, b, e, stream=st)

    def staged_update(self) -> None:
        """The update with the state streamed through device slots: piece j's
        master, m and v are copied in on one stream, updated in slot j mod 3
        (the roles rebound to the slot) on the step's stream, and copied back
        on a third; the copies of neighbouring pieces overlap the update."""
        pl, h, st = self.plan, self.plan.handle, self.stream
        host = (self.master, self.exp_avg, self.exp_avg_sq)
        roles = (DP_ROLE_MASTER, DP_ROLE_EXP_AVG, DP_ROLE_EXP_AVG_SQ)
        slot_free = [None, None, None]  # event: the slot's last copy-out finished
        done = []
        # every copy-in comes after the work already on the step's stream, which
        # includes the previous step's copy-outs
        self.copy_in.wait_stream(st)
        for j, (lo, hi) in enumerate(self.stage_pieces):
            k, n = j % 3, hi - lo
            slot = self.stage[k]
            if slot_free[k] is not None:
                self.copy_in.wait_event(slot_free[k])
            with torch.cuda.stream(self.copy_in):
                for d_, h_ in zip(slot, host):
                    d_[:n].copy_(h_[lo:hi], non_blocking=True)
            ready = torch.cuda.Event()
            ready.record(self.copy_in)
            st.wait_event(ready)
            for role, d_ in zip(roles, slot):
                dp_plan_bind_flat(h, role, 0, d_.data_ptr() - 4 * lo)
            pl.adam_step(self.lr, self.eps, self.weight_decay, lo, hi, stream=st.cuda_stream)
            updated = torch.cuda.Event()
            updated.record(st)
            self.copy_out.wait_event(updated)
            with torch.cuda.stream(self.copy_out):
                for d_, h_ in zip(slot, host):
                    h_[lo:hi].copy_(d_[:n], non_blocking=True)
            slot_free[k] = torch.cuda.Event()
            slot_free[k].record(self.copy_out)
            done.append(slot_free[k])
        for ev in done[-3:]:
            st.wait_event(ev)
        for role, t in zip(roles, host):  # the bindings point at the host state again
            dp_plan_bind_flat(h, role, 0, t.data_ptr())

    def step(self, produce: GradProducer, sync_scale: bool = True) -> Optional[dict]:
        self.steps_done += 1
        self.issue_gradients(produce, self.steps_done)
        self.finish()
        if sync_scale:
            s = self.read_state()
            self.scale = s["scale"]
            return s
        return None

    def step_overlapped(self, grad_slots: Sequence[int], produce: RangeProducer, buckets: Sequence[Tuple[int, int]],
                        reduce_stream: Optional[torch.cuda.Stream] = None, sync_scale: bool = True,
                        marks: Optional[Tuple[torch.cuda.Event, torch.cuda.Event]] = None,
                        micro_buckets: bool = False) -> Optional[dict]:
        """One step in which the backward pass of the last micro-step hands
        over its gradients bucket by bucket and the replica reduction follows
        bucket by bucket (``dp_accumulate_reduce_range``); with
        ``single_pass`` each bucket's reduction also updates its parameters
        (``dp_reduce_adam_range``, then ``dp_reduce_adam_finish``).  The
        earlier micro-steps accumulate without any exchange, as a
        data-parallel run with gradient accumulation does: over the whole
        space after their backward pass, or with ``micro_buckets`` bucket by
        bucket as it produces them (``dp_accumulate_all_range``).

        The gradient buffers are flat (grad_slots[r]: replica r's, P
        elements), and the producer fills them range by range on this step's
        stream.  With a separate reduce_stream, the reduction of a bucket runs
        there as soon as the producer has written it, overlapping the
        production of the next bucket (events order each bucket's reduction
        after its production, and the statistics after every reduction).
        Without one, production and reduction alternate on one stream.  Same
        bits as ``step`` in either case.  With bucketed micro-steps on a
        second stream, the producer rewrites a bucket of the gradient buffers
        only after the previous micro-step's accumulation has read it (one
        event per bucket).  marks, if given, are recorded on this step's
        stream before the last micro-step and after its last reduction."""
        pl, h = self.plan, self.plan.handle
        st = self.stream.cuda_stream
        self.steps_done += 1
        s = self.steps_done
        for r, addr in enumerate(grad_slots):
            dp_plan_bind_flat(h, DP_ROLE_GRAD, r, addr)
        last = 1 if self.partials else self.a
        rs = reduce_stream if reduce_stream is not None else self.stream
        two = rs is not self.stream
        read = {}  # bucket -> event on rs after the last launch that read its gradients

        def produce_bucket(k, i, lo, hi):
            # the producer rewrites bucket i once its previous contents are
            # read, and the consumer reads it once it is written
            if two and i in read:
                self.stream.wait_event(read[i])
            produce(s, k, lo, hi, st)
            if two:
                ev = torch.cuda.Event()
                ev.record(self.stream)
                rs.wait_event(ev)

        for k in range(1, last):
            if micro_buckets:
                for i, (lo, hi) in enumerate(buckets):
                    produce_bucket(k, i, lo, hi)
                    pl.accumulate_all_range(k == 1, lo, hi, stream=rs.cuda_stream)
                    if two:
                        read[i] = torch.cuda.Event()
                        read[i].record(rs)
            else:
                produce(s, k, 0, self.P, st)
                pl.accumulate_all(first=(k == 1), stream=st)
        if marks is not None:
            marks[0].record(self.stream)
        for i, (lo, hi) in enumerate(buckets):
            produce_bucket(last, i, lo, hi)
            if self.single_pass:
                pl.reduce_adam_range(self.lr, self.eps, self.weight_decay, lo, hi, stream=rs.cuda_stream)
            else:
                pl.accumulate_reduce_range(lo, hi, stream=rs.cuda_stream)
        if rs is not self.stream:
            ev = torch.cuda.Event()
            ev.record(rs)
            self.stream.wait_event(ev)
        if marks is not None:
            marks[1].record(self.stream)
        if self.single_pass:
            pl.reduce_adam_finish(stream=st)
        else:
            self.finish()
        if sync_scale:
            state = self.read_state()
            self.scale = state["scale"]
            return state
        return None

    def issue_fixed(self, grad_slots: Sequence[Sequence[int]]) -> None:
        """One whole step (accumulation, reduction, statistics, update) that
        reads micro-step k's gradient of replica r from grad_slots[k - 1][r],
        with no host synchronisation: the form a graph can capture."""
        pl, st, h = self.plan, self.stream.cuda_stream, self.plan.handle
        last = 1 if self.partials else self.a
        if not (self.partials or self.fused):
            raise ValueError("the fixed-buffer step uses the fused sequence")
        for k in range(1, last):
            for r in range(self.n):
                dp_plan_bind_flat(h, DP_ROLE_GRAD, r, grad_slots[k - 1][r])
            pl.accumulate_all(first=(k == 1), stream=st)
        for r in range(self.n):
            dp_plan_bind_flat(h, DP_ROLE_GRAD, r, grad_slots[last - 1][r])
        if not self.single_pass:
            pl.accumulate_reduce(stream=st)
        self.finish()

    def capture_step(self, grad_slots: Sequence[Sequence[int]]) -> "StepGraph":
        """Captures ``issue_fixed`` into a HIP graph on this step's stream
        (which must not be the null stream).  Each replay runs one more step on
        whatever the gradient buffers then hold; the plan's host-side call
        checks ran once, at capture.  The step's launches are kernels only (no
        memset nodes)."""
        if self.stream.cuda_stream == 0:
            raise ValueError("capture needs a non-default stream: pass stream=torch.cuda.Stream()")
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=self.stream):
            self.issue_fixed(grad_slots)
        return StepGraph(g, self.stream)

    def read_state(self) -> dict:
        return self.plan.read_state(stream=self.stream.cuda_stream)

    # -- checkpoints (dpckpt.h) ---------------------------------------------
    def save_checkpoint(self, directory: str, generation: int,
                        ranges: Optional[Sequence[Tuple[int, int]]] = None) -> None:
        """One shard file per range (default: the update's shard ranges), then
        the commit of the generation."""
        st = self.stream.cuda_stream
        for b, e in (ranges if ranges is not None else self.shards):
            self.plan.checkpoint_save(directory, generation, b, e, stream=st)
        self.plan.checkpoint_commit(directory, generation, stream=st)

    def load_checkpoint(self, directory: str, ranges: Optional[Sequence[Tuple[int, int]]] = None) -> dict:
        """Restores the state over the given partition of [0, P) (default: the
        update's shard ranges; any partition works) and resumes the step count
        and the loss scale from it."""
        st = self.stream.cuda_stream
        for i, (b, e) in enumerate(ranges if ranges is not None else self.shards):
            self.plan.checkpoint_load(directory, b, e, restore_scalars=(i == 0), stream=st)
        s = self.read_state()
        self.scale = s["scale"]
        self.steps_done = s["iter"]
        return s

    def state_tensors(self) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
        """(master, exp_avg, exp_avg_sq) of the current bank (synchronises)."""
        return self.banks[self.read_state()["bank"]]

    def close(self) -> None:
        """Destroys the plan and drops this step's arrays, so their memory
        returns to torch's allocator unless the caller still holds them."""
        self.plan.close()
        self.master = self.exp_avg = self.exp_avg_sq = self.param = self.gbar = None
        self.banks, self.acc = [], []
        for name in ("arena", "stage"):
            if hasattr(self, name):
                setattr(self, name, None)
