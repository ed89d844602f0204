"""One pass of the hot path on two HIP streams, built from the C-ABI calls.

One stream runs the signaling GEMM; the other runs the consumer and then the
post-communication reorder, over the whole output or group by group
(consumer(g), then the reorder of g's tiles, for each group in turn, so the
first groups are back in row-major order while the GEMM still computes the
last ones).  The two are linked on the device only through
the signal words (counting table + flags).  Passes are kept in order: a
pass's GEMM starts after the previous pass's post-reorder, as a layer's GEMM
waits for the previous layer's output.  The two streams swap roles every
pass, so that ordering is the hardware queue's own (the GEMM is queued
behind the previous post-reorder on the same stream) and no event sits on
the critical path.  The consumer needs no event either: it may start as soon
as the previous GEMM on its queue ends, but it touches its buffers only once
a flag of its own epoch is raised, i.e. after this pass's GEMM has started,
which is after the previous post-reorder (the last reader of recv) ended.

Consumer: ``consumer="gated"`` (the default) enqueues, per group, a stream
wait for the group's flag (one polling wave, in the runtime's implementation)
and then a streaming kernel over the span (``fo_consume_group_gated``): the
span kernel starts only once the group is signalled.  ``consumer="poll"`` runs the persistent consumer that
polls the flags on the CUs (``fo_consume_group``), one workgroup per CU beside
the GEMM.

Streams: both come from ``fo_stream_create``, so each has a hardware queue of
its own and the consumer really runs beside the GEMM.  Launch order: the GEMM
is enqueued before its consumer and waits only for earlier passes' kernels,
none of which wait for it, so even streams that shared a queue would
complete (serialised, without overlap).

Buffers (torch tensors, 16-bit elements stored as int16):
  A [M*K], B [problems*N*K], reorder_buf / peer / recv / out [M*N],
  sig int32 [sig_words] (cnt[P], then flag[P] from flag_offset; zeroed once;
  epochs count up), status int32 [1].
"""

from __future__ import annotations

from typing import Optional

from . import Plan, stream_create, stream_destroy


class Pipeline:
    def __init__(self, plan: Plan, A, B, peer, *, consumer_workgroups: int = 0, timeout_us: int = 0,
                 in_place: bool = False, post_per_group: bool = False, streams: Optional[tuple] = None,
                 consumer: str = "gated"):
        import torch
        self.torch = torch
        self.plan = plan
        if consumer not in ("gated", "poll"):
            raise ValueError("consumer must be 'gated' or 'poll'")
        self.consumer = consumer
        # post_per_group: the stream-B side runs consumer(g), post-reorder(g) for each group in turn,
        # so a group's tiles go back in place while later groups are computed
        self.post_per_group = post_per_group
        n = plan.M * plan.N
        dev = A.device
        self.A, self.B, self.peer = A, B, peer
        self.buf = torch.empty(n, dtype=torch.int16, device=dev)
        self.recv = self.buf if in_place else torch.empty(n, dtype=torch.int16, device=dev)
        self.out = torch.empty(n, dtype=torch.int16, device=dev)
        self.sig = plan.new_sig(dev)
        self.status = torch.zeros(1, dtype=torch.int32, device=dev)
        # each side gets a hardware queue of its own, or the consumer would run after the GEMM.
        # streams=(sa, sb): a pair from stream_create() shared with other pipelines (the caller
        # destroys it); the device has few hardware queues, and pipelines with a pair each can
        # end up with both sides of one pair on the same queue
        self.own_streams = streams is None
        if streams is None:
            with torch.cuda.device(dev):
                self.sa = stream_create()
                self.sb = stream_create()
        else:
            self.sa, self.sb = streams
        self.epoch = 0
        self.consumer_workgroups = consumer_workgroups
        self.timeout_us = timeout_us
        # inputs were produced on the current stream
        ready = torch.cuda.Event()
        ready.record(torch.cuda.current_stream(dev))
        self.sa.wait_event(ready)
        self.sb.wait_event(ready)
        self.post_stream = self.sb   # the queue the last post-reorder was enqueued on

    def close(self):
        """Wait for the streams, then release them."""
        if getattr(self, "sa", None) is not None:
            self.sa.synchronize()
            self.sb.synchronize()
            if self.own_streams:
                stream_destroy(self.sa)
                stream_destroy(self.sb)
            self.sa = self.sb = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def step(self, trace=None, consumer_trace=None, events: Optional[dict] = None, serial: bool = False):
        """Enqueue one pass; returns the epoch it used.  ``events`` may hold
        torch.cuda.Event pairs recorded around a kernel on its own stream, under
        any of the keys 'gemm', 'consume', 'post' -> (start, end).  ``serial``
        puts the three kernels on one queue, so the consumer starts only after
        the GEMM has finished (every flag already raised): the same pass without
        overlap, for comparison."""
        p = self.plan
        self.epoch += 1
        e = self.epoch
        # the previous pass's consumer and post-reorder ran on s_gemm: the GEMM queues behind them
        if serial:
            s_gemm = s_comm = self.sa
        else:
            s_gemm, s_comm = (self.sa, self.sb) if e % 2 == 0 else (self.sb, self.sa)
        if s_gemm is not self.post_stream:
            # only next to a pass without overlap: order this GEMM after the previous post-reorder
            # (two GEMMs in flight at once would interleave their epochs' counts)
            done = self.torch.cuda.Event()
            done.record(self.post_stream)
            s_gemm.wait_event(done)
        ev = events or {}
        if "gemm" in ev:
            ev["gemm"][0].record(s_gemm)
        p.gemm_signal(self.A, self.B, self.buf, self.sig, e, trace=trace, stream=s_gemm)
        if "gemm" in ev:
            ev["gemm"][1].record(s_gemm)
        if "consume" in ev:
            ev["consume"][0].record(s_comm)
        if self.post_per_group and p.P > 1:
            # events: 'consume' spans the whole stream-B side, 'post' the last group's post-reorder
            for g in range(p.P):
                self._consume(e, g, g + 1, consumer_trace, s_comm)
                if "post" in ev and g == p.P - 1:
                    ev["post"][0].record(s_comm)
                p.reorder_post(self.recv, self.out, stream=s_comm, groups=(g, g + 1))
            if "consume" in ev:
                ev["consume"][1].record(s_comm)
            if "post" in ev:
                ev["post"][1].record(s_comm)
        else:
            self._consume(e, 0, p.P, consumer_trace, s_comm)
            if "consume" in ev:
                ev["consume"][1].record(s_comm)
            if "post" in ev:
                ev["post"][0].record(s_comm)
            p.reorder_post(self.recv, self.out, stream=s_comm)
            if "post" in ev:
                ev["post"][1].record(s_comm)
        self.post_stream = s_comm
        return e

    def next_gemm_stream(self):
        """The stream the next overlapped pass will launch its GEMM on (the streams swap roles every pass)."""
        return self.sa if (self.epoch + 1) % 2 == 0 else self.sb

    def _consume(self, epoch, g0, g1, consumer_trace, stream):
        p = self.plan
        if self.consumer == "gated":
            p.consume_group_gated(self.buf, self.peer, self.recv, self.sig, epoch, self.status, g_begin=g0, g_end=g1,
                                  trace=consumer_trace, stream=stream)
        else:
            p.consume_group(self.buf, self.peer, self.recv, self.sig, epoch, self.status, g_begin=g0, g_end=g1,
                            timeout_us=self.timeout_us, num_workgroups=self.consumer_workgroups,
                            trace=consumer_trace, stream=stream)

    def join(self):
        """Make the current stream wait for both streams."""
        cur = self.torch.cuda.current_stream(self.A.device)
        ea, eb = self.torch.cuda.Event(), self.torch.cuda.Event()
        ea.record(self.sa)
        eb.record(self.sb)
        cur.wait_event(ea)
        cur.wait_event(eb)
