"""The decode step captured into one HIP graph per batch bucket.

A serving loop runs the step at whatever batch the scheduler holds; replaying
a captured graph removes the host's per-kernel launch work, but a graph is
fixed to one batch.  The page "How We Made Our Text-to-Speech API Free"
(section "GPU Infrastructure: Owning the Stack", part "Hardware and
Procurement") reports that capping captured batches at 24 left the GPU
under-used at 32 and 64 concurrent requests, and that capturing up to
min(max running requests, 64) restored the throughput curve.  So buckets
here go up to 64 by default.

A batch of b rows runs on the smallest bucket >= b: the caller's rows are
copied into the bucket's static input and the live row count b into a
device word the captured step reads; rows b and above are computed and
ignored, and append nothing to the KV caches (their kv_len must still be
valid, which it is when the state was built for the largest bucket), so
sequences parked in those rows keep their cache; the first b rows of the
bucket's output are returned.  Every bucket has its own
workspace, input and output buffers, so replays of different buckets never
share scratch memory.  The library makes no allocation, synchronisation or
memset inside the step, so capture needs nothing else.
"""

import torch

from . import ops

DEFAULT_BUCKETS = (1, 2, 4, 8, 16, 24, 32, 40, 48, 56, 64)


class StepGraphs:
    """One captured dual_ar_decode_step per batch bucket.

    model: ops.DualArModel; kv: ops.KvState whose kv_len (and caches) cover
    at least max(buckets) rows."""

    def __init__(self, model, kv, buckets=DEFAULT_BUCKETS, device="cuda"):
        n_rows = kv.kv_len.shape[0]
        self.buckets = sorted(set(int(b) for b in buckets if 1 <= b <= n_rows))
        if not self.buckets:
            raise ValueError("no bucket fits the KV state")
        self.model = model
        self.live = torch.zeros(1, dtype=torch.int32, device=device)
        self.kv = kv = kv.with_live_rows(self.live)
        C = len(model.embed)
        self.err = torch.zeros(1, dtype=torch.int32, device=device)
        self.graphs = {}
        for B in self.buckets:
            self.live.fill_(B)
            st = {"prev": torch.zeros((B, C), dtype=torch.int32, device=device),
                  "codes": torch.zeros((B, C), dtype=torch.int32, device=device),
                  "ws": model.new_workspace(B, kv.c.max_kv_len_hint, device)}

            def step(st=st):
                ops.dual_ar_decode_step(model, kv, st["prev"], codes=st["codes"], workspace=st["ws"], err=self.err)
            side = torch.cuda.Stream()               # warm-up off the capture stream
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                step()
            torch.cuda.current_stream().wait_stream(side)
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step()
            st["graph"] = g
            self.graphs[B] = st
        torch.cuda.synchronize()

    def bucket_for(self, b):
        for B in self.buckets:
            if B >= b:
                return B
        raise ValueError(f"batch {b} above the largest bucket {self.buckets[-1]}")

    def step(self, prev_codes):
        """Codes int32 [b, C] of one step for prev_codes int32 [b, C] (on the
        current stream; no synchronisation)."""
        b = prev_codes.shape[0]
        st = self.graphs[self.bucket_for(b)]
        st["prev"][:b].copy_(prev_codes)
        self.live.fill_(b)
        st["graph"].replay()
        return st["codes"][:b]

    def replay(self, B):
        """Replay bucket B as captured (its static input unchanged, all rows live)."""
        self.live.fill_(B)
        self.graphs[B]["graph"].replay()
        return self.graphs[B]["codes"]
