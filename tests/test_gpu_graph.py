"""The decode step captured into a HIP graph (torch.cuda.graph) replays like
the eager call: the library allocates, frees and synchronises nothing and
records no memsets, and its workspace control words are back at zero after
every call, so each replay starts from the same state.  Replays are
interleaved with eager work and eager calls, and every replay is compared
bit for bit with the eager result (codes, logits and the caches it appends
to)."""

import pytest
import torch

from fp8_transformer_step_amd import model, ops
from _helpers import need_gpu

pytestmark = pytest.mark.gpu


def test_step_graph_replays_match_eager():
    need_gpu()
    host = model.HostModel(model.scaled(model.TINY, batch=24, n_heads=8))
    c = host.cfg
    B, C, V = c.batch, c.n_codebooks, c.codebook_size
    dm = model.device_model(host)
    kv, ks, vs = model.device_kv(host)
    prev = torch.from_numpy(host.prev_codes).cuda()
    ws = dm.new_workspace(B, kv.c.max_kv_len_hint, prev.device)
    codes = torch.empty((B, C), dtype=torch.int32, device="cuda")
    logits = torch.empty((C, B, V), dtype=torch.float32, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")

    def step():
        ops.dual_ar_decode_step(dm, kv, prev, codes=codes, logits_tap=logits, workspace=ws, err=err)

    step()
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    ref_codes, ref_logits = codes.clone(), logits.clone()
    ref_k = [k.view(torch.int16).clone() for k in ks]
    ref_v = [v.view(torch.int16).clone() for v in vs]

    side = torch.cuda.Stream()                   # warm-up off the capture stream, as torch asks
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()

    def check(what):
        assert torch.equal(codes, ref_codes), what
        assert torch.equal(logits, ref_logits), what
        for s in range(c.kv_sets):
            assert torch.equal(ks[s].view(torch.int16), ref_k[s]), what
            assert torch.equal(vs[s].view(torch.int16), ref_v[s]), what
        assert int(err.item()) == 0, what

    for rep in range(4):
        codes.fill_(-1)                          # eager work between replays
        logits.zero_()
        graph.replay()
        torch.cuda.synchronize()
        check(f"replay {rep}")
        if rep % 2:
            step()                               # an eager call between replays
            torch.cuda.synchronize()
            check(f"eager call after replay {rep}")
