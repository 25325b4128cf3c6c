"""The decode step captured once per batch bucket (graphs.StepGraphs): every
bucket's replay equals the eager step at that batch bit for bit (codes,
logits of the eager call, caches), a batch between buckets runs on the next
bucket up and returns its first rows, and replays of different buckets
interleave without disturbing each other."""

import pytest
import torch

from fp8_transformer_step_amd import graphs, model, ops
from _helpers import need_gpu

pytestmark = pytest.mark.gpu


def test_bucket_replays_match_eager_steps():
    need_gpu()
    host = model.HostModel(model.scaled(model.TINY, batch=24, n_heads=8))
    c = host.cfg
    dm = model.device_model(host)
    kv, ks, vs = model.device_kv(host)
    prev_all = torch.from_numpy(host.prev_codes).cuda()
    sg = graphs.StepGraphs(dm, kv, buckets=(1, 3, 8, 24, 64))
    assert sg.buckets == [1, 3, 8, 24]                 # 64 is above the KV state's rows
    eager = {}
    for B in sg.buckets:
        ws = dm.new_workspace(B, kv.c.max_kv_len_hint)
        err = torch.zeros(1, dtype=torch.int32, device="cuda")
        eager[B] = ops.dual_ar_decode_step(dm, kv, prev_all[:B].contiguous(), workspace=ws, err=err).clone()
        torch.cuda.synchronize()
        assert int(err.item()) == 0
    k_ref = [k.view(torch.int16).clone() for k in ks]
    for rep in range(2):
        for b in (1, 2, 3, 5, 8, 17, 24):
            B = sg.bucket_for(b)
            sg.graphs[B]["prev"].copy_(prev_all[:B])       # the bucket's full input, as in the eager run
            out = sg.step(prev_all[:b]).clone()
            torch.cuda.synchronize()
            assert torch.equal(out, eager[B][:b]), (rep, b, B)
    assert int(sg.err.item()) == 0
    for s in range(c.kv_sets):                          # replays rewrite the same cache slots
        assert torch.equal(ks[s].view(torch.int16), k_ref[s])
    with pytest.raises(ValueError):
        sg.bucket_for(25)


def _parts(cache):
    """The byte tensors of a cache (bf16, or MXFP8 codes and exponents)."""
    return [cache.q, cache.e] if isinstance(cache, ops.MxKvCache) else [cache.view(torch.int16)]


@pytest.mark.parametrize("mx", [False, True], ids=["bf16_kv", "mxfp8_kv"])
def test_padding_rows_leave_their_cache_slots_alone(mx):
    """A batch of 5 on the bucket of 8: rows 5..7 hold other sequences' codes;
    the replay must leave their cache rows bit-identical (the step appends
    K/V for live rows only, in either cache format) and give rows 0..4 the
    codes of an eager step over the same 8 rows."""
    need_gpu()
    host = model.HostModel(model.scaled(model.TINY, batch=24, n_heads=8))
    c = host.cfg
    dm = model.device_model(host)
    kv, ks, vs = model.device_kv(host, mx=mx)
    prev_all = torch.from_numpy(host.prev_codes).cuda()
    sg = graphs.StepGraphs(dm, kv, buckets=(8, 24))
    other = (prev_all[:8] + 17) % c.codebook_size          # different codes in the padding rows
    sg.graphs[8]["prev"].copy_(other)
    before_k = [[t.clone() for t in _parts(k)] for k in ks]
    before_v = [[t.clone() for t in _parts(v)] for v in vs]
    out = sg.step(prev_all[:5]).clone()
    torch.cuda.synchronize()
    assert int(sg.err.item()) == 0
    for s in range(c.kv_sets):
        for now, before in zip(_parts(ks[s]) + _parts(vs[s]), before_k[s] + before_v[s]):
            assert torch.equal(now[5:8], before[5:8])
    changed = any(not torch.equal(_parts(ks[s])[0][:5], before_k[s][0][:5]) for s in range(c.kv_sets))
    assert changed                                       # the live rows did append their K/V
    full = torch.cat([prev_all[:5], other[5:8]]).contiguous()
    ref = ops.dual_ar_decode_step(dm, kv, full)
    torch.cuda.synchronize()
    assert torch.equal(out, ref[:5])
