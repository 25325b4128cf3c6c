"""gqa_decode_attn on the GPU against the oracle: the tiny workload, the
32/8/128 workload at B in {1, 16, 64} with ragged kv_len in 234..400 in a
32768-slot cache, the long sweep up to 8192, garbage-tail invariance, closed
forms, split invariance and invalid kv_len handling."""

import numpy as np
import pytest
import torch

from oracle import attention as oattn
from fp8_transformer_step_amd import inputs, ops
from _helpers import TOL_BF16_ATTN, f32, from_dev_bf16, log, max_rel_err, need_gpu, to_dev_bf16

pytestmark = pytest.mark.gpu


def _garbage_cache(B, Hkv, cap, D, seed):
    """A cache of random bytes (NaN and Inf bf16 patterns included)."""
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    out = torch.empty((B, Hkv, cap, D), dtype=torch.int16, device="cuda")
    for b in range(B):
        out[b] = torch.randint(-32768, 32768, (Hkv, cap, D), dtype=torch.int32, device="cuda",
                               generator=g).to(torch.int16)
    return out.view(torch.bfloat16)


def _make(workload, B, Hq, Hkv, D, cap, kv, seed=0, tail_seed=1, extra=0):
    Lmax = int(kv.max())
    qb, kb, vb = inputs.attention_prefix(workload, B, Hq, Hkv, D, Lmax, extra=extra)
    kc = _garbage_cache(B, Hkv, cap, D, tail_seed)
    vc = _garbage_cache(B, Hkv, cap, D, tail_seed + 7)
    kd, vd = to_dev_bf16(kb), to_dev_bf16(vb)
    for b in range(B):
        L = int(kv[b])
        kc[b, :, :L] = kd[b, :, :L]
        vc[b, :, :L] = vd[b, :, :L]
    return qb, kb, vb, kc, vc


def _oracle(qb, kb, vb, kv):
    return oattn.gqa_decode_attention(f32(qb), f32(kb), f32(vb), kv)


def _run(qb, kc, vc, kv, hint, err=None):
    out = ops.gqa_decode_attn(to_dev_bf16(qb), kc, vc, torch.from_numpy(kv).cuda(), hint, err=err)
    torch.cuda.synchronize()
    return out


def test_tiny_workload():
    need_gpu()
    kv = np.array([37], np.int32)
    qb, kb, vb, kc, vc = _make(inputs.W_TINY, 1, 4, 1, 64, 128, kv)
    out = _run(qb, kc, vc, kv, 128)
    assert max_rel_err(from_dev_bf16(out), _oracle(qb, kb, vb, kv)) <= TOL_BF16_ATTN


@pytest.mark.parametrize("B", [1, 16, 64])
def test_qwen_shape_short_context(B):
    need_gpu()
    kv = inputs.kv_lengths(inputs.W_ATTN, B, 234, 400, extra=B)
    log(f"attn B={B} kv range {kv.min()}..{kv.max()}")
    qb, kb, vb, kc, vc = _make(inputs.W_ATTN, B, 32, 8, 128, 32768, kv, extra=B)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = _run(qb, kc, vc, kv, 400, err)
    e = max_rel_err(from_dev_bf16(out), _oracle(qb, kb, vb, kv))
    log(f"  max rel err {e:.3e}")
    assert int(err.item()) == 0
    assert e <= TOL_BF16_ATTN


@pytest.mark.parametrize("B,lo,hi", [(16, 234, 8192), (4, 8192, 8192), (8, 1024, 4096)])
def test_long_context_sweep(B, lo, hi):
    need_gpu()
    kv = inputs.kv_lengths(inputs.W_ATTN, B, lo, hi, extra=10 * B + hi)
    log(f"attn long B={B} kv range {kv.min()}..{kv.max()}")
    qb, kb, vb, kc, vc = _make(inputs.W_ATTN, B, 32, 8, 128, 32768, kv, extra=10 * B + hi)
    out = _run(qb, kc, vc, kv, hi)
    assert max_rel_err(from_dev_bf16(out), _oracle(qb, kb, vb, kv)) <= TOL_BF16_ATTN


def test_garbage_tail_invariance_and_split_invariance():
    need_gpu()
    B = 16
    kv = inputs.kv_lengths(inputs.W_ATTN, B, 234, 400, extra=99)
    qb, kb, vb, kc, vc = _make(inputs.W_ATTN, B, 32, 8, 128, 4096, kv, tail_seed=5, extra=99)
    base = _run(qb, kc, vc, kv, 400)
    # a different garbage tail, and a zero tail: bit-identical output
    _, _, _, kc2, vc2 = _make(inputs.W_ATTN, B, 32, 8, 128, 4096, kv, tail_seed=11, extra=99)
    assert torch.equal(base, _run(qb, kc2, vc2, kv, 400))
    kz, vz = torch.zeros_like(kc), torch.zeros_like(vc)
    for b in range(B):
        L = int(kv[b])
        kz[b, :, :L] = kc[b, :, :L]
        vz[b, :, :L] = vc[b, :, :L]
    assert torch.equal(base, _run(qb, kz, vz, kv, 400))
    # other split plans (the hint sets the chunking) stay within tolerance
    ref = _oracle(qb, kb, vb, kv)
    for hint in (401, 1000, 4096):
        assert max_rel_err(from_dev_bf16(_run(qb, kc, vc, kv, hint)), ref) <= TOL_BF16_ATTN


def test_closed_forms():
    need_gpu()
    B, cap = 4, 256
    kv = np.array([1, 1, 1, 1], np.int32)
    qb, kb, vb, kc, vc = _make(inputs.W_ATTN, B, 32, 8, 128, cap, kv, extra=5)
    out = _run(qb, kc, vc, kv, cap)
    # one position: the output is that position's V, exactly (bf16)
    want = torch.from_numpy(np.repeat(vb[:, :, 0], 4, axis=1).view(np.int16)).cuda().view(torch.bfloat16)
    assert torch.equal(out, want)
    # zero query: the mean of the V prefix; kv_len = cap is valid
    kv = np.array([cap, 17, 100, 255], np.int32)
    qb, kb, vb, kc, vc = _make(inputs.W_ATTN, B, 32, 8, 128, cap, kv, extra=6)
    qz = np.zeros_like(qb)
    out = from_dev_bf16(_run(qz, kc, vc, kv, cap))
    mean = np.stack([np.repeat(f32(vb)[b, :, :kv[b]].mean(axis=1), 4, axis=0) for b in range(B)])
    assert max_rel_err(out, mean) <= TOL_BF16_ATTN


def test_gqa_matches_explicit_head_repeat():
    """Equality with attention over explicitly repeated KV heads (the
    repeat_interleave reference of the KV-cache page)."""
    need_gpu()
    B = 2
    kv = np.array([300, 391], np.int32)
    qb, kb, vb, kc, vc = _make(inputs.W_ATTN, B, 32, 8, 128, 512, kv, extra=31)
    out = from_dev_bf16(_run(qb, kc, vc, kv, 400))
    kr, vr = np.repeat(f32(kb), 4, axis=1), np.repeat(f32(vb), 4, axis=1)
    ref = oattn.gqa_decode_attention(f32(qb), kr, vr, kv)      # Hkv == Hq: one head each
    assert max_rel_err(out, ref) <= TOL_BF16_ATTN


@pytest.mark.parametrize("hint", [256, 16])
def test_invalid_kv_len_sets_flag_and_zeroes(hint):
    """hint 256 splits the prefix (64-position chunks) and merges; hint 16 is
    a single chunk whose kernel writes the output itself."""
    need_gpu()
    B, cap = 3, 256
    kv = np.array([10, 10, 10], np.int32)
    qb, kb, vb, kc, vc = _make(inputs.W_ATTN, B, 32, 8, 128, cap, kv, extra=41)
    bad = np.array([10, 0, 257], np.int32)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = _run(qb, kc, vc, bad, hint, err)
    assert int(err.item()) == ops.DEV_KVLEN_RANGE
    assert not out[1].float().abs().sum().item() and not out[2].float().abs().sum().item()
    ref = _oracle(qb[:1], kb[:1], vb[:1], kv[:1])
    assert max_rel_err(from_dev_bf16(out[:1]), ref) <= TOL_BF16_ATTN


@pytest.mark.parametrize("G", [4, 2])
def test_single_chunk_short_prefix(G):
    """Prefixes of at most 16 positions (the fast AR's few-slot cache): one
    chunk, no merge, output written by the split kernel."""
    need_gpu()
    B, Hkv, cap = 64, 8, 16
    kv = (np.arange(B) % 9 + 1).astype(np.int32)
    qb, kb, vb, kc, vc = _make(inputs.W_ATTN, B, Hkv * G, Hkv, 128, cap, kv, extra=50 + G)
    out = from_dev_bf16(_run(qb, kc, vc, kv, 9))
    assert max_rel_err(out, _oracle(qb, kb, vb, kv)) <= TOL_BF16_ATTN


def test_balanced_split_mixed_and_invalid_lengths():
    """Batches of 16+ take the balanced split: equal position ranges over the
    concatenated prefixes.  Mix one-position prefixes, the full capacity and
    invalid lengths (zero output, error flag) in one batch."""
    need_gpu()
    B, cap = 32, 1024
    kv = inputs.kv_lengths(inputs.W_ATTN, B, 1, cap, extra=201)
    kv[:4] = [1, cap, 1, 2]
    qb, kb, vb, kc, vc = _make(inputs.W_ATTN, B, 32, 8, 128, cap, kv, extra=201)
    bad = kv.copy()
    bad[5], bad[17] = 0, cap + 1
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = _run(qb, kc, vc, bad, cap, err)
    assert int(err.item()) == ops.DEV_KVLEN_RANGE
    assert not out[5].float().abs().sum().item() and not out[17].float().abs().sum().item()
    keep = [b for b in range(B) if b not in (5, 17)]
    ref = _oracle(qb[keep], kb[keep], vb[keep], kv[keep])
    assert max_rel_err(from_dev_bf16(out[keep]), ref) <= TOL_BF16_ATTN


def _balanced_taken(ws, kv):
    """The balanced split leaves a table of (first record, record count) int32
    pairs at the start of its workspace; a chunked split stores fp32 records
    there instead.  Every valid prefix has at least one record and at most
    as many as it has positions."""
    t = ws[: 8 * len(kv)].view(torch.int32).view(-1, 2).cpu().numpy()
    return bool(np.all(t[:, 1] >= 1) and np.all(t[:, 1] <= kv) and np.all(t[:, 0] >= 0))


@pytest.mark.parametrize("case", ["short_many", "one_long", "more_ranges_than_positions"])
def test_balanced_split_pieces_across_many_sequences(case):
    """Ranges that span many sequences (tiny prefixes), and batches whose
    prefixes total fewer positions than the balanced split has workgroups
    (every prefix one position, or a few), so that there are more workgroup
    slots than positions."""
    need_gpu()
    if case == "short_many":
        B, cap = 64, 1024
        kv = np.ones(B, np.int32)
    elif case == "one_long":
        B, cap = 20, 2048
        kv = (np.arange(B) % 3 + 1).astype(np.int32)
        kv[13] = cap
    else:
        B, cap = 16, 1024
        kv = (np.arange(B) % 4 + 2).astype(np.int32)
    qb, kb, vb, kc, vc = _make(inputs.W_ATTN, B, 32, 8, 128, cap, kv, extra=202)
    ws = torch.full((ops.attn_workspace_bytes(B, 32, 128, cap),), 0xFF, dtype=torch.uint8, device="cuda")
    out = ops.gqa_decode_attn(to_dev_bf16(qb), kc, vc, torch.from_numpy(kv).cuda(), cap, workspace=ws)
    torch.cuda.synchronize()
    assert _balanced_taken(ws, kv), "the balanced split did not run"
    assert max_rel_err(from_dev_bf16(out), _oracle(qb, kb, vb, kv)) <= TOL_BF16_ATTN


@pytest.mark.parametrize("shape", [(16, 32, 8, 128, 5), (16, 4, 1, 64, 37)])
def test_balanced_split_reused_workspace_few_positions(shape):
    """A workspace reused across calls keeps what earlier calls (or garbage)
    left there: here it is first filled with 0xFF bytes (NaN records), then a
    call at long prefixes leaves its own records, and a call whose prefixes
    total fewer positions than the balanced split has workgroups must still
    give the oracle's output, bit-identical to the same call on a fresh
    workspace."""
    need_gpu()
    B, Hq, Hkv, D, L = shape
    cap = 1024
    kv = np.full(B, L, np.int32)
    qb, kb, vb, kc, vc = _make(inputs.W_ATTN, B, Hq, Hkv, D, cap, kv, extra=300 + L)
    ws = torch.full((ops.attn_workspace_bytes(B, Hq, D, cap),), 0xFF, dtype=torch.uint8, device="cuda")
    kvd = torch.from_numpy(kv).cuda()
    out = ops.gqa_decode_attn(to_dev_bf16(qb), kc, vc, kvd, cap, workspace=ws)
    torch.cuda.synchronize()
    assert _balanced_taken(ws, kv), "the balanced split did not run"
    ref = _oracle(qb, kb, vb, kv)
    assert max_rel_err(from_dev_bf16(out), ref) <= TOL_BF16_ATTN
    # records of a long-prefix call, then the short call again on that workspace
    long_kv = torch.full((B,), cap, dtype=torch.int32, device="cuda")
    ops.gqa_decode_attn(to_dev_bf16(qb), kc, vc, long_kv, cap, workspace=ws)
    out2 = ops.gqa_decode_attn(to_dev_bf16(qb), kc, vc, kvd, cap, workspace=ws)
    fresh = ops.gqa_decode_attn(to_dev_bf16(qb), kc, vc, kvd, cap)
    torch.cuda.synchronize()
    assert torch.equal(out, out2) and torch.equal(out, fresh)


@pytest.mark.timeout(600)
def test_b64_long_context_sampled_rows():
    """B = 64, kv U[234, 8192], the full head configuration: every sequence
    runs in one launch; the oracle checks sampled sequences (first, last,
    longest, shortest and a spread)."""
    need_gpu()
    B, hi = 64, 8192
    kv = inputs.kv_lengths(inputs.W_ATTN, B, 234, hi, extra=900)
    log(f"attn B=64 kv range {kv.min()}..{kv.max()}")
    qb, kb, vb, kc, vc = _make(inputs.W_ATTN, B, 32, 8, 128, hi, kv, extra=900)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = from_dev_bf16(_run(qb, kc, vc, kv, hi, err))
    rows = sorted({0, 13, 29, 47, B - 1, int(np.argmax(kv)), int(np.argmin(kv))})
    ref = _oracle(qb[rows], kb[rows], vb[rows], kv[rows])
    e = max_rel_err(out[rows], ref)
    log(f"  rows {rows} kv {[int(kv[b]) for b in rows]}: max rel err {e:.3e}")
    assert int(err.item()) == 0
    assert e <= TOL_BF16_ATTN
