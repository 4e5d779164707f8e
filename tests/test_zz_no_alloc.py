"""tsa_attention_fwd_noalloc (the forward with the library's static scratch
instead of a workspace) against tsa_attention_fwd on the same inputs, through
the C ABI: three calls in a row, each smaller than the one before, so stale
scratch contents of a larger call would show in a smaller one.  The regular
entry point gets a workspace filled with garbage bytes, so neither path can
rely on memory that happens to be zero.  Both must agree bit for bit (they run
the same kernels) and stay within the oracle tolerance."""
import numpy as np
import pytest

import oracle
import workloads as W
from gpu_util import compare, say, small_workload, to_dev_mask, torch_or_skip

pytestmark = pytest.mark.gpu


def _banded(w, seed):
    # key tiles within 200 keys of the tile's rows, kept w.p. 0.5 (most 128-key
    # chunks of a 256-row group are not needed: the chunk-skipping kernel runs
    # and reads the chunk words of the scratch)
    rng = np.random.default_rng(seed)
    keep = np.zeros((w.B, w.H, w.T_q, w.T_k), dtype=bool)
    for b in range(w.B):
        for h in range(w.H):
            for i in range(w.T_q):
                r0 = i * w.M
                lo, hi = max(0, (r0 - 200) // w.N), min(w.T_k, (r0 + w.M + 200) // w.N + 1)
                keep[b, h, i, lo:hi] = rng.random(hi - lo) < 0.5
                keep[b, h, i, min(w.T_k - 1, r0 // w.N)] = True
    return W.pack_bits(keep)


def _case(w, bits, label):
    import torch

    import tile_sparse_attention_amd as T
    say(f"no-alloc {label}: B={w.B} H={w.H} L={w.L} d={w.d} {w.M}x{w.N} {w.dtype}")
    qh, kh, vh = W.make_qkv(w)
    q, k, v = qh.cuda(), kh.cuda(), vh.cuda()
    m = to_dev_mask(bits)
    pr = T.problem(w.B, w.H, w.L, w.d, w.M, w.N, T.DTYPE_BF16 if w.dtype == "bf16" else T.DTYPE_F32)
    ws = torch.full((T.workspace_size(T.OP_ATTENTION_FWD, pr),), 0xFF, dtype=torch.uint8, device="cuda")
    o_ref, l_ref = T.attention_fwd(q, k, v, m, w.M, w.N, w.scale, return_lse=True, workspace=ws)
    o = torch.full_like(q, float("nan"))
    lse = torch.full((w.B, w.H, w.L), float("nan"), dtype=torch.float32, device="cuda")
    T.attention_fwd_noalloc(q, k, v, m, w.M, w.N, w.scale, out=o, lse=lse)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref), f"{label}: O differs from tsa_attention_fwd"
    assert torch.equal(lse, l_ref), f"{label}: LSE differs from tsa_attention_fwd"
    ro, rl = oracle.attention(qh, kh, vh, bits, w.M, w.N, w.scale)
    compare(f"no-alloc {label}", o.float().cpu().numpy(), ro, w.dtype, lse.cpu().numpy(), rl)


def test_noalloc_matches_workspace_entry_point():
    torch_or_skip()
    w1 = small_workload("na1", 5000, 128, 16, 8, H=3, seed=71)
    _case(w1, _banded(w1, 1), "call 1 (bf16 16x8, chunk skipping)")
    w2 = small_workload("na2", 1200, 128, 16, 16, H=2, seed=72)
    _case(w2, _banded(w2, 2), "call 2 (smaller: bf16 16x16)")
    w3 = small_workload("na3", 512, 64, 16, 16, dtype="f32", H=2, p=0.5, seed=73)
    _case(w3, W.mask_bits(w3), "call 3 (smaller: f32 d64 16x16)")


def test_noalloc_rejects_problems_beyond_its_scratch():
    torch = torch_or_skip()
    import tile_sparse_attention_amd as T
    # 40 heads at L = 32760, d = 128: the workspace is about 338 MB
    B, H, L, d = 1, 40, 32760, 128
    q = torch.zeros((B, H, L, d), dtype=torch.bfloat16, device="cuda")
    k, v, o = torch.zeros_like(q), torch.zeros_like(q), torch.empty_like(q)
    m = torch.zeros((B, H, L // 16 + 1, T.mask_row_words(L, 8)), dtype=torch.int32, device="cuda")
    with pytest.raises(T.TsaError) as e:
        T.attention_fwd_noalloc(q, k, v, m, 16, 8, out=o)
    assert e.value.status == T.ERR_UNSUPPORTED and "scratch" in e.value.detail


def test_noalloc_forward_replays_in_a_captured_graph():
    """The use the entry point is for: one call captured in a HIP graph (after
    an eager call has looked up the scratch's address), replayed three times
    with eager no-alloc calls on another problem in between, which overwrite
    the shared scratch; every replay must equal the eager result bit for bit."""
    torch = torch_or_skip()
    import tile_sparse_attention_amd as T
    w = small_workload("nag", 3000, 128, 16, 8, H=2, seed=74)
    say("no-alloc graph capture: bf16 16x8 L=3000, three replays")
    qh, kh, vh = W.make_qkv(w)
    q, k, v = qh.cuda(), kh.cuda(), vh.cuda()
    m = to_dev_mask(_banded(w, 4))
    o_ref, l_ref = T.attention_fwd(q, k, v, m, w.M, w.N, w.scale, return_lse=True)
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.L), dtype=torch.float32, device="cuda")
    T.attention_fwd_noalloc(q, k, v, m, w.M, w.N, w.scale, out=o, lse=lse)
    # another problem for the eager calls between the replays
    w2 = small_workload("nag2", 1500, 128, 16, 16, H=3, seed=75)
    q2, k2, v2 = (x.cuda() for x in W.make_qkv(w2))
    m2 = to_dev_mask(W.mask_bits(w2))
    o2 = torch.empty_like(q2)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        T.attention_fwd_noalloc(q, k, v, m, w.M, w.N, w.scale, out=o, lse=lse)
    torch.cuda.synchronize()
    for i in range(3):
        o.fill_(float("nan"))
        lse.fill_(float("nan"))
        T.attention_fwd_noalloc(q2, k2, v2, m2, w2.M, w2.N, w2.scale, out=o2)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref), f"replay {i}: O differs"
        assert torch.equal(lse, l_ref), f"replay {i}: LSE differs"
