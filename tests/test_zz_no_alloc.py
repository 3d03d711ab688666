"""c2kv_attn_decode_noalloc (the decode step whose split partials live in the
library's static per-GPU scratch) against c2kv_attn_decode with a caller
workspace: two calls in a row through the C ABI, the second with a smaller
input, each compared bit for bit (same kernels and split plan), outputs,
log-sum-exp and the appended cache rows.  Also: it runs without the library
allocating, and a decode that needs more split scratch than the array holds
is rejected before any launch."""
import pytest
import torch



@pytest.fixture(scope="module")
def c2kv():
    import compressed_composable_kv_amd as m
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return m


def _case(seed, R, hq, hkv, d, lens, dtype):
    g = torch.Generator().manual_seed(seed)
    cap = max(lens) + 8
    ck = torch.randn((R, hkv, cap, d), generator=g).to(dtype).cuda()
    cv = torch.randn((R, hkv, cap, d), generator=g).to(dtype).cuda()
    q = torch.randn((R, hq, d), generator=g).to(dtype).cuda()
    kn = torch.randn((R, hkv, d), generator=g).to(dtype).cuda()
    vn = torch.randn((R, hkv, d), generator=g).to(dtype).cuda()
    pos = [3 * x + 11 for x in lens]
    return ck, cv, q, kn, vn, pos


def _compare(c2kv, seed, R, hq, hkv, d, lens, dtype, theta):
    ck, cv, q, kn, vn, pos = _case(seed, R, hq, hkv, d, lens, dtype)
    ck2, cv2 = ck.clone(), cv.clone()
    nbytes = c2kv.workspace_size_decode(lens, hq, hkv, d, dtype)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    o_ref, lse_ref = c2kv.attn_decode(q, kn, vn, ck, cv, lens, pos, theta, return_lse=True, workspace=ws)
    o = torch.full_like(q, float("nan"))
    lse = torch.full((R, hq), float("nan"), dtype=torch.float32, device="cuda")
    c2kv.attn_decode_noalloc(q, kn, vn, ck2, cv2, lens, pos, theta, out=o, lse_out=lse)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16 if dtype == torch.bfloat16 else torch.int32),
                       o_ref.view(torch.int16 if dtype == torch.bfloat16 else torch.int32))
    assert torch.equal(lse.view(torch.int32), lse_ref.view(torch.int32))
    assert torch.equal(ck2, ck) and torch.equal(cv2, cv)
    return nbytes


@pytest.mark.gpu
def test_noalloc_decode_equals_workspace_decode_twice(c2kv):
    print("noalloc: call 1 (4 requests, 32/8 heads, d 128, bf16)", flush=True)
    n1 = _compare(c2kv, 1, 4, 32, 8, 128, [3000, 1500, 700, 5000], torch.bfloat16, 5e5)
    assert n1 > 256, "the first call must use split partials"
    print("noalloc: call 2 (2 requests, 8/2 heads, d 64, fp32, smaller)", flush=True)
    n2 = _compare(c2kv, 2, 2, 8, 2, 64, [400, 90], torch.float32, 1e4)
    assert n2 < n1


@pytest.mark.gpu
def test_noalloc_decode_graph_capture(c2kv):
    """Captured in a HIP graph with every buffer made beforehand (the caller
    the entry point is for), replayed three times with eager work between."""
    ck, cv, q, kn, vn, pos = _case(3, 2, 28, 4, 128, [2000, 900], torch.bfloat16)
    lens = [2000, 900]
    o = torch.empty_like(q)
    ref_k, ref_v = ck.clone(), cv.clone()
    o_ref, _ = c2kv.attn_decode(q, kn, vn, ref_k, ref_v, lens, pos, 1e6)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        c2kv.attn_decode_noalloc(q, kn, vn, ck, cv, lens, pos, 1e6, out=o)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        c2kv.attn_decode_noalloc(q, kn, vn, ck, cv, lens, pos, 1e6, out=o)
    for _ in range(3):
        o.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref)
    assert torch.equal(ck, ref_k) and torch.equal(cv, ref_v)


def test_noalloc_decode_validation_before_any_hip_call():
    """Invalid arguments are rejected with the documented status before the
    scratch lookup or any launch (runs without a GPU)."""
    import ctypes
    from compressed_composable_kv_amd import _lib
    lib = _lib.load()
    FAKE = 0x10000

    def call(lens, pos, cap=100, hq=8, hkv=2, d=128, q=FAKE):
        arr = lambda v: (ctypes.c_int32 * len(v))(*v)  # noqa: E731
        return lib.c2kv_attn_decode_noalloc(q, FAKE, FAKE, FAKE, FAKE, cap, arr(lens), arr(pos), len(lens), hq, hkv,
                                            d, 1e6, FAKE, None, 0, None)
    assert call([100], [5]) == 4          # capacity: no room for the new row
    assert call([-1], [5]) == 1
    assert call([10], [5], hq=3) == 1
    assert call([10], [5], q=0) == 1
    assert call([10], [5], d=96) == 2

