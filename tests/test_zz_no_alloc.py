"""The entry point that allocates nothing (gqa_decode_noalloc), through the
C ABI: two calls in a row -- the second with a smaller input -- each give
the bits of gqa_decode_ex with the same options on the same inputs, and
match the float64 oracle within the bf16 tolerance (2e-3).  No device memory
is allocated by the calls.  Then the same entry point, and a caller
workspace's gqa_workspace_clear + decode, captured in HIP graphs and
replayed."""
import ctypes
import math

import numpy as np
import pytest
import torch

import gqa_inputs as gi

pytestmark = pytest.mark.gpu
TOL = 2e-3


@pytest.fixture(scope="module")
def gqa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import grouped_query_attention_decode_amd as m
    m.load_library()
    return m


def _call_noalloc(gqa, x, out, workgroups=0):
    lib = gqa.load_library()
    shape = gqa.shape_of(x["q"], x["k"])
    opts = gqa.Options()
    opts.workgroups = workgroups
    st = lib.gqa_decode_noalloc(ctypes.byref(shape), x["q"].data_ptr(), x["k"].data_ptr(), x["v"].data_ptr(),
                                x["seq_lens"].data_ptr(), ctypes.c_float(1.0 / math.sqrt(x["q"].shape[3])),
                                out.data_ptr(), ctypes.byref(opts),
                                ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    return st


CASES = [
    # a larger call (MQA-shaped: 32 rows per KV head, split segments merged by
    # the combine kernel), then a smaller ragged GQA-8 call (in-kernel merges)
    dict(B=16, H=32, G=1, D=128, T=2048, sq=1, seq_lens=[2048] * 16, seed=901),
    dict(B=3, H=32, G=8, D=128, T=1000, sq=1, seq_lens=[1000, 517, 1], seed=902),
    # and an fp16 cache, smaller again
    dict(B=2, H=32, G=8, D=64, T=500, sq=1, seq_lens=[500, 77], seed=904, dtype="f16"),
]


def test_noalloc_matches_decode_ex_twice(gqa):
    import oracle
    oracle.build(force=False)
    # the first call on a device resolves the scratch array's address (the
    # HIP runtime may set up state of its own then); later calls allocate
    # nothing at all
    w = gi.make_custom(1, 8, 2, 64, 40, 1, dtype="bf16", seed=900, seq_lens=[40], device="cuda")
    wout = torch.empty(w["q"].shape, dtype=torch.float32, device="cuda")
    assert _call_noalloc(gqa, w, wout) == gqa.GQA_OK
    torch.cuda.synchronize()
    for i, c in enumerate(CASES):
        x = gi.make_custom(c["B"], c["H"], c["G"], c["D"], c["T"], c["sq"], dtype=c.get("dtype", "bf16"),
                           seed=c["seed"], seq_lens=c["seq_lens"], device="cuda")
        want = gqa.decode(x["q"], x["k"], x["v"], x["seq_lens"])
        out = torch.full(x["q"].shape, float("nan"), dtype=torch.float32, device="cuda")
        torch.cuda.synchronize()
        free0 = torch.cuda.mem_get_info()[0]   # after the reference call grew the library's workspace
        assert _call_noalloc(gqa, x, out) == gqa.GQA_OK, gqa.load_library().gqa_last_error()
        torch.cuda.synchronize()
        assert torch.cuda.mem_get_info()[0] == free0        # nothing allocated
        assert torch.equal(out, want), "case %d: not the bits of gqa_decode_ex" % i
        # and the oracle on two whole sequences
        for b in (0, c["B"] - 1):
            xb = {k: v[b:b + 1].cpu() for k, v in x.items()}
            ref = oracle.decode_f64(xb["q"], xb["k"], xb["v"], xb["seq_lens"], 1.0 / math.sqrt(c["D"]), threads=8)
            err = float(np.abs(out[b:b + 1].double().cpu().numpy() - ref).max())
            assert err <= TOL, (i, b, err)
        del x, want, out


def test_noalloc_refuses_a_workspace_beyond_its_scratch(gqa):
    x = gi.make_custom(2, 32, 8, 128, 64, 64, dtype="bf16", seed=903, seq_lens=[64, 64], device="cuda")
    out = torch.zeros(x["q"].shape, dtype=torch.float32, device="cuda")
    st = _call_noalloc(gqa, x, out, workgroups=65536)
    assert st == gqa.GQA_ERR_ALLOC
    assert "scratch" in gqa.load_library().gqa_last_error().decode()
    # the binding says the same
    with pytest.raises(gqa.GqaError):
        gqa.decode_noalloc(x["q"], x["k"], x["v"], x["seq_lens"], out=out, workgroups=65536)
    # and a grid that fits works through the binding
    got = gqa.decode_noalloc(x["q"], x["k"], x["v"], x["seq_lens"], out=out)
    want = gqa.decode(x["q"], x["k"], x["v"], x["seq_lens"])
    torch.cuda.synchronize()
    assert torch.equal(got, want)


# HIP graph capture: the callers this entry point is for.  Replays give the
# eager call's bits, with other eager work -- including eager calls that
# share the scratch -- between replays (no memset node is recorded: the
# counters are cleared by a kernel).

def _inputs(B, H, G, D, T, seq_lens, seed):
    return gi.make_custom(B, H, G, D, T, 1, dtype="bf16", seed=seed, seq_lens=seq_lens, device="cuda")


@pytest.mark.parametrize("case", [
    dict(B=8, H=32, G=1, D=128, T=2048, seq_lens=[2048, 1900, 1500, 1024, 700, 333, 64, 1]),   # 32 rows: combine kernel
    dict(B=4, H=32, G=8, D=64, T=1024, seq_lens=[1024, 1000, 517, 0]),                        # 4 rows, row-split, in-kernel merge
], ids=["mqa_like", "gqa8_small"])
def test_noalloc_graph_replays(gqa, case):
    x = _inputs(case["B"], case["H"], case["G"], case["D"], case["T"], case["seq_lens"], 700 + case["D"])
    y = _inputs(case["B"], case["H"], case["G"], case["D"], case["T"], case["seq_lens"][::-1], 800 + case["D"])
    want = gqa.decode_noalloc(x["q"], x["k"], x["v"], x["seq_lens"],    # first call: scratch address resolved
                              out=torch.empty(x["q"].shape, dtype=torch.float32, device="cuda"))
    want_y = gqa.decode_noalloc(y["q"], y["k"], y["v"], y["seq_lens"],
                                out=torch.empty(y["q"].shape, dtype=torch.float32, device="cuda"))
    # the eager library-workspace call agrees to rounding (same plan: same bits)
    assert torch.equal(gqa.decode(x["q"], x["k"], x["v"], x["seq_lens"]), want)
    torch.cuda.synchronize()
    out = torch.full_like(want, float("nan"))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        gqa.decode_noalloc(x["q"], x["k"], x["v"], x["seq_lens"], out=out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        gqa.decode_noalloc(x["q"], x["k"], x["v"], x["seq_lens"], out=out)
    for r in range(4):
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, want), "replay %d" % r
        # an eager call with other inputs shares the scratch between replays
        oy = torch.empty_like(want_y)
        assert torch.equal(gqa.decode_noalloc(y["q"], y["k"], y["v"], y["seq_lens"], out=oy), want_y)
        torch.cuda.synchronize()


def test_workspace_clear_and_decode_in_a_graph(gqa):
    x = _inputs(4, 32, 8, 128, 1536, [1536, 1200, 77, 1], 901)
    want = gqa.decode(x["q"], x["k"], x["v"], x["seq_lens"])
    need = gqa.workspace_bytes(gqa.shape_of(x["q"], x["k"]))
    ws = torch.full((need,), 5, dtype=torch.uint8, device="cuda")
    out = torch.empty_like(want)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        gqa.workspace_clear(ws)
        gqa.decode(x["q"], x["k"], x["v"], x["seq_lens"], out=out, workspace=ws)
    for r in range(4):
        out.fill_(float("nan"))
        ws[: 1 << 20].fill_(3)                # garbage counters before every replay
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, want), "replay %d" % r
        assert int(ws[: 1 << 20].view(torch.int32).abs().sum().item()) == 0
