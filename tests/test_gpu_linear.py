"""GPU parity: the QLoRA linear forward and backward against the float64
oracle (relative Frobenius <= 5e-3 and max abs <= 2e-2 rms), plus exactness
probes that pin the in-GEMM dequantization to the standalone one."""
import numpy as np
import pytest
import torch

from oracle import nf4
from tests.helpers import (OracleLayer, assert_close, bf16_to_host_bits, bf16_to_host_f64, say,
                           to_dev_bf16, to_dev_f32)
from workloads import WORKLOADS, make_layer, random_bf16, random_weights, workload_layer

pytestmark = pytest.mark.gpu


def run_layer(inp, alpha, m=None, want_bwd=True):
    import bit_nf4_quantized_13_amd as q
    x = inp.x if m is None else inp.x[:m]
    w = q.qlora_nf4_quantize(to_dev_f32(inp.w0))
    xd, ad, bd = to_dev_bf16(x), to_dev_bf16(inp.a), to_dev_bf16(inp.b)
    y, u = q.qlora_linear_fwd(w, xd, ad, bd, alpha)
    out = {"y": bf16_to_host_f64(y), "u": u.cpu().numpy().astype(np.float64)}
    if want_bwd:
        dyd = to_dev_bf16(inp.dy if m is None else inp.dy[:m])
        dx, da, db = q.qlora_linear_bwd(w, xd, dyd, ad, bd, alpha, u=u)
        out.update(dx=bf16_to_host_f64(dx), da=da.cpu().numpy().astype(np.float64),
                   db=db.cpu().numpy().astype(np.float64))
    torch.cuda.synchronize()
    return out


def check_layer(inp, alpha, name, m=None, want_bwd=True, bf16_rounding_allowance=False):
    """bf16_rounding_allowance: only for off-workload edge cases whose outputs
    are so heavy-tailed that bf16 output rounding alone exceeds 2e-2 rms."""
    say(f"linear {name} d,k={inp.w0.shape} M={m or inp.x.shape[0]} r={inp.a.shape[0]}")
    got = run_layer(inp, alpha, m, want_bwd)
    ref = OracleLayer(inp.w0)
    x = inp.x if m is None else inp.x[:m]
    y, u = ref.forward(x, inp.a, inp.b, alpha)
    assert_close(got["u"], u, f"{name} U")
    assert_close(got["y"], y, f"{name} Y", bf16_output=bf16_rounding_allowance)
    if want_bwd:
        dy = inp.dy if m is None else inp.dy[:m]
        dx, da, db = ref.backward(x, dy, inp.a, inp.b, alpha)
        assert_close(got["dx"], dx, f"{name} dX", bf16_output=bf16_rounding_allowance)
        assert_close(got["da"], da, f"{name} dA")
        assert_close(got["db"], db, f"{name} dB")


def test_single_layer_workload():
    wl = WORKLOADS["single"]
    check_layer(workload_layer("single"), wl.alpha, "single")


@pytest.mark.parametrize("m,d,k,r", [(1, 256, 512, 8), (300, 320, 192, 8), (257, 512, 320, 1),
                                     (64, 264, 128, 7), (130, 256, 256, 33), (33, 512, 1024, 64),
                                     (20, 128, 256, 128), (16, 200, 448, 33), (3, 136, 1088, 16),
                                     (5, 4104, 4096, 16), (16, 64, 64, 1), (16, 1000, 2048, 16),
                                     (2, 4104, 256, 16), (1, 16408, 256, 16), (16, 16408, 512, 8),
                                     (700, 328, 192, 8), (1030, 200, 1088, 16), (1100, 4104, 320, 4),
                                     (1100, 5512, 256, 8), (300, 320, 192, 33), (600, 264, 1088, 64),
                                     (260, 200, 448, 128), (1030, 136, 4096, 17),
                                     (1100, 6600, 320, 8), (1100, 264, 6592, 8), (100, 264, 1024, 16),
                                     (200, 1032, 2048, 8)])
def test_shapes_ranks_and_ragged_tiles(m, d, k, r):
    """Ranks, ragged M, d, k tiles, the decode path (M <= 16; 16-row chunks up to
    32), the expanding GEMM (M <= 512) in 64-, 128-, 256- and 512-row tiles and
    the GEMM on the bf16 copy (M > 512) in its tile shapes (256 x 128 for most;
    256 x 256 for the forward at m = 1100, d = 6600 and for dX at m = 1100,
    k = 6592, over d = 264 not a multiple of 64), with partial last tiles; K
    split over 2-8 slices where the tiles leave most CUs idle (ragged last
    slices, also over d = 1032 not a multiple of 64); r > 16 with M >= 256
    takes the split-K row products for U and G (ragged row groups and slices,
    r = 17 .. 128)."""
    inp = make_layer(21, m * 7 + r, d, k, m, r)
    check_layer(inp, 16.0, f"shape m={m} d={d} k={k} r={r}", bf16_rounding_allowance=True)


def test_layer4096_full():
    wl = WORKLOADS["layer4096"]
    check_layer(workload_layer("layer4096"), wl.alpha, "layer4096")


@pytest.mark.parametrize("proj", [0, 1])
@pytest.mark.parametrize("m", [1, 4, 16])
def test_decode_shapes_forward(proj, m):
    wl = WORKLOADS["decode"]
    check_layer(workload_layer("decode", proj), wl.alpha, f"decode {wl.projections[proj].name}",
                m=m, want_bwd=False)


def test_decode_workspace_reuse_and_garbage():
    """The one-kernel decode path keeps per-group counters in the workspace
    when it splits k over workgroups (few row tiles, here d = 512): a
    workspace full of garbage, reused across calls and shapes, must give the
    same bits as a fresh zeroed one every time."""
    for d in (512, 4096):
        check_decode_workspace(d)


@pytest.mark.parametrize("m,d,k", [(1, 16, 4096), (16, 48, 1024), (4, 1016, 4096), (7, 520, 2048),
                                   (2, 104, 1472), (16, 8, 640), (5, 1016, 4096), (6, 104, 1472),
                                   (8, 16, 4096), (32, 1016, 4096), (17, 48, 1024)])
def test_decode_k_split_shapes(m, d, k):
    """Few row tiles: the decode forward splits k over 2..8
    workgroups per tile group (even and uneven block counts per slice), whose
    partial sums the last one to arrive adds.  Forward parity, and the
    same bits on a second call on the same workspace (the counters left ready
    by the first).  M = 17, 32: 16-row chunks, one launch each, sharing the
    counters and partial sums in stream order."""
    import bit_nf4_quantized_13_amd as q
    inp = make_layer(47, d + m, d, k, m, 16)
    check_layer(inp, 32.0, f"decode k-split m={m} d={d} k={k}", want_bwd=False, bf16_rounding_allowance=True)
    w = q.qlora_nf4_quantize(to_dev_f32(inp.w0))
    xd, ad, bd = (to_dev_bf16(t) for t in (inp.x, inp.a, inp.b))
    ws = torch.empty(q.linear_workspace_bytes(m, d, k, 16), dtype=torch.uint8, device="cuda")
    y1, u1 = q.qlora_linear_fwd(w, xd, ad, bd, 32.0, workspace=ws)
    y2, u2 = q.qlora_linear_fwd(w, xd, ad, bd, 32.0, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2) and torch.equal(u1, u2)


@pytest.mark.parametrize("m,d,k,r", [(1, 8192, 64, 1), (2, 16392, 512, 16), (1, 8200, 1088, 7), (2, 12296, 3200, 9),
                                     (3, 8200, 1088, 7), (4, 8192, 64, 1), (18, 8200, 1088, 7)])
def test_decode_dot_path_shapes(m, d, k, r):
    """M <= 2, r <= 16, k <= 4096, d >= 8192: the dot-product decode kernel
    (the decode workloads' own 14336-row shape is in
    test_decode_shapes_forward), and M = 3, 4 on such shapes through the
    matrix-core kernel; M = 18: a 16-row chunk, then two rows on the
    dot-product kernel.  Four to eight rounds of 8 rows per workgroup, more
    workgroups than a round of the chip (d = 16392: 257), k chunks past the
    row end (k = 64, 1088, 3200), ranks below 16."""
    inp = make_layer(59, m * 31 + r, d, k, m, r)
    check_layer(inp, 2.0 * r, f"decode dot m={m} d={d} k={k} r={r}", want_bwd=False,
                bf16_rounding_allowance=True)


def test_decode_chunks_equal_separate_calls():
    """A forward of 17..32 rows runs the decode kernel on consecutive 16-row
    chunks of X: the same bits (Y and U) as separate calls on the chunks."""
    import bit_nf4_quantized_13_amd as q
    for m, d, k, r in ((32, 4096, 1024, 16), (27, 8200, 512, 8), (17, 520, 2048, 24), (31, 1016, 1024, 4)):
        inp = make_layer(61, m + r, d, k, m, r)
        w = q.qlora_nf4_quantize(to_dev_f32(inp.w0))
        xd, ad, bd = (to_dev_bf16(t) for t in (inp.x, inp.a, inp.b))
        ws = torch.empty(q.linear_workspace_bytes(m, d, k, r), dtype=torch.uint8, device="cuda")
        y, u = q.qlora_linear_fwd(w, xd, ad, bd, 2.0 * r, workspace=ws)
        parts = [q.qlora_linear_fwd(w, xd[m0:m0 + 16].contiguous(), ad, bd, 2.0 * r, workspace=ws)
                 for m0 in range(0, m, 16)]
        torch.cuda.synchronize()
        assert torch.equal(y, torch.cat([p_[0] for p_ in parts])), (m, d, k, r)
        assert torch.equal(u, torch.cat([p_[1] for p_ in parts])), (m, d, k, r)


def check_decode_workspace(d):
    import bit_nf4_quantized_13_amd as q
    say(f"decode workspace garbage / reuse, d={d}")
    inp = make_layer(43, 0, d, 4096, 64, 16)
    w = q.qlora_nf4_quantize(to_dev_f32(inp.w0))
    xd, ad, bd = (to_dev_bf16(t) for t in (inp.x, inp.a, inp.b))
    nbytes = max(q.linear_workspace_bytes(m, d, 4096, 16) for m in (1, 4, 16, 64))
    clean = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    dirty = torch.full((nbytes,), 0xFF, dtype=torch.uint8, device="cuda")
    for m in (16, 1, 4, 16):
        ya, ua = q.qlora_linear_fwd(w, xd[:m], ad, bd, 32.0, workspace=clean)
        yb, ub = q.qlora_linear_fwd(w, xd[:m], ad, bd, 32.0, workspace=dirty)
        assert torch.equal(ya, yb) and torch.equal(ua, ub), m
    # a larger-M call in between writes other data into the same workspace
    q.qlora_linear_fwd(w, xd, ad, bd, 32.0, workspace=dirty)
    q.qlora_linear_bwd(w, xd, to_dev_bf16(inp.dy), ad, bd, 32.0, workspace=dirty)
    yb, ub = q.qlora_linear_fwd(w, xd[:16], ad, bd, 32.0, workspace=dirty)
    ya, ua = q.qlora_linear_fwd(w, xd[:16], ad, bd, 32.0, workspace=clean)
    assert torch.equal(ya, yb) and torch.equal(ua, ub)
    torch.cuda.synchronize()


def canon(bits: np.ndarray) -> np.ndarray:
    """-0 and +0 are the same sum (an fp32 accumulator starts at +0)."""
    out = bits.copy()
    out[out == 0x8000] = 0
    return out


def test_one_hot_inputs_return_dequantized_weights_exactly():
    """With B = 0, Y = X What^T; one-hot rows of X select columns of What, and
    one-hot rows of dY select rows of What in dX -- bit-exactly, because every
    product is exact and the sums add zeros."""
    import bit_nf4_quantized_13_amd as q
    say("one-hot exactness probe")
    d, k, r = 320, 384, 8
    w0 = random_weights(31, (d, k))
    w = q.qlora_nf4_quantize(to_dev_f32(w0))
    what = bf16_to_host_bits(q.qlora_nf4_dequantize(w))
    one = np.uint16(0x3F80)
    x = np.zeros((k, k), np.uint16)
    x[np.arange(k), np.arange(k)] = one
    a = random_bf16(32, (r, k))
    b = np.zeros((d, r), np.uint16)
    y, u = q.qlora_linear_fwd(w, to_dev_bf16(x), to_dev_bf16(a), to_dev_bf16(b), 16.0)
    assert np.array_equal(canon(bf16_to_host_bits(y)), canon(what.T.copy()))
    dy = np.zeros((d, d), np.uint16)
    dy[np.arange(d), np.arange(d)] = one
    xx = random_bf16(33, (d, k))
    dx, da, db = q.qlora_linear_bwd(w, to_dev_bf16(xx), to_dev_bf16(dy), to_dev_bf16(a),
                                    to_dev_bf16(b), 16.0)
    assert np.array_equal(canon(bf16_to_host_bits(dx)), canon(what))
    assert np.all(da.cpu().numpy() == 0)          # B = 0 => G = 0 => dA = 0 exactly
    ref = nf4.dequantize(nf4.quantize(w0), (d, k))
    assert np.array_equal(what, ref)


@pytest.mark.parametrize("m,r", [(200, 16), (520, 64)])
def test_recomputed_u_matches_saved_u_and_runs_are_deterministic(m, r):
    """Reruns give the same bits, and a backward that recomputes U (and its
    planes) matches one given the forward's U bit for bit -- with r = 64 and
    M >= 256 through the split-K row products and their reduction."""
    import bit_nf4_quantized_13_amd as q
    say(f"determinism / U recompute m={m} r={r}")
    inp = make_layer(41, r, 512, 512, m, r)
    w = q.qlora_nf4_quantize(to_dev_f32(inp.w0))
    xd, ad, bd, dyd = (to_dev_bf16(t) for t in (inp.x, inp.a, inp.b, inp.dy))
    y1, u1 = q.qlora_linear_fwd(w, xd, ad, bd, 32.0)
    y2, u2 = q.qlora_linear_fwd(w, xd, ad, bd, 32.0)
    assert torch.equal(y1, y2) and torch.equal(u1, u2)
    g1 = q.qlora_linear_bwd(w, xd, dyd, ad, bd, 32.0, u=u1)
    g2 = q.qlora_linear_bwd(w, xd, dyd, ad, bd, 32.0, u=None)
    for t1, t2 in zip(g1, g2):
        assert torch.equal(t1, t2)
    _, da, db = q.qlora_linear_bwd(w, xd, dyd, ad, bd, 32.0, u=u1, need_dx=False)
    assert torch.equal(da, g1[1]) and torch.equal(db, g1[2])


@pytest.mark.parametrize("m,d,k,r", [(4096, 512, 512, 8), (1400, 1032, 320, 3), (300, 264, 512, 16)])
def test_backward_g_paths_agree(m, d, k, r):
    """G = dY B runs straight from B as stored when B is 16-byte aligned (one
    launch, with U's planes) and through a transposed copy of B otherwise (B
    only 2-byte aligned): both give the same bits, with the forward's U and
    with U recomputed.  d % 128 != 0 puts a partial chunk of B rows at the end."""
    import bit_nf4_quantized_13_amd as q
    say(f"backward G paths m={m} d={d} k={k} r={r}")
    inp = make_layer(43, r, d, k, m, r)
    w = q.qlora_nf4_quantize(to_dev_f32(inp.w0))
    xd, ad, bd, dyd = (to_dev_bf16(t) for t in (inp.x, inp.a, inp.b, inp.dy))
    store = torch.empty(d * r + 1, dtype=torch.bfloat16, device="cuda")
    b_off = store[1:].view(d, r)
    b_off.copy_(bd)
    assert b_off.data_ptr() % 16 != 0 and bd.data_ptr() % 16 == 0
    _, u = q.qlora_linear_fwd(w, xd, ad, bd, 32.0)
    for uu in (u, None):
        g1 = q.qlora_linear_bwd(w, xd, dyd, ad, bd, 32.0, u=uu)
        g2 = q.qlora_linear_bwd(w, xd, dyd, ad, b_off, 32.0, u=uu)
        for t1, t2 in zip(g1, g2):
            assert torch.equal(t1, t2)


def test_alpha_zero_gives_base_output_and_zero_adapter_grads():
    import bit_nf4_quantized_13_amd as q
    say("alpha = 0")
    inp = make_layer(42, 0, 256, 256, 64, 8)
    w = q.qlora_nf4_quantize(to_dev_f32(inp.w0))
    xd, ad, bd, dyd = (to_dev_bf16(t) for t in (inp.x, inp.a, inp.b, inp.dy))
    y, _ = q.qlora_linear_fwd(w, xd, ad, bd, 0.0)
    y0, _ = q.qlora_linear_fwd(w, xd, ad, to_dev_bf16(np.zeros_like(inp.b)), 16.0)
    assert torch.equal(y, y0)
    _, da, db = q.qlora_linear_bwd(w, xd, dyd, ad, bd, 0.0)
    assert torch.count_nonzero(da) == 0 and torch.count_nonzero(db) == 0


@pytest.mark.parametrize("m", [200, 600])
def test_gemm_only_reruns_the_calls_gemm(m):
    """qlora_linear_gemm_only re-launches just the dequant-GEMM on the workspace
    the preceding call prepared: the output must be bit-identical, also from
    the kernel that expands the codes tile by tile (M = 600: the call itself
    used the bf16 copy)."""
    import bit_nf4_quantized_13_amd as q
    say(f"gemm_only M={m}")
    inp = make_layer(44, m, 384, 320, m, 8)
    w = q.qlora_nf4_quantize(to_dev_f32(inp.w0))
    xd, ad, bd, dyd = (to_dev_bf16(t) for t in (inp.x, inp.a, inp.b, inp.dy))
    ws = torch.empty(q.linear_workspace_bytes(m, 384, 320, 8), dtype=torch.uint8, device="cuda")
    y, u = q.qlora_linear_fwd(w, xd, ad, bd, 16.0, workspace=ws)
    y2 = torch.full_like(y, 7)
    q.qlora_linear_gemm_only(w, False, xd, 8, y2, ws)
    assert torch.equal(y, y2)
    # the expanding kernel on the same operands (with M > 512 the call itself streams a bf16 copy)
    y3 = torch.full_like(y, 7)
    q.qlora_linear_gemm_only(w, False, xd, 8, y3, ws, expand=True)
    assert torch.equal(y, y3)
    dx, _, _ = q.qlora_linear_bwd(w, xd, dyd, ad, bd, 16.0, u=u, workspace=ws)
    dx2 = torch.full_like(dx, 7)
    q.qlora_linear_gemm_only(w, True, dyd, 8, dx2, ws)
    assert torch.equal(dx, dx2)
    dx3 = torch.full_like(dx, 7)
    q.qlora_linear_gemm_only(w, True, dyd, 8, dx3, ws, expand=True)
    assert torch.equal(dx, dx3)
    torch.cuda.synchronize()
