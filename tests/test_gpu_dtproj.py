"""GPU parity of dt_proj (ssm_dt_proj through the C ABI) against the fp64
oracle (oracle_dt_proj, pinned by unit rows, an exact integer brute force, the
rank-one closed form and linearity) on the same seeded inputs.

Tolerance (gpu_util.err, max relative error with an rms floor): 2e-2 for bf16
io (one rounding of the fp32 sum to bf16: about 4e-3), 1e-5 for fp32 io (fp32
accumulation over rank <= 160 terms).
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import gpu_util as G
import oracle
from selective_scan_ssm_amd import inputs as gen

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from selective_scan_ssm_amd import _lib
    _lib.load()


def run(inp, rows_3d=None):
    from selective_scan_ssm_amd import ops
    io = inp["io"]
    xd = G.to_torch(inp["x_dbl"], io)
    if rows_3d:
        xd = xd.view(rows_3d[0], rows_3d[1], inp["ldx"])
    out = ops.dt_proj(xd[..., :inp["rank"]], G.to_torch(inp["W"], io))
    torch.cuda.synchronize()
    return G.from_torch(out).reshape(inp["rows"], inp["dim"])


def expect(inp, rows=None):
    io = inp["io"]
    x = gen.to_f64(inp["x_dbl"], io)
    if rows is not None:
        x = x[rows]
    return oracle.dt_proj(x, gen.to_f64(inp["W"], io), threads=G.ORACLE_THREADS)


@pytest.mark.parametrize("io,rows,rank,dim,ldx", [
    (gen.BF16, 300, 48, 200, 80),      # the 130m layer's rank, ragged rows and channels
    (gen.BF16, 129, 160, 132, 192),    # the 2.8b layer's rank: two whole K chunks and a half
    (gen.BF16, 64, 8, 4, 8),           # one K piece, four channels
    (gen.F32, 130, 160, 260, 192),
    (gen.F32, 77, 4, 36, 12),
])
def test_dt_proj_small(io, rows, rank, dim, ldx):
    inp = gen.make_dtproj_inputs(rows, rank, dim, ldx, io=io, seed=900 + rank)
    G.say(f"[dt_proj] io={io} rows={rows} rank={rank} dim={dim} ldx={ldx}")
    e = G.err(run(inp), expect(inp))
    G.say(f"[dt_proj] err={e:.2e}")
    assert e <= G.TOL[io], e


def test_dt_proj_reads_only_the_rank_columns():
    # the x_proj columns after the rank (B and C) hold NaN: nothing of them may show
    inp = gen.make_dtproj_inputs(200, 48, 136, 80, io=gen.F32, seed=950)
    inp["x_dbl"][:, 48:] = np.nan
    got = run(inp)
    assert np.all(np.isfinite(got))
    assert G.err(got, expect(inp)) <= 1e-5


def test_dt_proj_batch_seqlen_view_and_empty():
    from selective_scan_ssm_amd import ops
    inp = gen.make_dtproj_inputs(3 * 70, 48, 96, 80, io=gen.BF16, seed=951)
    assert G.err(run(inp, rows_3d=(3, 70)), expect(inp)) <= 2e-2
    x = torch.zeros((0, 80), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((96, 48), dtype=torch.bfloat16, device="cuda")
    assert ops.dt_proj(x[:, :48], w).shape == (0, 96)
    # one row, and (batch, 1, rank): the row stride comes from the axes longer than 1
    one = gen.make_dtproj_inputs(1, 48, 96, 80, io=gen.BF16, seed=953)
    assert G.err(run(one), expect(one)) <= 2e-2
    five = gen.make_dtproj_inputs(5, 48, 96, 80, io=gen.BF16, seed=954)
    assert G.err(run(five, rows_3d=(5, 1)), expect(five)) <= 2e-2


def test_dt_proj_mamba2p8b_layer_sampled():
    """The 2.8b layer's dt_proj at full size (4 x 8192 rows, rank 160, x_proj
    rows of 160 + 2 x 16, d_inner 5120) in the launch the bench times; 96
    sampled rows (every channel) against the oracle, all of delta finite."""
    rows, rank, dim, ldx = 4 * 8192, 160, 5120, 192
    inp = gen.make_dtproj_inputs(rows, rank, dim, ldx, io=gen.BF16, seed=952)
    G.say(f"[dt_proj] 2.8b layer rows={rows} rank={rank} dim={dim}")
    got = run(inp)
    assert np.all(np.isfinite(got))
    pick = np.r_[0:32, rows // 2 - 16:rows // 2 + 16, rows - 32:rows]
    e = G.err(got[pick], expect(inp, rows=pick))
    G.say(f"[dt_proj] 2.8b layer sampled err={e:.2e}")
    assert e <= 2e-2, e


@pytest.mark.parametrize("rank", [48, 104])
def test_dt_proj_bf16_reads_only_the_rank_columns(rank):
    # bf16 runs the persistent kernel, whose xdt fragments are 8 columns wide
    # and whose last K step reaches past the rank: those columns (B and C of
    # the x_proj row) hold NaN here, and nothing of them may show
    inp = gen.make_dtproj_inputs(300, rank, 264, rank + 32, io=gen.BF16, seed=960 + rank)
    inp["x_dbl"][:, rank:] = gen.bf16_from_f32(np.full((300, 32), np.nan, np.float32))
    got = run(inp)
    assert np.all(np.isfinite(got))
    assert G.err(got, expect(inp)) <= 2e-2


def test_dt_proj_bf16_many_slabs_per_workgroup():
    """600 and a part 128-row slabs over 21 channel tiles: each persistent
    workgroup walks about 25 slabs, the last one ragged, and d_inner % 8 == 4
    sends rows out in 8-byte halves; sampled rows against the oracle."""
    rows, rank, dim, ldx = 128 * 600 + 37, 160, 2564, 192
    inp = gen.make_dtproj_inputs(rows, rank, dim, ldx, io=gen.BF16, seed=970)
    got = run(inp)
    assert np.all(np.isfinite(got))
    pick = np.r_[0:40, 128 * 317 - 20:128 * 317 + 20, rows - 45:rows]
    e = G.err(got[pick], expect(inp, rows=pick))
    G.say(f"[dt_proj] many slabs err={e:.2e}")
    assert e <= 2e-2, e


def test_dt_proj_bf16_rank_above_the_persistent_kernel():
    # rank 168 > 160: the tiled kernel with K staged through LDS
    inp = gen.make_dtproj_inputs(200, 168, 136, 200, io=gen.BF16, seed=971)
    assert G.err(run(inp), expect(inp)) <= 2e-2


def test_dt_proj_mamba130m_layer_sampled():
    """The 130m layer's dt_proj at full size (8 x 2048 rows, rank 48, x_proj
    rows of 48 + 2 x 16, d_inner 1536); sampled rows against the oracle."""
    rows, rank, dim, ldx = 8 * 2048, 48, 1536, 80
    inp = gen.make_dtproj_inputs(rows, rank, dim, ldx, io=gen.BF16, seed=972)
    got = run(inp)
    assert np.all(np.isfinite(got))
    pick = np.r_[0:64, rows - 64:rows]
    assert G.err(got[pick], expect(inp, rows=pick)) <= 2e-2
