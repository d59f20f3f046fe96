"""GPU parity at the largest launches: the row limit and past 2^32 elements.

The largest parity cases elsewhere hold a few hundred million elements.
These launches reach the limits the header states and the places where
32-bit arithmetic would break:

* AARMS_MAX_TOKENS rows (2^31 - 1) of the narrowest widths, where one block
  per row quartet is more work-items than a grid dimension counts (2^32) and
  the grid becomes two-dimensional; the SwiGLU's row-chunked grid runs 32,769
  slices deep in z there.
* Norms of 16,384-wide rows past 2^32 elements per tensor, and forced
  variants (16 waves a row, the resident rows) past the 1-D grid's reach.
* SwiGLU rows of 2^33 outputs (the width limit) in every static form.
* The per-tensor E4M3 SwiGLU of 28,672-wide rows at the flat grid's last
  launch under 2^32 jobs and at the first launch past it (the row-chunked
  grid then takes over), with the job index crossing 2^31 inside.

Inputs are generated on the device from a seeded generator.  The oracle
checks sampled rows -- the first and last rows, the rows on each side of
every grid and index boundary above, and random rows -- copied back to the
host, to the same bar as the other parity tests.  A property checked on
every element: each output was written (outputs are filled with a NaN
pattern first; finite inputs give finite outputs).

Each test needs up to 172 GB of device memory and is skipped when the
device has less free.
"""

from __future__ import annotations

import gc

import numpy as np
import pytest
import torch

import activation_add_rmsnorm_amd as A
from tests import parity as P

pytestmark = pytest.mark.gpu

DEV = "cuda"
MAX_T = 2**31 - 1
CHUNK = 1 << 30                                # elements per generation / scan step


def announce(*what):
    print("[gpu]", *what, flush=True)


@pytest.fixture(autouse=True)
def _release():
    yield
    gc.collect()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _need(nbytes: float):
    torch.cuda.empty_cache()
    free = torch.cuda.mem_get_info()[0]
    if free < nbytes * 1.03 + (2 << 30):
        pytest.skip("needs %.1f GB of free device memory, %.1f GB free" % (nbytes / 1e9, free / 1e9))


def _randn(shape, std, seed):
    """bf16 ~N(0, std^2), generated in place chunk by chunk."""
    t = torch.empty(shape, dtype=torch.bfloat16, device=DEV)
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    flat = t.view(-1)
    for i in range(0, flat.numel(), CHUNK):
        flat[i:i + CHUNK].normal_(0.0, std, generator=g)
    return t


def _poisoned(shape, dtype):
    t = torch.empty(shape, dtype=dtype, device=DEV)
    if t.element_size() == 2:
        t.view(torch.int16).fill_(0x7FC1)      # a bf16 NaN
    elif t.element_size() == 1:
        t.view(torch.uint8).fill_(0x7F)        # the E4M3 NaN code
    else:
        t.fill_(float("nan"))
    return t


def _all_written(t: torch.Tensor, name: str):
    flat = t.view(-1)
    for i in range(0, flat.numel(), CHUNK):
        c = flat[i:i + CHUNK]
        if t.element_size() == 1:
            hit = ((c.view(torch.uint8) & 0x7F) == 0x7F).any()
        else:
            hit = torch.isnan(c).any()
        assert not bool(hit), "%s: elements %d.. still hold the fill pattern or a NaN" % (name, i)


def _rows(T: int, boundaries, seed: int, n_random: int = 48) -> np.ndarray:
    """Rows 0-3, the last four, two on each side of every boundary, and random rows."""
    r = set(range(4)) | set(range(T - 4, T))
    for b in boundaries:
        r |= set(range(b - 2, b + 2))
    rng = np.random.default_rng(seed)
    r |= set(rng.integers(0, T, n_random).tolist())
    return np.array(sorted(x for x in r if 0 <= x < T), dtype=np.int64)


def _take(t: torch.Tensor, rows: np.ndarray) -> np.ndarray:
    idx = torch.from_numpy(rows).to(DEV)
    return P.from_gpu_bits(t.index_select(0, idx))


def _weight(H: int, seed: int) -> torch.Tensor:
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    return (1.0 + 0.1 * torch.randn(H, device=DEV, generator=g)).to(torch.bfloat16)


# ------------------------------------------------------------------ norms at the row limit

def _grid_rows(T: int, rows_per_block: int, threads: int):
    """Rows where a 32-bit work-item count of a 1-D grid would wrap, and the
    first rows of each row of 2^21 blocks of the two-dimensional grid."""
    out = []
    wrap_blocks = (1 << 32) // threads
    out += [k * wrap_blocks * rows_per_block for k in (1, 2, 3)]
    step = (1 << 21) * rows_per_block
    out += [k * step for k in (1, 2, 3, 8, 64)] + [(T // step) * step]
    return out


def test_norms_at_the_row_limit_narrow_rows():
    T, H = MAX_T, 8
    _need(4 * T * H * 2)
    eps = 1e-6
    announce("max rows: inputs [%d, %d]" % (T, H))
    x, r = _randn((T, H), 1.0, 1), _randn((T, H), 1.0, 2)
    w = _weight(H, 3)
    rows = _rows(T, _grid_rows(T, 4, 256), 4)
    xs, rs, ws = _take(x, rows), _take(r, rows), P.from_gpu_bits(w)

    announce("max rows: fused_add_rmsnorm, variant", A.variant_name(A.OP_NORM, A.pick_variant(A.OP_NORM, T, H, 0)))
    out, res = _poisoned((T, H), torch.bfloat16), _poisoned((T, H), torch.bfloat16)
    A.fused_add_rmsnorm(x, r, w, eps, out=out, residual_out=res)
    torch.cuda.synchronize()
    _all_written(out, "out")
    _all_written(res, "residual_out")
    P.check_norm(xs, rs, ws, eps, _take(out, rows), _take(res, rows))
    del out, res

    announce("max rows: fused_add_rmsnorm_quant_fp8 (per token)")
    q = _poisoned((T, H), torch.float8_e4m3fn)
    s = _poisoned((T,), torch.float32)
    res = _poisoned((T, H), torch.bfloat16)
    A.fused_add_rmsnorm_quant_fp8(x, r, w, 1e-5, out=q, scale_out=s, residual_out=res)
    torch.cuda.synchronize()
    _all_written(q, "codes")
    _all_written(s, "scales")
    _all_written(res, "residual_out")
    sel = torch.from_numpy(rows).to(DEV)
    P.check_norm_fp8(xs, rs, ws, 1e-5, _take(q, rows), P.from_gpu_bits(s.index_select(0, sel)), _take(res, rows))


def test_forced_wide_variants_past_the_one_dimensional_grid():
    """16 waves a row (1,024-thread blocks) on 5,000,000 rows, the norm and
    the per-token SwiGLU, and the resident rows (four 512-wide rows a block)
    on 2^26 + 12 rows: every grid is more than 2^32 work-items along one
    dimension."""
    eps = 1e-6
    T, H = 5_000_000, 8
    v16 = next(i for i in range(A.variant_count(A.OP_NORM)) if A.variant_name(A.OP_NORM, i) == "16 waves/row x1 vec")
    _need(4 * T * H * 2)
    announce("16 waves a row on [%d, %d]" % (T, H))
    x, r = _randn((T, H), 1.0, 5), _randn((T, H), 1.0, 6)
    w = _weight(H, 7)
    rows = _rows(T, _grid_rows(T, 1, 1024), 8)
    out, res = _poisoned((T, H), torch.bfloat16), _poisoned((T, H), torch.bfloat16)
    A.fused_add_rmsnorm(x, r, w, eps, out=out, residual_out=res, variant=v16)
    torch.cuda.synchronize()
    _all_written(out, "out")
    _all_written(res, "residual_out")
    P.check_norm(_take(x, rows), _take(r, rows), P.from_gpu_bits(w), eps, _take(out, rows), _take(res, rows))
    del x, r, out, res

    # the per-token SwiGLU on 16-wave rows: [5,000,000, 2 x 8]
    N = 8
    vq = next(i for i in range(A.variant_count(A.OP_SWIGLU_DYNAMIC))
              if A.variant_name(A.OP_SWIGLU_DYNAMIC, i) == "16 waves/row x2 jobs")
    announce("swiglu_quant_fp8_dynamic, 16 waves a row, on [%d, %d]" % (T, 2 * N))
    gu = _randn((T, 2 * N), 1.0, 24)
    q = _poisoned((T, N), torch.float8_e4m3fn)
    s = _poisoned((T,), torch.float32)
    A.swiglu_quant_fp8_dynamic(gu, out=q, scale_out=s, variant=vq)
    torch.cuda.synchronize()
    _all_written(q, "codes")
    _all_written(s, "scales")
    sel = torch.from_numpy(rows).to(DEV)
    P.check_swiglu_fp8_dynamic(_take(gu, rows), _take(q, rows), P.from_gpu_bits(s.index_select(0, sel)))
    del gu, q, s

    T, H = (1 << 26) + 12, 512
    _need(2 * T * H * 2)
    for name in ("wave/row x32 vec, resident, 6-slice window", "wave/row x32 vec, resident, 10-slice window"):
        vr = next(i for i in range(A.variant_count(A.OP_RMSNORM)) if A.variant_name(A.OP_RMSNORM, i) == name)
        announce("rmsnorm, %s, on [%d, %d]" % (name, T, H))
        x = _randn((T, H), 1.0, 9)
        w = _weight(H, 10)
        rows = _rows(T, _grid_rows(T, 4, 256), 11)
        out = _poisoned((T, H), torch.bfloat16)
        A.rmsnorm(x, w, eps, out=out, variant=vr)
        torch.cuda.synchronize()
        _all_written(out, "out")
        P.check_rmsnorm(_take(x, rows), P.from_gpu_bits(w), eps, _take(out, rows))
        del x, out


def test_norms_past_2_32_elements_wide_rows():
    """[262,147, 16,384]: 2^32 + 49,152 elements per tensor; the heuristic's
    variant and the resident rows forced."""
    T, H = 262_147, 16384
    _need(4 * T * H * 2)
    eps = 1e-5
    x, r = _randn((T, H), 1.0, 12), _randn((T, H), 1.0, 13)
    w = _weight(H, 14)
    # rows where the element index crosses 2^31 and 2^32
    rows = _rows(T, [(1 << 31) // H, (1 << 32) // H], 15)
    xs, rs, ws = _take(x, rows), _take(r, rows), P.from_gpu_bits(w)
    resident = [i for i in range(A.variant_count(A.OP_NORM)) if "resident" in A.variant_name(A.OP_NORM, i)]
    for v in [-1] + resident:
        announce("[%d, %d] norm, variant" % (T, H), v)
        out, res = _poisoned((T, H), torch.bfloat16), _poisoned((T, H), torch.bfloat16)
        A.fused_add_rmsnorm(x, r, w, eps, out=out, residual_out=res, variant=v)
        torch.cuda.synchronize()
        _all_written(out, "out")
        P.check_norm(xs, rs, ws, eps, _take(out, rows), _take(res, rows))
        del out
        q = _poisoned((T, H), torch.float8_e4m3fn)
        s = _poisoned((T,), torch.float32)
        res.view(torch.int16).fill_(0x7FC1)
        A.fused_add_rmsnorm_quant_fp8(x, r, w, eps, out=q, scale_out=s, residual_out=res, variant=v)
        torch.cuda.synchronize()
        _all_written(q, "codes")
        _all_written(res, "residual_out")
        sel = torch.from_numpy(rows).to(DEV)
        P.check_norm_fp8(xs, rs, ws, eps, _take(q, rows), P.from_gpu_bits(s.index_select(0, sel)), _take(res, rows))
        del q, s, res


# ------------------------------------------------------------------ SwiGLU at the row limit

def test_swiglu_at_the_row_limit_narrow_rows():
    """[2^31 - 1, 2 x 8] -> [2^31 - 1, 8]: one job a row, the row-chunked grid
    65,535 rows along y and 32,769 slices along z; the per-token form on the
    two-dimensional grid."""
    T, N = MAX_T, 8
    _need(T * 2 * N * 2 + T * N * 2)
    gu = _randn((T, 2 * N), 1.0, 16)
    y_rows = 65535
    rows = _rows(T, [y_rows, 2 * y_rows, 32768 * y_rows] + _grid_rows(T, 4, 256), 17)
    gus = _take(gu, rows)

    announce("max rows: swiglu bf16")
    y = _poisoned((T, N), torch.bfloat16)
    A.swiglu(gu, out=y)
    torch.cuda.synchronize()
    _all_written(y, "y")
    P.check_swiglu(gus, _take(y, rows))
    del y

    announce("max rows: swiglu_quant_fp8 (per tensor)")
    scale = torch.tensor([0.05], dtype=torch.float32, device=DEV)
    q = _poisoned((T, N), torch.float8_e4m3fn)
    A.swiglu_quant_fp8(gu, scale, out=q)
    torch.cuda.synchronize()
    _all_written(q, "codes")
    P.check_swiglu_fp8(gus, 0.05, _take(q, rows))

    announce("max rows: swiglu_quant_fp8_dynamic (per token)")
    q.view(torch.uint8).fill_(0x7F)
    s = _poisoned((T,), torch.float32)
    A.swiglu_quant_fp8_dynamic(gu, out=q, scale_out=s)
    torch.cuda.synchronize()
    _all_written(q, "codes")
    _all_written(s, "scales")
    sel = torch.from_numpy(rows).to(DEV)
    P.check_swiglu_fp8_dynamic(gus, _take(q, rows), P.from_gpu_bits(s.index_select(0, sel)))


def test_swiglu_fp8_flat_grid_at_its_job_limit():
    """Per-tensor E4M3 on 28,672-wide rows (3,584 jobs a row): 1,198,372 rows
    are the flat grid's largest launch (4,294,965,248 jobs), 1,198,373 rows
    take the row-chunked grid.  gate_up ~N(0, 2^2), scale 0.05."""
    N = 28672
    njobs = N // 8
    T0 = 0xFFFFFF00 // njobs
    T1 = T0 + 1
    _need(T1 * 2 * N * 2 + T1 * N)
    flat = A.pick_variant(A.OP_SWIGLU, T0, N, 1)
    assert A.variant_name(A.OP_SWIGLU, flat) == "1 job/lane, flat rows"
    assert A.variant_name(A.OP_SWIGLU, A.pick_variant(A.OP_SWIGLU, T1, N, 1)) != "1 job/lane, flat rows"
    gu = _randn((T1, 2 * N), 2.0, 18)
    scale = torch.tensor([0.05], dtype=torch.float32, device=DEV)
    q = torch.empty((T1, N), dtype=torch.float8_e4m3fn, device=DEV)
    for T in (T0, T1):
        # rows where the job index crosses 2^31, the grid's y slices, the last rows
        rows = _rows(T, [(1 << 31) // njobs, 65535, 18 * 65535], 19 + T - T0, n_random=24)
        announce("swiglu_quant_fp8 on [%d, %d], variant %s" % (T, 2 * N, A.variant_name(A.OP_SWIGLU, A.pick_variant(A.OP_SWIGLU, T, N, 1))))
        qt = q[:T]
        qt.view(torch.uint8).fill_(0x7F)
        A.swiglu_quant_fp8(gu[:T], scale, out=qt)
        torch.cuda.synchronize()
        _all_written(qt, "codes")
        P.check_swiglu_fp8(_take(gu, rows), 0.05, _take(qt, rows))


def test_swiglu_past_2_32_outputs_qwen_rows():
    """[479,350, 2 x 8,960] -> [479,350, 8,960]: 2^32 + 9,984 outputs; bf16 on
    the row-chunked grid (8 slices along z) and the per-token E4M3 rows."""
    N = 8960
    T = (1 << 32) // N + 1
    _need(T * 2 * N * 2 + T * N * 2)
    gu = _randn((T, 2 * N), 1.0, 20)
    rows = _rows(T, [(1 << 31) // N, (1 << 32) // N, 65535, 7 * 65535], 21, n_random=24)
    gus = _take(gu, rows)
    announce("swiglu bf16 on [%d, %d]" % (T, 2 * N))
    y = _poisoned((T, N), torch.bfloat16)
    A.swiglu(gu, out=y)
    torch.cuda.synchronize()
    _all_written(y, "y")
    P.check_swiglu(gus, _take(y, rows))
    del y
    announce("swiglu_quant_fp8_dynamic on [%d, %d]" % (T, 2 * N))
    q = _poisoned((T, N), torch.float8_e4m3fn)
    s = _poisoned((T,), torch.float32)
    A.swiglu_quant_fp8_dynamic(gu, out=q, scale_out=s)
    torch.cuda.synchronize()
    _all_written(q, "codes")
    _all_written(s, "scales")
    sel = torch.from_numpy(rows).to(DEV)
    P.check_swiglu_fp8_dynamic(gus, _take(q, rows), P.from_gpu_bits(s.index_select(0, sel)))


# ------------------------------------------------------------------ SwiGLU at the row-width limit

def test_swiglu_widest_rows_every_static_form():
    """[2, 2 x 2^33] -> [2, 2^33] (AARMS_MAX_INTER): one row holds 2^33
    outputs, so output, scale and `up` offsets pass 2^31 and 2^32 within a
    row; bf16, per-tensor E4M3 (the flat grid, 2^31 jobs), MXFP4, NVFP4 and
    per-128 E4M3.  Sampled: aligned 128-output blocks (whole scale blocks of
    every form) at both ends of each row and around 2^31 and 2^32."""
    T, N = 2, 1 << 33
    _need(T * 2 * N * 2 + T * N * 2)
    gu = _randn((T, 2 * N), 2.0, 22)
    rng = np.random.default_rng(23)
    starts = [0, 1 << 30, (1 << 31) - 128, 1 << 31, (1 << 32) - 128, 1 << 32, N - 256, N - 128]
    starts += (rng.integers(0, N // 128, 6) * 128).tolist()
    cols = np.unique(np.concatenate([np.arange(c, c + 128) for c in starts]))
    blocks = lambda per: torch.from_numpy(np.unique(cols // per)).to(DEV)
    idx = torch.from_numpy(cols).to(DEV)
    gus = P.from_gpu_bits(torch.cat([gu.index_select(1, idx), gu.index_select(1, idx + N)], dim=1))
    take_cols = lambda t, ix: P.from_gpu_bits(t.index_select(1, ix))
    name = lambda q: A.variant_name(A.OP_SWIGLU, A.pick_variant(A.OP_SWIGLU, T, N, q))

    announce("widest rows: swiglu bf16, variant", name(0))
    y = _poisoned((T, N), torch.bfloat16)
    A.swiglu(gu, out=y)
    torch.cuda.synchronize()
    _all_written(y, "y")
    P.check_swiglu(gus, take_cols(y, idx))
    del y

    announce("widest rows: swiglu_quant_fp8, variant", name(1))
    scale = torch.tensor([0.05], dtype=torch.float32, device=DEV)
    q = _poisoned((T, N), torch.float8_e4m3fn)
    A.swiglu_quant_fp8(gu, scale, out=q)
    torch.cuda.synchronize()
    _all_written(q, "codes")
    P.check_swiglu_fp8(gus, 0.05, take_cols(q, idx))

    announce("widest rows: swiglu_quant_fp8_group, variant", name(4))
    q.view(torch.uint8).fill_(0x7F)
    s = _poisoned((T, N // 128), torch.float32)
    A.swiglu_quant_fp8_group(gu, out=q, scale_out=s)
    torch.cuda.synchronize()
    _all_written(q, "codes")
    _all_written(s, "scales")
    P.check_swiglu_fp8_group(gus, take_cols(q, idx), take_cols(s, blocks(128)))
    del q, s

    # E2M1 codes have no unused pattern; the scale bytes are checked written
    # (0xFF is the E8M0 NaN scale, 0x7F the E4M3 NaN: neither comes from
    # finite inputs)
    half = torch.from_numpy(np.unique(cols // 2)).to(DEV)
    announce("widest rows: swiglu_quant_mxfp4, variant", name(2))
    q4 = torch.empty((T, N // 2), dtype=torch.uint8, device=DEV)
    s4 = torch.full((T, N // 32), 0xFF, dtype=torch.uint8, device=DEV)
    A.swiglu_quant_mxfp4(gu, out=q4, scale_out=s4)
    torch.cuda.synchronize()
    assert not bool((s4 == 0xFF).any()), "MXFP4 scales: a block was not written"
    P.check_swiglu_mxfp4(gus, take_cols(q4, half), take_cols(s4, blocks(32)))

    announce("widest rows: swiglu_quant_nvfp4, variant", name(3))
    g = torch.tensor([0.05], dtype=torch.float32, device=DEV)
    s16 = torch.full((T, N // 16), 0x7F, dtype=torch.uint8, device=DEV)
    A.swiglu_quant_nvfp4(gu, g, out=q4, scale_out=s16)
    torch.cuda.synchronize()
    assert not bool(((s16 & 0x7F) == 0x7F).any()), "NVFP4 scales: a block was not written"
    P.check_swiglu_nvfp4(gus, 0.05, take_cols(q4, half), take_cols(s16, blocks(16)))
