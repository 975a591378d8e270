"""The algorithmic work bench.py divides by the measured durations, pinned
on hand-counted cases: a symmetric product of d x d matrices is d^2 (d + 1)
flops (upper triangle, diagonal included); a Newton root of K steps, j of
them float64, runs 3 products on M per step (M^2, T2^2, T4 M) and 1 on X,
the last step only its finish (X q: 1 product; degree 2: q from M^2, then
X q; degree 4: M^2, E^2 R, X q), and the first X product is no product (the
init writes X1 = q(M0))."""

import bench


def test_symmetric_product_flops():
    assert bench.sym_gemm_flops(1) == 2
    assert bench.sym_gemm_flops(4) == 16 * 5
    assert bench.sym_gemm_flops(4096) == 4096 ** 2 * 4097


def test_newton_flops_width_1024_schedule():
    # the width-1024 Grams' schedule: 8 steps, 2 float64, degree-2 finish
    g = bench.sym_gemm_flops(4096)
    f64, low = bench.newton_flops(4096, 8, 2, final_degree=2)
    # float64: steps 0, 1 -> 3 M products each
    assert f64 == 6 * g
    # split: X product of step 1 (step 0's is the init's), steps 2..6 -> 4
    # products each, step 7 -> q(M) and X q
    assert low == (1 + 5 * 4 + 2) * g


def test_newton_flops_finishes_and_float64_x():
    g = bench.sym_gemm_flops(100)
    # degree-1 last step: only its X product; degree 4: three products
    assert bench.newton_flops(100, 3, 1, final_degree=1) == (3 * g, (0 + 4 + 1) * g)
    assert bench.newton_flops(100, 3, 1, final_degree=4) == (3 * g, (0 + 4 + 3) * g)
    # X in float64 (not x_low): every product of the float64 steps is float64,
    # the first X product included
    assert bench.newton_flops(100, 3, 2, x_low=False, final_degree=1) == ((4 + 4) * g, 1 * g)


def test_root_stream_bytes():
    d, n = 1024, 1024 * 1024
    b = bench.root_stream_bytes(d, 8, False, 8, 2)
    # two float64 steps with products: M read (8) and cut into six digit planes
    # (6 per element, d = 1024 needs no padding) with d row exponents, each
    assert b == {"root_stats": 8 * n, "root_init": 8 * n + 16 * n, "newton_convert": 12 * n,
                 "newton_slice": 2 * (8 * n + 6 * n + 4 * d), "root_finalize": (4 + 4 + 4) * n}
    bp = bench.root_stream_bytes(d, 8, True, 2, 5)  # packed state, every step float64
    assert bp["root_stats"] == 8 * (d * (d + 1) // 2) and bp["newton_convert"] == 0
    assert bp["root_finalize"] == (4 + 8 + 4) * n
    assert bp["newton_slice"] == 8 * n + 6 * n + 4 * d  # K = 2: the last step has no products
    # a ragged size pads the planes to a multiple of 128
    br = bench.root_stream_bytes(1100, 8, False, 6, 1)
    assert br["newton_slice"] == 8 * 1100 * 1100 + 6 * 1152 * 1152 + 4 * 1152
    # below 1024 the float64 steps keep the float64 kernel: no planes
    assert bench.root_stream_bytes(512, 4, False, 9, 3)["newton_slice"] == 0
    assert bench.f64_class(512) == "newton_f64" and bench.f64_class(1024) == "newton_i8"


def test_bench_refuses_more_than_one_gpu(capsys):
    assert bench.main(["--gpus", "2"]) == 2
    assert "one GPU only" in capsys.readouterr().err
