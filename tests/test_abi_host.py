"""Host-side tests of the C ABI (CPU only, no GPU needed).

* the shared library loads and exports every function include/*.h declares;
* argument validation returns the documented status before anything is
  launched (so these calls are safe without a GPU);
* T == 0 is a successful no-op that accepts NULL tensors;
* workspace sizes are monotone in T, so a workspace sized for the largest
  microbatch serves every smaller one;
* the validation code, built alone with g++ and AddressSanitizer, passes a
  table of cases (host code only).
"""
import ctypes
import glob
import os
import re
import shutil
import subprocess

import pytest

import token_dispatch_grouped_amd as moe
from token_dispatch_grouped_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = sorted(glob.glob(os.path.join(ROOT, "include", "*.h")))
CSRC = os.path.join(ROOT, "token_dispatch_grouped_amd", "csrc")


def declared_functions():
    text = "".join(open(h).read() for h in HEADERS)
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = moe.load()
    names = declared_functions()
    assert len(names) >= 14
    for n in names:
        assert hasattr(lib, n), f"{n} declared in include/ but not exported"
    # and the binding wraps each of them
    assert set(names) <= set(L.exported_names())


def test_peak_probe_argument_rules():
    """The attainable-peak probes reject bad arguments before any launch."""
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_peak_mfma(FAKE, 0, stream=0)
    assert ei.value.status == L.MOE_ERR_INVALID_ARGUMENT
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_peak_mfma(FAKE + 4, 10, stream=0)
    assert ei.value.status == L.MOE_ERR_MISALIGNED
    for src, dst, n, st in ((FAKE, FAKE + (1 << 12), 100, L.MOE_ERR_INVALID_ARGUMENT),
                            (FAKE, FAKE + 16, 4096, L.MOE_ERR_INVALID_ARGUMENT),   # overlap
                            (FAKE + 8, FAKE + (1 << 16), 4096, L.MOE_ERR_MISALIGNED),
                            (None, FAKE, 4096, L.MOE_ERR_INVALID_ARGUMENT)):
        with pytest.raises(moe.MoeError) as ei:
            moe.moe_peak_copy(src, dst, n, stream=0)
        assert ei.value.status == st


def test_ep_argument_rules():
    """The expert-parallel calls validate before any launch."""
    s = shape(T=64, E=8, k=2)
    with pytest.raises(moe.MoeError) as ei:   # ep does not divide E
        moe.moe_ep_send_plan(s, 3, FAKE, FAKE, FAKE, FAKE, stream=0)
    assert ei.value.status == L.MOE_ERR_UNSUPPORTED
    with pytest.raises(moe.MoeError) as ei:   # more ranks than the stand-in holds
        moe.moe_ep_send_plan(shape(T=64, E=16, k=2), 16, FAKE, FAKE, FAKE, FAKE, stream=0)
    assert ei.value.status == L.MOE_ERR_UNSUPPORTED
    with pytest.raises(moe.MoeError) as ei:   # counts needed when T > 0
        moe.moe_ep_send_plan(s, 2, None, FAKE, FAKE, FAKE, stream=0)
    assert ei.value.status == L.MOE_ERR_INVALID_ARGUMENT and "counts" in str(ei.value)
    with pytest.raises(moe.MoeError) as ei:   # ep * e_local > 256
        moe.moe_ep_recv_plan(4, 65, 100, FAKE, FAKE, FAKE, FAKE, FAKE, stream=0)
    assert ei.value.status == L.MOE_ERR_UNSUPPORTED
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_ep_recv_plan(2, 4, -1, FAKE, FAKE, FAKE, FAKE, FAKE, stream=0)
    assert ei.value.status == L.MOE_ERR_INVALID_ARGUMENT
    with pytest.raises(moe.MoeError) as ei:   # one workgroup per row: at most 2^24 - 1 rows
        moe.moe_ep_recv_plan(2, 4, 1 << 24, FAKE, FAKE, FAKE, FAKE, FAKE, stream=0)
    assert ei.value.status == L.MOE_ERR_UNSUPPORTED
    with pytest.raises(moe.MoeError) as ei:   # overlapping regroup buffers
        moe.moe_ep_regroup(64, L.MOE_DTYPE_BF16, 100, 2, FAKE, FAKE, FAKE, FAKE + 256, stream=0)
    assert ei.value.status == L.MOE_ERR_INVALID_ARGUMENT and "overlap" in str(ei.value)
    with pytest.raises(moe.MoeError) as ei:   # d not a multiple of 64
        moe.moe_ep_regroup(96, L.MOE_DTYPE_BF16, 100, 2, FAKE, FAKE, FAKE, FAKE << 4, stream=0)
    assert ei.value.status == L.MOE_ERR_UNSUPPORTED
    with pytest.raises(moe.MoeError) as ei:   # a NULL receive buffer with rows to receive
        moe.moe_ep_exchange_loopback(2, 64, L.MOE_DTYPE_BF16, [FAKE, FAKE], [10, 10], [FAKE, FAKE], [FAKE, None],
                                     [20, 20], [FAKE, FAKE], stream=0)
    assert ei.value.status == L.MOE_ERR_INVALID_ARGUMENT and "recv_bufs" in str(ei.value)
    with pytest.raises(moe.MoeError) as ei:   # a NULL regroup map for a destination with capacity
        moe.moe_ep_exchange_loopback(2, 64, L.MOE_DTYPE_BF16, [FAKE, FAKE], [10, 10], [FAKE, FAKE], [FAKE, FAKE],
                                     [20, 20], [FAKE, FAKE], regroup_rows=[FAKE, None], stream=0)
    assert ei.value.status == L.MOE_ERR_INVALID_ARGUMENT and "regroup_rows" in str(ei.value)
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_ep_exchange_counts_loopback(2, 4, [FAKE, None], [FAKE, FAKE], stream=0)
    assert ei.value.status == L.MOE_ERR_INVALID_ARGUMENT
    # a zero-capacity regroup is a no-op that accepts NULL buffers
    moe.moe_ep_regroup(64, L.MOE_DTYPE_BF16, 0, 2, None, None, None, None, stream=0)


def test_version_and_status_strings():
    assert "gfx950" in moe.moe_version()
    assert moe.moe_status_string(0) == "ok"
    assert "workspace" in moe.moe_status_string(3)


def shape(T=64, d=64, E=4, k=2, F=128, dtype=L.MOE_DTYPE_BF16, flags=0):
    return L.make_shape(T, d, E, k, F, dtype, flags)


@pytest.mark.parametrize("kw,status", [
    (dict(k=5, E=4), L.MOE_ERR_INVALID_ARGUMENT),        # k > E
    (dict(T=-1), L.MOE_ERR_INVALID_ARGUMENT),
    (dict(d=0), L.MOE_ERR_INVALID_ARGUMENT),
    (dict(d=96), L.MOE_ERR_UNSUPPORTED),                 # not a multiple of 64
    (dict(F=100), L.MOE_ERR_UNSUPPORTED),
    (dict(E=257, k=2), L.MOE_ERR_UNSUPPORTED),
    (dict(E=32, k=17), L.MOE_ERR_UNSUPPORTED),
    (dict(dtype=7), L.MOE_ERR_UNSUPPORTED),
    (dict(flags=8), L.MOE_ERR_UNSUPPORTED),              # unknown flag bit
    (dict(T=2 ** 28, E=8, k=8), L.MOE_ERR_UNSUPPORTED),  # T*k >= 2^31
    (dict(T=2 ** 24, E=8, k=1), L.MOE_ERR_UNSUPPORTED),  # 256 threads per token: 2^32 threads
    (dict(T=2 ** 20, d=32768, E=8, k=1), L.MOE_ERR_UNSUPPORTED),  # T*d/8 = 2^32 chunks
    (dict(T=2 ** 19, d=32768, E=256, k=1, F=32768), L.MOE_ERR_UNSUPPORTED),  # weight-gradient grid
    # fp32 grouped GEMM: 16-wide tiles over 2^25 rows pass 2^32 threads
    (dict(T=2 ** 24 - 1, E=8, k=2, F=64, dtype=L.MOE_DTYPE_F32), L.MOE_ERR_UNSUPPORTED),
])
def test_shape_validation(kw, status):
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_workspace_size(shape(**kw))
    assert ei.value.status == status


def test_large_shapes_within_the_launch_bounds_are_accepted():
    # just inside each bound: 2^24 - 1 tokens, T*d/8 just under 2^32
    moe.moe_workspace_size(shape(T=2 ** 24 - 1, E=8, k=1))
    moe.moe_workspace_size(shape(T=2 ** 20 - 1, d=32768, E=8, k=1))
    # the routing test at the largest token count: bf16, top-2
    moe.moe_workspace_size(shape(T=2 ** 24 - 1, E=8, k=2, F=64))


def test_empty_microbatch_is_a_noop_with_nulls():
    s = shape(T=0)
    moe.moe_route(s, None, None, None, None, None, None, None, None, None, None, None, 0, stream=0)
    moe.moe_permute(s, None, None, None, stream=0)
    moe.moe_grouped_gemm_fwd(s, None, None, None, None, None, None, None, None, 0, stream=0)
    moe.moe_unpermute_combine(s, None, None, None, None, stream=0)
    moe.moe_unpermute_combine_bwd(s, None, None, None, None, None, None, stream=0)
    moe.moe_route_bwd(s, None, None, None, None, None, None, None, None, None, None, 0, stream=0)
    moe.moe_grouped_gemm_bwd(s, None, None, None, None, None, None, None, None, None, None, None, 0, stream=0)
    moe.moe_permute_bwd(s, None, None, None, None, stream=0)


def test_route_noalloc_argument_rules():
    """The allocation-free route validates like moe_route and rejects, before
    any launch, shapes whose histograms exceed its 16 MiB static scratch."""
    moe.moe_route_noalloc(shape(T=0), None, None, None, None, None, None, None, None, None, None, stream=0)
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_route_noalloc(shape(T=300), None, None, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, stream=0)
    assert ei.value.status == L.MOE_ERR_INVALID_ARGUMENT and "src_of_row" in str(ei.value)
    # ceil(T/64) * E * 4 bytes: 16385 workgroups of 256 experts is one past the 16 MiB
    big = shape(T=16384 * 64 + 1, E=256, k=8)
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_route_noalloc(big, None, None, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, stream=0)
    assert ei.value.status == L.MOE_ERR_UNSUPPORTED and "static scratch" in str(ei.value)


def test_empty_microbatch_still_validates_shape():
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_permute(shape(T=0, k=9, E=4), None, None, None, stream=0)
    assert ei.value.status == L.MOE_ERR_INVALID_ARGUMENT


FAKE = 1 << 20  # an aligned, never dereferenced address: validation fails first


def test_null_pointer_is_rejected():
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_permute(shape(), FAKE, None, FAKE, stream=0)
    assert ei.value.status == L.MOE_ERR_INVALID_ARGUMENT
    assert "row_of_slot" in str(ei.value)


def test_misaligned_pointer_is_rejected():
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_unpermute_combine(shape(), FAKE, FAKE + 4, FAKE, FAKE, stream=0)
    assert ei.value.status == L.MOE_ERR_MISALIGNED


def test_router_mode_argument_rules():
    s = shape()
    # logits given (no router): x must be NULL
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_route(s, FAKE, None, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 20, stream=0)
    assert ei.value.status == L.MOE_ERR_INVALID_ARGUMENT
    # router mode without x
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_route(s, None, FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 20, stream=0)
    assert ei.value.status == L.MOE_ERR_INVALID_ARGUMENT
    # route_bwd in router mode needs dx_router and dw_router
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_route_bwd(s, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, 1 << 20, stream=0)
    assert ei.value.status == L.MOE_ERR_INVALID_ARGUMENT


def test_workspace_rules():
    s = shape()
    route_ws, fwd_ws, bwd_ws = moe.moe_workspace_size(s)
    assert route_ws > 0 and bwd_ws > 0
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_route(s, None, None, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, route_ws - 1, stream=0)
    assert ei.value.status == L.MOE_ERR_WORKSPACE
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_grouped_gemm_bwd(s, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, stream=0)
    assert ei.value.status == L.MOE_ERR_WORKSPACE


@pytest.mark.parametrize("dtype", [L.MOE_DTYPE_BF16, L.MOE_DTYPE_F32])
def test_recompute_workspace_and_argument_rules(dtype):
    """MOE_FLAG_RECOMPUTE: the forward workspace holds a [R,F]; the backward
    workspace holds dH (over the recomputed h), the expert order and the
    recomputed a; h and a must be NULL in both calls."""
    T, d, E, k, F = 4096, 1024, 8, 2, 2816
    es = 2 if dtype == L.MOE_DTYPE_BF16 else 4
    R = T * k
    plain = moe.moe_workspace_size(shape(T, d, E, k, F, dtype))
    rc = moe.moe_workspace_size(shape(T, d, E, k, F, dtype, flags=L.MOE_FLAG_RECOMPUTE))
    align = lambda n: (n + 255) // 256 * 256
    assert plain[1] == 0 and rc[1] == align(R * F * es)
    assert rc[0] == plain[0]
    assert rc[2] == plain[2] + align(R * F * es)
    s = shape(T, d, E, k, F, dtype, flags=L.MOE_FLAG_RECOMPUTE)
    with pytest.raises(moe.MoeError) as ei:   # h given under recompute
        moe.moe_grouped_gemm_fwd(s, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, rc[1], stream=0)
    assert ei.value.status == L.MOE_ERR_INVALID_ARGUMENT and "h" in str(ei.value)
    with pytest.raises(moe.MoeError) as ei:   # forward workspace missing
        moe.moe_grouped_gemm_fwd(s, FAKE, FAKE, FAKE, FAKE, None, None, FAKE, None, 0, stream=0)
    assert ei.value.status == L.MOE_ERR_WORKSPACE
    with pytest.raises(moe.MoeError) as ei:   # a given under recompute
        moe.moe_grouped_gemm_bwd(s, FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, rc[2],
                                 stream=0)
    assert ei.value.status == L.MOE_ERR_INVALID_ARGUMENT and "a" in str(ei.value)
    with pytest.raises(moe.MoeError) as ei:   # backward workspace one byte short
        moe.moe_grouped_gemm_bwd(s, FAKE, FAKE, None, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, rc[2] - 1,
                                 stream=0)
    assert ei.value.status == L.MOE_ERR_WORKSPACE
    # without the flag, h and a are required
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_grouped_gemm_fwd(shape(T, d, E, k, F, dtype), FAKE, FAKE, FAKE, FAKE, None, None, FAKE, None, 0,
                                 stream=0)
    assert ei.value.status == L.MOE_ERR_INVALID_ARGUMENT


@pytest.mark.parametrize("dtype", [L.MOE_DTYPE_BF16, L.MOE_DTYPE_F32])
def test_workspace_monotone_in_T(dtype):
    prev = None
    for T in [0, 1, 7, 255, 256, 257, 4096, 7001, 16384, 32768]:
        ws = moe.moe_workspace_size(shape(T=T, d=2048, E=32, k=8, F=1408, dtype=dtype))
        if prev is not None:
            assert all(a >= b for a, b in zip(ws, prev)), (T, ws, prev)
        prev = ws
    # the gemm backward workspace holds dH: R * 2F elements of the layer dtype
    R = 32768 * 8
    es = 2 if dtype == L.MOE_DTYPE_BF16 else 4
    assert prev[2] >= R * 2 * 1408 * es


@pytest.mark.parametrize("kw,status", [
    (dict(lr=-1e-3), L.MOE_ERR_INVALID_ARGUMENT),
    (dict(beta1=1.0), L.MOE_ERR_INVALID_ARGUMENT),
    (dict(beta2=-0.1), L.MOE_ERR_INVALID_ARGUMENT),
    (dict(eps=0.0), L.MOE_ERR_INVALID_ARGUMENT),
    (dict(weight_decay=-0.5), L.MOE_ERR_INVALID_ARGUMENT),
    (dict(grad_scale=float("inf")), L.MOE_ERR_INVALID_ARGUMENT),
    (dict(lr=float("nan")), L.MOE_ERR_INVALID_ARGUMENT),
    (dict(step=0), L.MOE_ERR_INVALID_ARGUMENT),
])
def test_adamw_config_validation(kw, status):
    args = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01, grad_scale=1.0, step=1)
    args.update(kw)
    cfg = L.make_adamw_config(**args)
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_adamw_step(cfg, 16, FAKE, FAKE, FAKE, FAKE, None, stream=0)
    assert ei.value.status == status


def test_adamw_argument_rules():
    cfg = L.make_adamw_config(1e-3)
    moe.moe_adamw_step(cfg, 0, None, None, None, None, None, stream=0)  # n == 0: no-op, NULLs accepted
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_adamw_step(cfg, -1, FAKE, FAKE, FAKE, FAKE, None, stream=0)
    assert ei.value.status == L.MOE_ERR_INVALID_ARGUMENT
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_adamw_step(cfg, 1 << 35, FAKE, FAKE, FAKE, FAKE, None, stream=0)
    assert ei.value.status == L.MOE_ERR_UNSUPPORTED
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_adamw_step(cfg, 16, FAKE, None, FAKE, FAKE, None, stream=0)
    assert ei.value.status == L.MOE_ERR_INVALID_ARGUMENT and "grad" in str(ei.value)
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_adamw_step(cfg, 16, FAKE, FAKE, FAKE, FAKE, FAKE + 8, stream=0)
    assert ei.value.status == L.MOE_ERR_MISALIGNED
    bad = L.make_adamw_config(1e-3)
    bad.flags = 2
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_adamw_step(bad, 16, FAKE, FAKE, FAKE, FAKE, None, stream=0)
    assert ei.value.status == L.MOE_ERR_UNSUPPORTED


def test_aux_loss_argument_rules():
    s = shape(T=300, E=16, k=4)
    route_ws, _, _ = moe.moe_workspace_size(s)
    ok = L.make_aux_config(0.01, 1e-3)
    # T == 0 with no losses or metrics asked for, or nothing requested: no-op with NULLs
    moe.moe_aux_loss(shape(T=0, E=16, k=4), None, None, ok, None, None, None, None, 0, stream=0)
    moe.moe_aux_loss(s, None, None, ok, None, None, None, None, 0, stream=0)
    # T == 0 writes the zero losses, so its output pointers are validated first
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_aux_loss(shape(T=0, E=16, k=4), None, None, ok, FAKE + 4, None, None, None, 0, stream=0)
    assert ei.value.status == L.MOE_ERR_MISALIGNED
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_aux_loss(s, FAKE, FAKE, L.make_aux_config(float("nan"), 0.0), FAKE, None, None, FAKE, route_ws,
                         stream=0)
    assert ei.value.status == L.MOE_ERR_INVALID_ARGUMENT
    bad = L.make_aux_config(0.01, 0.0)
    bad.flags = 4
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_aux_loss(s, FAKE, FAKE, bad, FAKE, None, None, FAKE, route_ws, stream=0)
    assert ei.value.status == L.MOE_ERR_UNSUPPORTED
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_aux_loss(s, FAKE, None, ok, FAKE, None, None, FAKE, route_ws, stream=0)
    assert ei.value.status == L.MOE_ERR_INVALID_ARGUMENT and "counts" in str(ei.value)
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_aux_loss(s, FAKE, FAKE, ok, FAKE, None, None, None, 0, stream=0)
    assert ei.value.status == L.MOE_ERR_WORKSPACE
    # the route workspace covers the auxiliary pass at any T
    for T in (1, 255, 256, 257, 32768, 1 << 20):
        rw, _, _ = moe.moe_workspace_size(shape(T=T, E=256, k=8, d=64, F=64))
        blocks = -(-T // max(256, (-(-T // 1024) + 3) // 4 * 4))
        assert rw >= blocks * (256 + 3) * 4


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_validation_built_alone_with_asan(tmp_path):
    """The validation unit is plain C++: build it with g++ (no HIP) and
    AddressSanitizer, and check a table of cases."""
    driver = tmp_path / "drv.cpp"
    driver.write_text(r'''
#include "validate.h"
#include <cstdio>
using namespace moe;
static int fails = 0;
static void expect(moe_status got, moe_status want, const char* what) {
  if (got != want) { std::printf("FAIL %s: got %d want %d\n", what, (int)got, (int)want); ++fails; }
}
int main() {
  std::string why;
  moe_shape s{32768, 2048, 32, 8, 1408, MOE_DTYPE_BF16, 0};
  expect(validate_shape(&s, &why), MOE_OK, "ep share");
  expect(validate_shape(nullptr, &why), MOE_ERR_INVALID_ARGUMENT, "null shape");
  moe_shape b = s; b.E = 64; b.k = 33; expect(validate_shape(&b, &why), MOE_ERR_UNSUPPORTED, "k>16");
  b = s; b.k = 40; b.E = 32; expect(validate_shape(&b, &why), MOE_ERR_INVALID_ARGUMENT, "k>E");
  b = s; b.F = 1400; expect(validate_shape(&b, &why), MOE_ERR_UNSUPPORTED, "F%64");
  b = s; b.T = 0; expect(validate_shape(&b, &why), MOE_OK, "T=0");
  WorkspaceLayout w = workspace_layout(s);
  if (w.gemm_bwd_total < (size_t)32768 * 8 * 2 * 1408 * 2) { std::printf("FAIL dh size\n"); ++fails; }
  int x = 0;
  PtrArg ok[] = {{"a", (void*)0x1000, true, false}, {"b", nullptr, false, true}};
  expect(validate_ptrs(ok, 2, &why), MOE_OK, "ptrs ok");
  PtrArg mis[] = {{"a", (void*)0x1004, true, false}};
  expect(validate_ptrs(mis, 1, &why), MOE_ERR_MISALIGNED, "misaligned");
  PtrArg nul[] = {{"a", nullptr, true, false}};
  expect(validate_ptrs(nul, 1, &why), MOE_ERR_INVALID_ARGUMENT, "null");
  PtrArg must[] = {{"a", &x, false, true}};
  expect(validate_ptrs(must, 1, &why), MOE_ERR_INVALID_ARGUMENT, "must be null");
  moe_adamw_config ac{1e-3f, 0.9f, 0.999f, 1e-8f, 0.01f, 1.f, 1, 0};
  expect(validate_adamw(&ac, 100, &why), MOE_OK, "adamw ok");
  expect(validate_adamw(nullptr, 100, &why), MOE_ERR_INVALID_ARGUMENT, "adamw null");
  moe_adamw_config ab = ac; ab.step = 0; expect(validate_adamw(&ab, 100, &why), MOE_ERR_INVALID_ARGUMENT, "step 0");
  ab = ac; ab.beta2 = 1.f; expect(validate_adamw(&ab, 100, &why), MOE_ERR_INVALID_ARGUMENT, "beta2 1");
  ab = ac; ab.flags = 8; expect(validate_adamw(&ab, 100, &why), MOE_ERR_UNSUPPORTED, "adamw flag");
  expect(validate_adamw(&ac, (int64_t)1 << 35, &why), MOE_ERR_UNSUPPORTED, "adamw n");
  expect(validate_adamw(&ac, ((int64_t)1 << 35) - 1, &why), MOE_OK, "adamw n below the bound");
  expect(validate_workspace(nullptr, 0, 0, &why), MOE_OK, "no ws needed");
  expect(validate_workspace(nullptr, 0, 16, &why), MOE_ERR_WORKSPACE, "ws null");
  expect(validate_workspace((void*)0x1000, 8, 16, &why), MOE_ERR_WORKSPACE, "ws short");
  std::printf("%d failures\n", fails);
  return fails != 0;
}
''')
    exe = tmp_path / "drv"
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-omit-frame-pointer",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC, str(driver), os.path.join(CSRC, "validate.cpp"),
           "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "0 failures" in r.stdout
