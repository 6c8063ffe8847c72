"""Parity of the fused AdamW update (moe_adamw_step, through the C ABI)
with the fp64 oracle (oracle.adamw_step), and one full training step of the
layer: forward, backward, optimizer update, next forward.

Bars: the weight change theta_new - theta_old within 1e-4 * max|ref change|
plus one fp32 ulp of theta_new per element (theta is stored in fp32, so its
new value carries that rounding whatever the size of the change: an element
whose change is pure weight decay moves by ~1e-8 of theta); the moments
within max|gpu - ref| / max|ref| <= 1e-4 (fp32 arithmetic); the bf16 working copy
bit-exact against nearest-even rounding of the GPU's own fp32 weights (the
rounding decision is taken in the kernel's precision on both sides); a
zeroed gradient exactly zero, an untouched one bit-identical.
"""
import numpy as np
import pytest

import oracle
from tests.parity_util import TOL, assert_close, to_device, to_host64
from workloads import BF16, F32, WORKLOADS, f32_to_bf16_bits, make_inputs, small_workload, to_f64

pytestmark = pytest.mark.gpu

TOL_F32 = TOL[F32]


def assert_update_close(name, new_gpu32, old32, new_ref64):
    """Per element: |(new_gpu - old) - (new_ref - old)| <= 1e-4 max|new_ref - old|
    + ulp32(max(|old|, |new_gpu|)): the kernel rounds twice in fp32 (theta times
    the decay factor, then the subtraction of the step), half an ulp each."""
    new_gpu32 = np.asarray(new_gpu32, dtype=np.float32)
    old32 = np.asarray(old32, dtype=np.float32)
    d_gpu = new_gpu32.astype(np.float64) - old32.astype(np.float64)
    d_ref = new_ref64 - old32.astype(np.float64)
    allow = TOL_F32 * np.max(np.abs(d_ref)) + np.spacing(np.maximum(np.abs(old32), np.abs(new_gpu32))).astype(
        np.float64)
    err = np.abs(d_gpu - d_ref)
    worst = int(np.argmax(err - allow))
    assert np.all(err <= allow), (f"{name}: element {worst} change {d_gpu[worst]:.6e} vs {d_ref[worst]:.6e} "
                                  f"(allowed {allow[worst]:.2e})")


def _moe():
    import token_dispatch_grouped_amd as m
    return m


def _state(n, seed):
    rng = np.random.default_rng(seed)
    theta = rng.normal(0, 0.02, n).astype(np.float32)
    grads = []
    for i in range(3):
        g = (rng.normal(0, 1e-3, n) * (1 + i)).astype(np.float32)
        g[i::11] = 0.0  # exactly zero gradients on some elements
        grads.append(g)
    return theta, grads


def _run_steps(n, seed, lr=1e-3, betas=(0.9, 0.95), eps=1e-8, wd=0.01, scale=0.5, zero_grad=True, lowp=True):
    import torch
    m = _moe()
    theta, grads = _state(n, seed)
    th_d = torch.from_numpy(theta.copy()).cuda()
    m_d = torch.zeros(n, device="cuda")
    v_d = torch.zeros(n, device="cuda")
    bf_d = torch.zeros(n, dtype=torch.bfloat16, device="cuda") if lowp else None
    th_o, m_o, v_o = theta.astype(np.float64), np.zeros(n), np.zeros(n)
    for t, g in enumerate(grads, start=1):
        g_d = torch.from_numpy(g.copy()).cuda()
        before = th_d.clone()
        cfg = m.make_adamw_config(lr, betas[0], betas[1], eps, wd, scale, t, zero_grad)
        m.moe_adamw_step(cfg, n, th_d, g_d, m_d, v_d, bf_d)
        torch.cuda.synchronize()
        th_o_new, m_o, v_o = oracle.adamw_step(th_o, g.astype(np.float64), m_o, v_o, t, lr, betas[0], betas[1],
                                               eps, wd, grad_scale=scale)
        if n:
            # the oracle runs its own chain from the same start; compare this
            # step's change from the GPU's previous weights
            assert_update_close(f"step {t} theta", th_d.cpu().numpy(), before.cpu().numpy(),
                                before.double().cpu().numpy() + (th_o_new - th_o))
            assert_close(f"step {t} exp_avg", to_host64(m_d), m_o, TOL_F32)
            assert_close(f"step {t} exp_avg_sq", to_host64(v_d), v_o, TOL_F32)
            if lowp:
                want = f32_to_bf16_bits(th_d.cpu().numpy())
                got = bf_d.view(torch.int16).cpu().numpy().view(np.uint16)
                assert np.array_equal(got, want), "bf16 copy is not the nearest-even rounding of theta"
            if zero_grad:
                assert bool((g_d == 0).all()), "gradient not zeroed"
            else:
                assert torch.equal(g_d, torch.from_numpy(g).cuda()), "gradient changed without ZERO_GRAD"
        th_o = th_o_new


def test_adamw_three_steps_ragged_tail():
    print("[adamw] n=1000003, 3 steps", flush=True)
    _run_steps(1_000_003, seed=41)


@pytest.mark.parametrize("n", [0, 1, 3, 4, 5, 511, 512, 513, 2049])
def test_adamw_small_sizes(n):
    _run_steps(n, seed=42 + n)


def test_adamw_no_copy_no_zeroing_no_decay():
    _run_steps(4099, seed=43, wd=0.0, scale=1.0, zero_grad=False, lowp=False)


def test_adamw_fullsize_expert_weights():
    """One update of the gate/up weights of the 32k EP-share layer
    (E*2F*d = 184.5M elements): sampled elements against the oracle, the
    bf16 copy and the zeroed gradient checked in full on the device."""
    import torch
    m = _moe()
    w = WORKLOADS["ep_share_32k"]
    n = w.E * 2 * w.F * w.d
    print(f"[adamw] full size n={n}", flush=True)
    gen = torch.Generator(device="cuda").manual_seed(5)
    th = torch.randn(n, device="cuda", generator=gen) * 0.02
    g = torch.randn(n, device="cuda", generator=gen) * 1e-3
    mo = torch.randn(n, device="cuda", generator=gen).abs_() * 1e-4
    vo = torch.randn(n, device="cuda", generator=gen).square_() * 1e-7
    idx = torch.from_numpy(np.random.default_rng(6).integers(0, n, 200_000)).cuda()
    s_th, s_g, s_m, s_v = (to_host64(a[idx]) for a in (th, g, mo, vo))
    bf = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    t = 7
    cfg = m.make_adamw_config(2e-4, 0.9, 0.95, 1e-8, 0.1, 1.0 / 4, t, True)
    m.moe_adamw_step(cfg, n, th, g, mo, vo, bf)
    torch.cuda.synchronize()
    r_th, r_m, r_v = oracle.adamw_step(s_th, s_g, s_m, s_v, t, 2e-4, 0.9, 0.95, 1e-8, 0.1, grad_scale=0.25)
    assert_update_close("theta (sampled)", th[idx].cpu().numpy(), s_th, r_th)
    assert_close("exp_avg (sampled)", to_host64(mo[idx]), r_m, TOL_F32)
    assert_close("exp_avg_sq (sampled)", to_host64(vo[idx]), r_v, TOL_F32)
    assert torch.equal(bf, th.to(torch.bfloat16)), "bf16 copy is not the nearest-even rounding of theta"
    assert bool((g == 0).all())


def test_training_step_forward_backward_update_forward():
    """Forward, backward, AdamW on the accumulated dW (two microbatches),
    then the next forward on the updated bf16 weights; the update is checked
    against the oracle's AdamW of the same dW, the second forward against
    the oracle layer on the updated weights."""
    import torch
    m = _moe()
    from token_dispatch_grouped_amd.layer import MoeLayer
    from token_dispatch_grouped_amd.optim import ExpertAdamW
    w = small_workload(640, 256, 8, 2, 192, BF16, "zipf", seed=44, n_empty=1, micro_T=(640, 0, 301))
    inp = make_inputs(w)
    W = inp["weights"]
    wgu, wdn = to_device(W["w_gu"], BF16), to_device(W["w_down"], BF16)
    layer = MoeLayer(640, w.d, w.E, w.k, w.F, m.MOE_DTYPE_BF16)
    dgu = torch.zeros(w.E, 2 * w.F, w.d, device="cuda")
    ddn = torch.zeros(w.E, w.d, w.F, device="cuda")
    opt = ExpertAdamW([wgu, wdn], lr=1e-3, betas=(0.9, 0.95), eps=1e-8, weight_decay=0.1)
    for mb in inp["micro"]:
        T = mb["x"].shape[0]
        layer.forward(T, to_device(mb["x"], BF16), wgu, wdn, logits=to_device(mb["logits"], F32))
        layer.backward(T, to_device(mb["dout"], BF16), wgu, wdn, dgu, ddn)
    torch.cuda.synchronize()
    g_gu, g_dn = to_host64(dgu), to_host64(ddn)
    opt.step([dgu, ddn], grad_scale=0.5)
    torch.cuda.synchronize()
    assert bool((dgu == 0).all()) and bool((ddn == 0).all())
    for name, w0, g, mst, wt in (("w_gu", W["w_gu"], g_gu, opt.master[0], wgu),
                                 ("w_down", W["w_down"], g_dn, opt.master[1], wdn)):
        th0 = to_f64(w0, BF16)
        ref, _, _ = oracle.adamw_step(th0, g, np.zeros_like(th0), np.zeros_like(th0), 1, 1e-3, 0.9, 0.95, 1e-8,
                                      0.1, grad_scale=0.5)
        assert_update_close(f"{name} update", mst.cpu().numpy(), th0, ref)
        assert torch.equal(wt, mst.to(torch.bfloat16)), f"{name} working copy"
    # the next forward runs on the updated weights
    mb = inp["micro"][0]
    sv = layer.forward(640, to_device(mb["x"], BF16), wgu, wdn, logits=to_device(mb["logits"], F32))
    torch.cuda.synchronize()
    out, _ = oracle.layer_fwd(to_f64(mb["x"], BF16), to_host64(wgu), to_host64(wdn), w.k,
                              logits=mb["logits"].astype(np.float64))
    assert_close("out after update", to_host64(sv.out), out, TOL[BF16])
