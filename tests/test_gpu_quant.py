"""GPU parity of the online per-tensor e4m3 quantisation (bslp_quantize_e4m3)
and of the fp8 pipeline fed by it through device-side scales, against the
oracle, through the C ABI.

Bar: codes and scales bit-exact (the oracle takes the same float32 decisions);
the prefill on the device-quantised inputs as the fp8 parity bar (selections
bit-exact outside the band, outputs <= 2e-2) against the oracle run on the
oracle's own quantisation of the same bf16 inputs."""
import numpy as np
import pytest

import oracle
from harness import assert_parity, compare, log
from workloads import Workload, make_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_sparse_long_pooled_amd as bslp
    bslp.load_library()


def gpu_quantize(x):
    import torch

    import block_sparse_long_pooled_amd as bslp
    xd = x.cuda()
    codes = torch.full((max(1, x.numel()),), 0x55, dtype=torch.uint8, device="cuda")
    scale = torch.full((1,), float("nan"), dtype=torch.float32, device="cuda")
    bslp.quantize_e4m3(xd.reshape(-1), codes, scale)
    torch.cuda.synchronize()
    return codes[:x.numel()].cpu().numpy(), np.float32(scale.cpu().item())


@pytest.mark.parametrize("n", [1, 7, 8, 4099, 1 << 20])
@pytest.mark.parametrize("src", ["bf16", "f32"])
def test_quantize_bit_exact(n, src):
    import torch
    rng = np.random.default_rng(n)
    x = (rng.standard_normal(n) * rng.choice([1e-3, 1.0, 50.0], n)).astype(np.float32)
    x[rng.integers(0, n, max(1, n // 1000))] *= 30  # outliers set the scale
    t = torch.from_numpy(x)
    if src == "bf16":
        t = t.to(torch.bfloat16)
    ref_codes, ref_scale = oracle.quantize_per_tensor(t.float().numpy())
    codes, scale = gpu_quantize(t)
    log(f"[quant] {src} n={n} scale={scale!r} ref={ref_scale!r} "
        f"mismatch={int((codes != ref_codes).sum())}")
    assert scale.view(np.uint32) == ref_scale.view(np.uint32)
    assert np.array_equal(codes, ref_codes)


def test_quantize_all_zero_and_signed_zero():
    import torch
    x = torch.tensor([0.0, -0.0, 0.0, -0.0, 0.0, 0.0, -0.0, 0.0, 0.0], dtype=torch.bfloat16)
    codes, scale = gpu_quantize(x)
    assert scale == 1.0
    assert codes.tolist() == oracle.encode_e4m3fn(x.float().numpy()).tolist()


ONLINE = [
    Workload("online-fp8-g8", (1300, 640), 16, 2, 128, 128, "bf16", sigma_c=1.5),
    Workload("online-fp8-paged-b64", (700, 260), 8, 2, 64, 64, "bf16", page_size=16),
]


@pytest.mark.parametrize("w", ONLINE, ids=lambda w: w.name)
def test_online_fp8_pipeline(w):
    import torch

    import block_sparse_long_pooled_amd as bslp
    inp = make_inputs(w, 21)  # bf16 inputs
    # device side: quantise the tensors the kernels read, scales stay on the GPU
    dev = {name: getattr(inp, name).cuda() for name in ("q", "k", "v")}
    codes = {name: torch.empty(t.shape, dtype=torch.uint8, device="cuda") for name, t in dev.items()}
    scales = torch.full((3,), float("nan"), dtype=torch.float32, device="cuda")
    for i, name in enumerate(("q", "k", "v")):
        bslp.quantize_e4m3(dev[name].reshape(-1), codes[name].reshape(-1), scales[i:i + 1])
    table = torch.from_numpy(inp.table).cuda() if inp.table is not None else None
    fw = w.replace(dtype="fp8")
    prob = bslp.make_problem("fp8", w.hq, w.hkv, w.d, w.block, w.seqlens, softmax_scale=w.scale,
                             page_table=table, page_size=w.page_size, scales_dev=scales)
    params = bslp.make_params(w.alpha, w.sink, w.window, w.recent, w.correction)
    bufs = bslp.prefill(prob, params, codes["q"], codes["k"], codes["v"])
    torch.cuda.synchronize()
    # oracle side: its own quantisation of the same bf16 values (logical K/V;
    # unused pages are zero, so the physical and logical scales agree)
    k_log = inp.k_logical if inp.k_logical is not None else inp.k
    v_log = inp.v_logical if inp.v_logical is not None else inp.v
    oq = {n: oracle.quantize_per_tensor(t.float().numpy()) for n, t in
          (("q", inp.q), ("k", k_log), ("v", v_log))}
    got_scales = scales.cpu().numpy()
    for i, n in enumerate(("q", "k", "v")):
        assert got_scales[i].view(np.uint32) == oq[n][1].view(np.uint32), n
    assert np.array_equal(codes["q"].cpu().numpy(), oq["q"][0])
    ref = make_inputs(fw, 21)  # shapes and page table; values replaced below
    ref.q = torch.from_numpy(oq["q"][0])
    ref.q_scale, ref.k_scale, ref.v_scale = (float(oq[n][1]) for n in ("q", "k", "v"))
    if ref.k_logical is not None:
        ref.k_logical, ref.v_logical = torch.from_numpy(oq["k"][0]), torch.from_numpy(oq["v"][0])
    else:
        ref.k, ref.v = torch.from_numpy(oq["k"][0]), torch.from_numpy(oq["v"][0])
    from harness import GpuResult
    c = lambda t: t.cpu().numpy()
    g = GpuResult(c(bufs.kbar), c(bufs.vbar), c(bufs.scores), c(bufs.counts), c(bufs.cu),
                  c(bufs.idx), c(bufs.out.float()), c(bufs.lse))
    rep = compare(fw, ref, g)
    log(f"[online-fp8] {w.name}: {rep}")
    assert_parity(fw, rep)
