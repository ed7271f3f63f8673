"""Host-resident experts: moe_experts_mxfp4_ptrs reads each expert through a
table of per-expert pointers, so some experts can live in pinned host
memory (the experts a card's memory does not hold: "cortiq-engine 0.8.77,
src/qtensor/moe_fast.rs", module contract; "cortiq-engine 0.8.40,
src/gpu_wgpu/mxfp4.rs", global_bank_case).  The GPU reads their weights over
the host link with the same kernels, so the output must equal
moe_experts_mxfp4's on the same weights bit for bit; the bank itself is
pinned by the oracle tests of moe_experts_mxfp4."""
import numpy as np
import pytest
import torch

from gemm_mxfp4_dequant_amd import inputs
from tests.helpers import dev, host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def m():
    from gemm_mxfp4_dequant_amd import mxfp4
    mxfp4.lib()
    return mxfp4


def split_bank(bank, n_experts, nb, host_experts):
    """Per-expert tensors: experts in ``host_experts`` in pinned host memory,
    the others on the device."""
    out = []
    for e in range(n_experts):
        src = torch.from_numpy(np.ascontiguousarray(bank[e * nb:(e + 1) * nb]))
        if e in host_experts:
            t = torch.empty(nb, dtype=torch.uint8, pin_memory=True)
            t.copy_(src)
        else:
            t = src.cuda()
        out.append(t)
    return out


def run_both(m, c, E, H, I, host_experts):
    d = {k: dev(v) for k, v in c.items()}
    ref = host(m.moe_experts_mxfp4(d["gate"], d["up"], d["down"], E, H, I, d["x"], d["ids"],
                                   d["w"]))
    nb_gu, nb_dn = m.mxfp4_nbytes(I, H), m.mxfp4_nbytes(H, I)
    gates = split_bank(c["gate"], E, nb_gu, host_experts)
    ups = split_bank(c["up"], E, nb_gu, host_experts)
    downs = split_bank(c["down"], E, nb_dn, host_experts)
    tg = m.expert_table(gates, I, H)
    tu = m.expert_table(ups, I, H)
    td = m.expert_table(downs, H, I)
    got = host(m.moe_experts_mxfp4_ptrs(tg, tu, td, E, H, I, d["x"], d["ids"], d["w"]))
    torch.cuda.synchronize()
    return ref, got


@pytest.mark.parametrize("xd", ["f32", "bf16"])
def test_some_experts_in_host_memory(m, xd):
    E, H, I, T, K = 8, 1024, 512, 12, 3
    c = inputs.moe_case(71, E, H, I, T, K, xd, "softmax", scale_lo=100, scale_hi=114)
    ref, got = run_both(m, c, E, H, I, {0, 3, 5})
    assert np.array_equal(ref, got)


def test_many_tokens_tiled_kernels(m):
    """Tens of tokens per expert (the tiled kernels) with the hottest expert
    host-resident."""
    E, H, I, T, K = 4, 1024, 512, 96, 2
    c = inputs.moe_case(72, E, H, I, T, K, "bf16", "softmax", scale_lo=100, scale_hi=114)
    hot = int(np.bincount(c["ids"].reshape(-1), minlength=E).argmax())
    ref, got = run_both(m, c, E, H, I, {hot})
    assert np.array_equal(ref, got)


def test_decode_layer_with_cold_experts(m):
    """The 64-expert decode layer's shapes with its four most-routed experts
    host-resident, and every expert host-resident."""
    E, H, I, T, K = 64, 4096, 2048, 8, 6
    c = inputs.moe_case(73, E, H, I, T, K, "f32", "softmax")
    cnt = np.bincount(c["ids"].reshape(-1), minlength=E)
    hot = set(int(e) for e in np.argsort(-cnt, kind="stable")[:4])
    ref, got = run_both(m, c, E, H, I, hot)
    assert np.array_equal(ref, got)
    ref2, got2 = run_both(m, c, E, H, I, set(range(E)))
    assert np.array_equal(ref2, got2) and np.array_equal(ref, ref2)


def test_device_address_and_table_refusals(m):
    nb = m.mxfp4_nbytes(64, 512)
    d = torch.zeros(nb, dtype=torch.uint8, device="cuda")
    assert m.mxfp4_device_address(d) == d.data_ptr()
    p = torch.zeros(nb, dtype=torch.uint8, pin_memory=True)
    assert m.mxfp4_device_address(p) != 0
    pageable = torch.zeros(nb, dtype=torch.uint8)
    with pytest.raises(m.Mxfp4Error):
        m.mxfp4_device_address(pageable)
    with pytest.raises(ValueError, match="pinned"):
        m.expert_table([d, pageable], 64, 512)
    with pytest.raises(ValueError):
        m.expert_table([d[:-1]], 64, 512)
    with pytest.raises(ValueError):
        m.expert_table([p[:-16]], 64, 512)
