"""The Python binding's refusals that need device tensors: strided views,
wrong element types and buffers shorter than the sizes passed with them.
Each refusal is raised before the library is called, so no kernel runs on
a bad buffer; a good call right after each one shows nothing was left
behind."""
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def m():
    from gemm_mxfp4_dequant_amd import mxfp4
    mxfp4.lib()
    return mxfp4


def nb(rows, cols):
    return rows * cols // 2 + rows * cols // 32


def test_gemm_refusals(m):
    rows, cols, b = 64, 512, 4
    w = torch.zeros(nb(rows, cols), dtype=torch.uint8, device="cuda")
    x = torch.zeros((b, cols), device="cuda")
    bad = [
        (ValueError, lambda: m.mxfp4_gemm(w[:-1], rows, cols, x)),                # short w
        (TypeError, lambda: m.mxfp4_gemm(w.view(torch.int8), rows, cols, x)),     # w dtype
        (ValueError, lambda: m.mxfp4_gemm(w, rows, cols, x[:, :256])),            # strided x
        (ValueError, lambda: m.mxfp4_gemm(w, rows, cols, x, b=5)),                # short x
        (TypeError, lambda: m.mxfp4_gemm(w, rows, cols, x.half())),               # x dtype
        (ValueError, lambda: m.mxfp4_gemm(w, rows, cols, x,
                                          y=torch.empty((b, rows - 1), device="cuda"))),
        (TypeError, lambda: m.mxfp4_gemm(w, rows, cols, x,
                                         y=torch.empty((b, rows), device="cuda",
                                                       dtype=torch.float16))),
        (ValueError, lambda: m.mxfp4_matvec(w, rows, cols, x[0, :100])),
        (TypeError, lambda: m.mxfp4_matvec(w, rows, cols, x[0].bfloat16())),
        (ValueError, lambda: m.mxfp4_dequant(w, rows, cols,
                                             out=torch.empty(rows * cols - 1, device="cuda"))),
    ]
    for i, (exc, f) in enumerate(bad):
        with pytest.raises(exc):
            f()
    y = m.mxfp4_gemm(w, rows, cols, x)
    torch.cuda.synchronize()
    assert torch.all(y == 0)


def test_expert_bank_refusals(m):
    E, H, I, T, K = 4, 512, 256, 3, 2
    bank = torch.zeros(E * nb(I, H), dtype=torch.uint8, device="cuda")
    down = torch.zeros(E * nb(H, I), dtype=torch.uint8, device="cuda")
    ids = torch.zeros((T, K), dtype=torch.int32, device="cuda")
    wr = torch.full((T, K), 0.5, device="cuda")
    x = torch.zeros((T, H), device="cuda")
    ws_need = m.moe_experts_mxfp4_workspace_size(T, K, E, H, I, torch.float32)
    bad = [
        (ValueError, lambda: m.moe_experts_mxfp4(bank[:-16], bank, down, E, H, I, x, ids, wr)),
        (ValueError, lambda: m.moe_experts_mxfp4(bank, bank, down[:-1], E, H, I, x, ids, wr)),
        (TypeError, lambda: m.moe_experts_mxfp4(bank, bank, down, E, H, I, x, ids.long(), wr)),
        (ValueError, lambda: m.moe_experts_mxfp4(bank, bank, down, E, H, I, x, ids, wr[:, :1])),
        (TypeError, lambda: m.moe_experts_mxfp4(bank, bank, down, E, H, I, x, ids, wr.half())),
        (ValueError, lambda: m.moe_experts_mxfp4(bank, bank, down, E, H, I, x[:2], ids, wr)),
        (ValueError, lambda: m.moe_experts_mxfp4(
            bank, bank, down, E, H, I, x, ids, wr,
            out=torch.empty((T, H - 1), dtype=torch.bfloat16, device="cuda"))),
        (ValueError, lambda: m.moe_experts_mxfp4(
            bank, bank, down, E, H, I, x, ids, wr,
            workspace=torch.empty(ws_need - 1, dtype=torch.uint8, device="cuda"))),
        (ValueError, lambda: m.moe_experts_mxfp4_stages(
            bank, bank, down, E, H, I, x, ids, wr,
            h_out=torch.empty((T * K, I - 1), device="cuda"))),
        (TypeError, lambda: m.moe_experts_mxfp4_stages(
            bank, bank, down, E, H, I, x, ids, wr,
            h_out=torch.empty((T * K, I), dtype=torch.bfloat16, device="cuda"))),
        # V4.1 with a shared expert needs n_experts + 1 tensors per role
        (ValueError, lambda: m.moe_experts_mxfp4_v41(bank, bank, down, E, H, I, x.bfloat16(),
                                                     ids, wr, has_shared=True)),
        (TypeError, lambda: m.moe_experts_mxfp4_v41(bank, bank, down, E, H, I, x, ids, wr)),
        (ValueError, lambda: m.moe_route_group(ids, E,
                                               offsets=torch.empty(E, dtype=torch.int32,
                                                                   device="cuda"))),
        (TypeError, lambda: m.moe_route_topk(torch.zeros((T, E), device="cuda").double(), K)),
    ]
    for i, (exc, f) in enumerate(bad):
        with pytest.raises(exc):
            f()
    out = m.moe_experts_mxfp4(bank, bank, down, E, H, I, x, ids, wr)
    torch.cuda.synchronize()
    assert torch.all(out == 0)
