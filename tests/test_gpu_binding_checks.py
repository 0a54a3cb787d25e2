"""The binding rejects buffers whose shape or dtype does not match the sizes
it hands to the library (which sees raw pointers only), before any launch."""
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def B():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from block_sparse_long_infllmv2_amd import binding
    return binding


def _prefill_args(n_q=8, n_k=256, h_q=4, h_kv=2, d=64):
    bf = dict(dtype=torch.bfloat16, device="cuda")
    q = torch.zeros((n_q, h_q, d), **bf)
    k = torch.zeros((h_kv, n_k, d), **bf)
    v = torch.zeros((h_kv, n_k, d), **bf)
    out = torch.empty_like(q)
    lse = torch.empty((n_q, h_q), dtype=torch.float32, device="cuda")
    return q, k, v, out, lse


def test_prefill_rejects_mismatched_buffers(B):
    p = B.default_params(dense_len=1 << 30)          # dense: no block list needed
    q, k, v, out, lse = _prefill_args()
    B.infllmv2_sparse_attn_prefill(q, k, v, 256, None, out, lse, p)   # well-formed: runs
    torch.cuda.synchronize()
    with pytest.raises(ValueError, match="out"):
        B.infllmv2_sparse_attn_prefill(q, k, v, 256, None, out[:4], lse, p)
    with pytest.raises(ValueError, match="v_cache"):
        B.infllmv2_sparse_attn_prefill(q, k, v[:, :128], 256, None, out, lse, p)
    with pytest.raises(TypeError, match="lse"):
        B.infllmv2_sparse_attn_prefill(q, k, v, 256, None, out, lse.double(), p)
    with pytest.raises(TypeError, match="k_cache"):
        B.infllmv2_sparse_attn_prefill(q, k.float(), v, 256, None, out, lse, p)
    bad_idx = torch.zeros((8, 2, 3), dtype=torch.int32, device="cuda")   # topk is 64
    with pytest.raises(ValueError, match="block_idx"):
        B.infllmv2_sparse_attn_prefill(q, k, v, 256, bad_idx, out, lse, p)


def test_decode_and_backward_reject_mismatched_buffers(B):
    p = B.default_params()
    batch, h_q, h_kv, d, cap = 2, 32, 2, 128, 512
    bf = dict(dtype=torch.bfloat16, device="cuda")
    q = torch.zeros((batch, h_q, d), **bf)
    k = torch.zeros((batch, h_kv, cap, d), **bf)
    seqlens = torch.tensor([100, 200], dtype=torch.int32, device="cuda")
    out = torch.empty_like(q)
    ws = torch.empty(1 << 20, dtype=torch.uint8, device="cuda")
    with pytest.raises(ValueError, match="seqlens"):
        B.infllmv2_sparse_attn_decode(q, k, k, seqlens[:1], 200, None, out, None, ws, p)
    with pytest.raises(TypeError, match="ws"):
        B.infllmv2_sparse_attn_decode(q, k, k, seqlens, 200, None, out, None,
                                      ws.view(torch.int32), p)
    n_q, n_k = 16, 512
    qq = torch.zeros((n_q, h_q, d), **bf)
    kk = torch.zeros((h_kv, n_k, d), **bf)
    lse = torch.empty((n_q, h_q), dtype=torch.float32, device="cuda")
    dk = torch.zeros((h_kv, n_k, d), dtype=torch.float32, device="cuda")
    with pytest.raises(ValueError, match="dv"):
        B.infllmv2_sparse_attn_prefill_backward(qq, kk, kk, n_k, None, qq, lse, qq,
                                                torch.empty_like(qq), dk, dk[:, :8], ws, p)
    with pytest.raises(ValueError, match="lse"):
        B.infllmv2_sparse_attn_prefill_backward(qq, kk, kk, n_k, None, qq, None, qq,
                                                torch.empty_like(qq), dk, dk, ws, p)
