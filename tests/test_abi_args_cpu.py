"""The binding's own argument checks (no GPU needed): every tensor handed to the C ABI
is checked for shape, dtype and contiguity before a pointer is taken, because the
library sees raw pointers only. Host tensors with the right shapes get past the checks
and are then refused for not living on the GPU; any wrong shape, dtype or layout is
refused first."""
import pytest
import torch

from bit_quantized_lora_fp4_amd import abi

M, N, K, R, S = 64, 96, 128, 16, 16


def _mx4(rows, cols):
    return abi.Mx4(torch.zeros((rows, cols // 2), dtype=torch.uint8),
                   torch.zeros(((rows + 31) // 32, cols // 32), dtype=torch.uint8), rows, cols)


def _lin(n=N, k=K, r=R, s=S):
    bf = torch.bfloat16
    return abi.Linear(_mx4(n, k), torch.zeros((r, k), dtype=bf), torch.zeros((n, r), dtype=bf),
                      torch.zeros((s, k), dtype=bf), torch.zeros((n, s), dtype=bf))


def _t(*shape, dtype=torch.bfloat16):
    return torch.zeros(shape, dtype=dtype)


def _fwd_args(**over):
    a = dict(L=_lin(), x=_t(M, K), y=_t(M, N, dtype=torch.float32), xl_saved=_t(M, R + S), ws=_t(1024, dtype=torch.uint8))
    a.update(over)
    return a


def _bwd_args(**over):
    a = dict(L=_lin(), dy=_t(M, N), x=_t(M, K), xl_saved=_t(M, R + S), dx=_t(M, K, dtype=torch.float32),
             d_lora_a=_t(R, K, dtype=torch.float32), d_lora_b=_t(N, R, dtype=torch.float32),
             ws=_t(1024, dtype=torch.uint8))
    a.update(over)
    return a


def _refused(fn, args, needle):
    with pytest.raises((ValueError, TypeError)) as e:
        fn(**args)
    assert needle in str(e.value), str(e.value)


def test_valid_host_arguments_pass_the_checks():
    _refused(abi.fourtune_linear_fwd, _fwd_args(), "must live on the GPU")
    _refused(abi.fourtune_linear_bwd, _bwd_args(), "must live on the GPU")


@pytest.mark.parametrize("over,needle", [
    (dict(x=_t(M, K + 32)), "x has shape"),
    (dict(x=_t(M, K, dtype=torch.float16)), "x has dtype"),
    (dict(x=_t(K, M).t()), "x must be contiguous"),
    (dict(y=_t(M, N - 32, dtype=torch.float32)), "y has shape"),
    (dict(y=_t(M + 1, N, dtype=torch.float32)), "y has shape"),
    (dict(xl_saved=_t(M, R + S, dtype=torch.float32)), "xl_saved has dtype"),
    (dict(xl_saved=None), "xl_saved is required"),
    (dict(ws=_t(16, 64, dtype=torch.uint8)), "ws must be"),
    (dict(L=abi.Linear(_mx4(N, K), _t(R, K, dtype=torch.float32), _t(N, R), _t(S, K), _t(N, S))), "L.A has dtype"),
    (dict(L=abi.Linear(_mx4(N, K), _t(R, K), _t(N, R + 16), _t(S, K), _t(N, S))), "L.B has shape"),
    (dict(L=abi.Linear(_mx4(N, K), _t(R, K), _t(N, R), _t(S, K - 32), _t(N, S))), "L.L1 has shape"),
    (dict(L=abi.Linear(_mx4(N, K), _t(R, K), _t(N, R), _t(S, K), _t(N - 32, S))), "L.L2 has shape"),
    (dict(L=abi.Linear(abi.Mx4(_t(N, K, dtype=torch.uint8), _t(3, 4, dtype=torch.uint8), N, K),
                       _t(R, K), _t(N, R), _t(S, K), _t(N, S))), "L.rq.codes has shape"),
])
def test_linear_fwd_refuses(over, needle):
    _refused(abi.fourtune_linear_fwd, _fwd_args(**over), needle)


@pytest.mark.parametrize("over,needle", [
    (dict(dy=_t(M, N + 32)), "dy has shape"),
    (dict(dx=_t(M, K, dtype=torch.float16)), "dx has dtype"),
    (dict(d_lora_a=_t(R, K)), "d_lora_a has dtype"),
    (dict(d_lora_b=_t(N, R + 1, dtype=torch.float32)), "d_lora_b has shape"),
    (dict(d_lora_b=None), "d_lora_b is required"),
    (dict(xl_saved=_t(M - 1, R + S)), "xl_saved has shape"),
])
def test_linear_bwd_refuses(over, needle):
    _refused(abi.fourtune_linear_bwd, _bwd_args(**over), needle)


def test_rank_zero_gradients_may_be_omitted():
    L = _lin(r=0)
    _refused(abi.fourtune_linear_bwd, _bwd_args(L=L, xl_saved=_t(M, S), d_lora_a=None, d_lora_b=None),
             "must live on the GPU")


def test_quantized_operand_and_mlp_checks():
    L = _lin()
    _refused(abi.fourtune_linear_fwd, _fwd_args(xq_out=_mx4(M, K + 32)), "xq_out is")
    fc1, fc2 = _lin(n=256, k=K), _lin(n=K, k=256)
    base = dict(fc1=fc1, fc2=fc2, x=_t(M, K), y=_t(M, K), xl1_saved=_t(M, R + S), pre_saved=_t(M, 256),
                hl2_saved=_t(M, R + S), ws=_t(64, dtype=torch.uint8))
    _refused(abi.fourtune_mlp_fwd, base, "must live on the GPU")
    _refused(abi.fourtune_mlp_fwd, dict(base, fc1=fc2), "outputs")
    _refused(abi.fourtune_mlp_fwd, dict(base, pre_saved=_t(M, 256, dtype=torch.float32)), "pre_saved has dtype")
    _refused(abi.fourtune_mlp_fwd, dict(base, h_debug=_t(M, 256)), "h_debug has dtype")
    bwd = dict(fc1=fc1, fc2=fc2, dy=_t(M, K), x=_t(M, K), xl1_saved=_t(M, R + S), pre_saved=_t(M, 256),
               hl2_saved=_t(M, R + S), dx=_t(M, K), d_a1=_t(R, K, dtype=torch.float32),
               d_b1=_t(256, R, dtype=torch.float32), d_a2=_t(R, 256, dtype=torch.float32),
               d_b2=_t(K, R, dtype=torch.float32), ws=_t(64, dtype=torch.uint8))
    _refused(abi.fourtune_mlp_bwd, bwd, "must live on the GPU")
    _refused(abi.fourtune_mlp_bwd, dict(bwd, d_a2=_t(R, K, dtype=torch.float32)), "d_a2 has shape")
    _refused(abi.fourtune_mlp_bwd, dict(bwd, dp_debug=_t(M, 255, dtype=torch.float32)), "dp_debug has shape")
    _refused(abi.fourtune_gemm_fwd, dict(L=L, xq=_mx4(M, K), xl=_t(M, R + S), y=_t(M, N + 32)), "y has shape")
    _refused(abi.fourtune_gemm_bwd, dict(L=L, gq=_mx4(M, N), gb=_t(M, R), dx=_t(M, K)), "gb has shape")
    _refused(abi.fourtune_linear_fwd_prec, dict(prec="W4A16G4", **_fwd_args(x=_t(M, K - 32))), "x has shape")
    _refused(abi.fourtune_linear_bwd_unfused, _bwd_args(dx=_t(M, K + 32)), "dx has shape")


def test_quantize_checks():
    x = _t(M, K)
    _refused(abi.fourtune_quantize, dict(x=x, out=_mx4(M, K)), "must live on the GPU")
    _refused(abi.fourtune_quantize, dict(x=x, out=_mx4(M, K + 32)), "out is")
    _refused(abi.fourtune_quantize, dict(x=_t(M, K, dtype=torch.float16), out=_mx4(M, K)), "x has dtype")
    _refused(abi.fourtune_quantize, dict(x=_t(K, M).t(), out=_mx4(M, K)), "unit column stride")
    _refused(abi.fourtune_quantize_groups, dict(x=x, out=_mx4(M, K)), "out.scales has shape")
    _refused(abi.fourtune_quantize_groups, dict(x=x, out=abi.Mx4.empty_groups(M, K, device="cpu")),
             "must live on the GPU")
