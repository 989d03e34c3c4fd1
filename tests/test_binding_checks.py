"""The Python binding's argument checks (CPU only). The C ABI takes plain
pointers and cannot see buffer sizes, so the binding checks every tensor it
passes (shape, dtype, contiguity, then one GPU) and raises before anything
reaches the library; these tests use CPU tensors, which the shape checks see
first and the device check refuses last."""
import pytest
import torch

import causal_flashattention_prefill_amd as zy

B, S, H, Hk, D = 1, 64, 4, 2, 128


def _qkv(dtype=torch.bfloat16, layout="bshd", sk=S, dv=128):
    shp = (lambda s, h, d: (B, s, h, d)) if layout == "bshd" else (lambda s, h, d: (B, h, s, d))
    return (torch.zeros(shp(S, H, D), dtype=dtype), torch.zeros(shp(sk, Hk, D), dtype=dtype),
            torch.zeros(shp(sk, Hk, dv), dtype=dtype))


def test_fwd_refuses_a_shorter_key_tensor():
    q, _, _ = _qkv()
    _, k, v = _qkv(sk=S - 1)
    with pytest.raises(ValueError, match="k: shape"):
        zy.zyfa_fwd(q, k, v)


def test_fwd_refuses_mismatched_v_and_dtypes():
    q, k, _ = _qkv()
    with pytest.raises(ValueError, match="v: shape"):
        zy.zyfa_fwd(q, k, torch.zeros((B, S, Hk + 1, 128), dtype=torch.bfloat16))
    q8, k8, v8 = _qkv(torch.float8_e4m3fn)
    with pytest.raises(TypeError, match="k: dtype"):
        zy.zyfa_fwd(q, k8, v8)
    with pytest.raises(TypeError, match="unsupported input dtype"):
        zy.zyfa_fwd(q.float(), k.float(), k.float())


@pytest.mark.parametrize("layout", ["bshd", "bhsd"])
def test_fwd_refuses_wrong_out_and_lse(layout):
    q, k, v = _qkv(layout=layout)
    bad_out = torch.zeros((B, S, H, 64), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="out: shape"):
        zy.zyfa_fwd(q, k, v, bad_out, layout=layout)
    good_out = torch.zeros((B, S, H, 128) if layout == "bshd" else (B, H, S, 128), dtype=torch.bfloat16)
    with pytest.raises(TypeError, match="out: dtype"):
        zy.zyfa_fwd(q, k, v, good_out.float(), layout=layout)
    with pytest.raises(ValueError, match="lse: shape"):
        zy.zyfa_fwd(q, k, v, good_out, torch.zeros((B, S, H), dtype=torch.float32), layout=layout)


def test_fwd_refuses_bad_descales_and_non_contiguous_inputs():
    q8, k8, v8 = _qkv(torch.float8_e4m3fn)
    ds = torch.ones(1, dtype=torch.float32)
    with pytest.raises(ValueError, match="k_descale"):
        zy.zyfa_fwd(q8, k8, v8, q_descale=ds, k_descale=torch.ones(1, dtype=torch.float64), v_descale=ds)
    with pytest.raises(ValueError, match="v_descale"):
        zy.zyfa_fwd(q8, k8, v8, q_descale=ds, k_descale=ds, v_descale=torch.ones(0, dtype=torch.float32))
    q, k, v = _qkv()
    qt = torch.zeros((B, H, S, D), dtype=torch.bfloat16).transpose(1, 2)   # bshd shape, not contiguous
    with pytest.raises(ValueError, match="contiguous"):
        zy.zyfa_fwd(qt, k, v)


def test_fwd_refuses_host_tensors():
    q, k, v = _qkv()
    with pytest.raises(ValueError, match="GPU"):
        zy.zyfa_fwd(q, k, v)
    with pytest.raises(ValueError, match="GPU"):
        zy.zyfa_fwd(q, k, v, softmax_scale=0.1, p_mode="exact")


def test_noalloc_needs_out_and_checks_it():
    q, k, v = _qkv()
    with pytest.raises(ValueError, match="caller-given out"):
        zy.zyfa_fwd_noalloc(q, k, v, None)
    with pytest.raises(ValueError, match="out: shape"):
        zy.zyfa_fwd_noalloc(q, k, v, torch.zeros((B, S, H, 127), dtype=torch.bfloat16))


def test_range_checks_k_against_v():
    q, _, _ = _qkv()
    _, k, _ = _qkv(sk=100)
    _, _, v = _qkv(sk=99)
    with pytest.raises(ValueError, match="v: shape"):
        zy.zyfa_fwd_range(q, k, v, 0, 0)
    _, _, v = _qkv(sk=100)
    with pytest.raises(ValueError, match="lse: shape"):
        zy.zyfa_fwd_range(q, k, v, 0, 0, lse=torch.zeros((B, H, 100), dtype=torch.float32))
    with pytest.raises(ValueError, match="GPU"):
        zy.zyfa_fwd_range(q, k, v, 0, 0)


def test_merge_checks_shapes():
    oa = torch.zeros((B, S, H, 128), dtype=torch.bfloat16)
    la = torch.zeros((B, H, S), dtype=torch.float32)
    with pytest.raises(ValueError, match="out_a: shape"):
        zy.zyfa_lse_merge(oa, la, oa, la, layout="bhsd")
    with pytest.raises(ValueError, match="out: shape"):
        zy.zyfa_lse_merge(oa, la, oa, la, out=torch.zeros((B, S, H, 64), dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="GPU"):
        zy.zyfa_lse_merge(oa, la, oa, la)


def test_quantize_and_key_mean_check_outputs():
    x = torch.zeros((S, 128), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="x8: shape"):
        zy.zyfa_fp8_quantize(x, x8=torch.zeros((S - 1, 128), dtype=torch.uint8))
    with pytest.raises(ValueError, match="descale"):
        zy.zyfa_fp8_quantize(x, descale=torch.zeros(1, dtype=torch.float16))
    with pytest.raises(ValueError, match="GPU"):
        zy.zyfa_fp8_quantize(x)
    with pytest.raises(ValueError, match="x8: shape"):
        zy.zyfa_fp8_quantize_rotated(x, x8=torch.zeros((S, 64), dtype=torch.uint8))
    k = torch.zeros((B, S, Hk, 128), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="mean: shape"):
        zy.zyfa_key_mean(k, mean=torch.zeros((B, Hk + 1, 128), dtype=torch.float32))
    with pytest.raises(ValueError, match="GPU"):
        zy.zyfa_key_mean(k)
