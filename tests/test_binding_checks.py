"""The Python binding rejects tensors the C ABI cannot check for itself.

The library receives untyped device pointers, so a weight in another dtype
than x, an output of the wrong shape, a gate matrix with too few columns or a
host tensor would make its kernels read or write outside the buffers.  The
binding raises TypeError / ValueError for each of these before anything is
launched; these tests need no GPU because every check runs before the first
device call.
"""
import pytest
import torch

gg = pytest.importorskip("grouped_gemm_permute_amd")

T, D, F, E, K = 8, 64, 128, 4, 2


def layer(dtype=torch.bfloat16, device="cpu"):
    z = dict(dtype=dtype, device=device)
    return dict(
        x=torch.zeros((T, D), **z), W1=torch.zeros((E, D, F), **z), W3=torch.zeros((E, D, F), **z),
        W2=torch.zeros((E, F, D), **z),
        idx=torch.zeros((T, K), dtype=torch.int32, device=device),
        w=torch.zeros((T, K), dtype=torch.float32, device=device),
        shared=(torch.zeros((D, F), **z), torch.zeros((D, F), **z), torch.zeros((F, D), **z)))


def fwd(a, **kw):
    args = dict(a)
    args.update(kw)
    return gg.forward(args["x"], args["idx"], args["w"], args["W1"], args["W3"], args["W2"],
                      args["shared"], y=args.get("y"))


@pytest.mark.parametrize("name", ["W1", "W3", "W2"])
def test_weight_dtype_must_match_x(name):
    a = layer()
    a[name] = a[name].float()
    with pytest.raises(TypeError, match=name):
        fwd(a)


def test_fp32_x_with_bf16_weights_is_refused():
    a = layer()
    a["x"] = a["x"].float()
    with pytest.raises(TypeError):
        fwd(a)


def test_output_shape_and_dtype():
    a = layer()
    with pytest.raises(ValueError, match="y"):
        fwd(a, y=torch.zeros((T, D + 8), dtype=torch.bfloat16))
    with pytest.raises(TypeError, match="y"):
        fwd(a, y=torch.zeros((T, D), dtype=torch.float32))


def test_shared_weight_shapes_and_dtypes():
    a = layer()
    Ws1, Ws3, Ws2 = a["shared"]
    with pytest.raises(ValueError, match="Ws2"):
        fwd(a, shared=(Ws1, Ws3, torch.zeros((D, F), dtype=torch.bfloat16)))
    with pytest.raises(TypeError, match="Ws1"):
        fwd(a, shared=(Ws1.float(), Ws3, Ws2))


def test_routing_dtypes_and_shapes():
    a = layer()
    with pytest.raises(TypeError, match="topk_idx"):
        fwd(a, idx=a["idx"].long())
    with pytest.raises(TypeError, match="topk_w"):
        fwd(a, w=a["w"].double())
    with pytest.raises(ValueError, match="topk_w"):
        fwd(a, w=torch.zeros((T, K + 1), dtype=torch.float32))


def test_non_contiguous_weight():
    a = layer()
    a["W2"] = torch.zeros((E, D, F), dtype=torch.bfloat16).transpose(1, 2)
    with pytest.raises(ValueError, match="contiguous"):
        fwd(a)


def test_host_tensors_are_refused():
    """Well-formed tensors that live in host memory: their addresses are not
    device pointers."""
    with pytest.raises(ValueError, match="GPU"):
        fwd(layer())


def test_router_gate_shape():
    x = torch.zeros((T, D), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="gate_w"):
        gg.router_topk(x, torch.zeros((D + 1, E), dtype=torch.bfloat16), K)
    with pytest.raises(TypeError, match="gate_w"):
        gg.router_topk(x, torch.zeros((D, E), dtype=torch.float32), K)
    with pytest.raises(ValueError, match="GPU"):
        gg.router_topk(x, torch.zeros((D, E), dtype=torch.bfloat16), K)


def test_forward_routed_gate_columns_match_experts():
    a = layer()
    with pytest.raises(ValueError, match="gate_w"):
        gg.forward_routed(a["x"], torch.zeros((D, E - 1), dtype=torch.bfloat16), a["W1"], a["W3"],
                          a["W2"], a["shared"], k=K)
    with pytest.raises(ValueError, match="k must be"):
        gg.forward_routed(a["x"], torch.zeros((D, E), dtype=torch.bfloat16), a["W1"], a["W3"],
                          a["W2"], a["shared"], k=E + 1)


def test_backward_gradient_buffers():
    a = layer()
    dy = torch.zeros((T, D), dtype=torch.bfloat16)
    with pytest.raises(TypeError, match="dy"):
        gg.backward(a["x"], a["idx"], a["w"], a["W1"], a["W3"], a["W2"], a["shared"], dy.float())
    with pytest.raises(TypeError, match="dW2"):
        gg.backward(a["x"], a["idx"], a["w"], a["W1"], a["W3"], a["W2"], a["shared"], dy,
                    out={"dW2": torch.zeros((E, F, D), dtype=torch.bfloat16)})
    with pytest.raises(ValueError, match="dW1"):
        gg.backward(a["x"], a["idx"], a["w"], a["W1"], a["W3"], a["W2"], a["shared"], dy,
                    out={"dW1": torch.zeros((E, F, D), dtype=torch.float32)})


def test_permute_index_dtype():
    with pytest.raises(TypeError, match="topk_idx"):
        gg.expert_permute(torch.zeros((T, K), dtype=torch.int64), E)


def test_kept_gate_up_shape_and_dtype():
    """forward_save_gu's gu and backward's gu are [T*k + T (shared), 2F] in
    x's dtype: a smaller array would let the kernels write or read past it."""
    a = layer()
    R = T * K + T
    args = (a["x"], a["idx"], a["w"], a["W1"], a["W3"], a["W2"], a["shared"])
    with pytest.raises(ValueError, match="gu"):
        gg.forward_save_gu(*args, gu=torch.zeros((R - 1, 2 * F), dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="gu"):
        gg.forward_save_gu(*args, gu=torch.zeros((R, F), dtype=torch.bfloat16))
    with pytest.raises(TypeError, match="gu"):
        gg.forward_save_gu(*args, gu=torch.zeros((R, 2 * F), dtype=torch.float32))
    dy = torch.zeros((T, D), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="gu"):
        gg.backward(*args, dy, gu=torch.zeros((T * K, 2 * F), dtype=torch.bfloat16))
