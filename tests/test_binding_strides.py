"""CPU: the (sequence, position, head) stride triples the Python binding hands
to the C ABI.

The ABI reads an all-zero triple as the dense layout, so a triple built from a
view must never come out all zero unless the view is dense; size-1 dimensions
(whose stride never moves an address) are given their dense stride, and
expanded views (stride 0 on a dimension of size > 1) are refused before any
call reaches the library.
"""
import pytest
import torch

import causal_attention_fwd_amd as attn


def test_dense_tensor_gives_dense_triple():
    t = torch.empty(3, 17, 4, 64, dtype=torch.bfloat16)
    assert attn._strides("q", [("q", t)]) == (17 * 4 * 64, 4 * 64, 64)


def test_size_one_dims_take_the_dense_stride_not_zero():
    # one sequence, one position, one head: every leading dim has size 1
    t = torch.empty(1, 1, 1, 64, dtype=torch.bfloat16)
    assert attn._strides("q", [("q", t)]) == (64, 64, 64)
    # a shared decode cache with Smax = Hkv = 1
    k = torch.empty(5, 1, 1, 128, dtype=torch.bfloat16)
    st = attn._strides("cache", [("k", k), ("v", k.clone())])
    assert st == (128, 128, 128) and st != (0, 0, 0)


def test_strided_view_of_a_fused_projection():
    qkv = torch.empty(2, 33, 3, 8, 64, dtype=torch.bfloat16)
    q = qkv[:, :, 0]
    assert attn._strides("q", [("q", q)]) == (33 * 3 * 8 * 64, 3 * 8 * 64, 64)
    # one sequence of such a view: the batch stride is the dense one
    q1 = qkv[:1, :, 1]
    assert attn._strides("q", [("q", q1)]) == (33 * 8 * 64, 3 * 8 * 64, 64)


def test_group_members_must_share_strides():
    a = torch.empty(2, 16, 4, 64, dtype=torch.bfloat16)
    b = torch.empty(2, 16, 8, 64, dtype=torch.bfloat16)[:, :, :4]
    with pytest.raises(ValueError):
        attn._strides("k/v", [("k", a), ("v", b)])


@pytest.mark.parametrize("shape,expand", [((1, 1, 1, 64), (4, 1, 1, 64)), ((1, 7, 2, 64), (3, 7, 2, 64)),
                                          ((2, 1, 2, 64), (2, 9, 2, 64)), ((2, 5, 1, 64), (2, 5, 6, 64))])
def test_expanded_views_are_refused(shape, expand):
    t = torch.empty(*shape, dtype=torch.bfloat16).expand(*expand)
    with pytest.raises(ValueError, match="expanded"):
        attn._reject_expanded("q", t)


def test_views_with_real_strides_pass():
    attn._reject_expanded("q", torch.empty(4, 1, 1, 64, dtype=torch.bfloat16))
    attn._reject_expanded("q", torch.empty(2, 9, 3, 8, 64, dtype=torch.bfloat16)[:, :, 1])
