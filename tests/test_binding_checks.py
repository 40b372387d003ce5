"""The Python binding refuses mis-shaped or mis-typed tensors before any
pointer reaches the library (which sees only pointers and sizes and could
not tell). Runs on the CPU: the checks precede the GPU-tensor check."""
import pytest
import torch

import context_partial_attention_amd as cpa


def _pass_kv_args(tq=10, tk=12, hq=4, hkv=2, d=64, dtype=torch.bfloat16):
    q = torch.zeros((tq, hq, d), dtype=dtype)
    k = torch.zeros((tk, hkv, d), dtype=dtype)
    v = torch.zeros((tk, hkv, d), dtype=dtype)
    q_pos = torch.arange(tq, dtype=torch.int32)
    k_pos = torch.arange(tk, dtype=torch.int32)
    cu_q = torch.tensor([0, tq], dtype=torch.int32)
    cu_k = torch.tensor([0, tk], dtype=torch.int32)
    return q, q_pos, cu_q, k, v, k_pos, cu_k


def _raises(match, fn, *a, **kw):
    with pytest.raises(ValueError, match=match):
        fn(*a, **kw)


def test_partial_attn_checks_before_the_device():
    q, q_pos, cu_q, k, v, k_pos, cu_k = _pass_kv_args()
    # well-formed CPU tensors get as far as the GPU check
    _raises("must be a GPU tensor", cpa.partial_attn, q, q_pos, cu_q, k, v, k_pos, cu_k, 10, 0.125)
    _raises("q_pos has dtype int64", cpa.partial_attn, q, q_pos.long(), cu_q, k, v, k_pos, cu_k, 10, 0.125)
    _raises("cu_q has dtype int64", cpa.partial_attn, q, q_pos, cu_q.long(), k, v, k_pos, cu_k, 10, 0.125)
    _raises("k_pos has dtype", cpa.partial_attn, q, q_pos, cu_q, k, v, k_pos.float(), cu_k, 10, 0.125)
    _raises("cu_k has shape", cpa.partial_attn, q, q_pos, cu_q, k, v, k_pos, cu_k[:1], 10, 0.125)
    _raises("k has dtype float32", cpa.partial_attn, q, q_pos, cu_q, k.float(), v, k_pos, cu_k, 10, 0.125)
    _raises("v has shape", cpa.partial_attn, q, q_pos, cu_q, k, v[:5], k_pos, cu_k, 10, 0.125)
    _raises(r"k must be \[tokens, hkv, 64\]", cpa.partial_attn, q, q_pos, cu_q, k[..., :32], v, k_pos, cu_k, 10,
            0.125)
    _raises("must be a multiple of hkv", cpa.partial_attn, q[:, :3], q_pos, cu_q, k, v, k_pos, cu_k, 10, 0.125)
    _raises("q_pos has shape", cpa.partial_attn, q, q_pos[:4], cu_q, k, v, k_pos, cu_k, 10, 0.125)
    _raises("out has shape", cpa.partial_attn, q, q_pos, cu_q, k, v, k_pos, cu_k, 10, 0.125,
            out=torch.zeros((10, 4, 32)))
    _raises("lse has dtype", cpa.partial_attn, q, q_pos, cu_q, k, v, k_pos, cu_k, 10, 0.125,
            lse=torch.zeros((10, 4), dtype=torch.float64))
    _raises("q has dtype", cpa.partial_attn, q.half(), q_pos, cu_q, k.half(), v.half(), k_pos, cu_k, 10, 0.125)


def test_multi_and_merged_check_every_shard():
    q, q_pos, cu_q, k, v, k_pos, cu_k = _pass_kv_args()
    ks, vs, kps, cus = [k, k], [v, v], [k_pos, k_pos], [cu_k, cu_k]
    _raises("must be a GPU tensor", cpa.partial_attn_multi, q, q_pos, cu_q, ks, vs, kps, cus, 10, 0.125)
    _raises(r"vs\[1\] has dtype", cpa.partial_attn_multi, q, q_pos, cu_q, ks, [v, v.float()], kps, cus, 10, 0.125)
    _raises(r"k_poss\[0\] has dtype", cpa.partial_attn_multi, q, q_pos, cu_q, ks, vs, [k_pos.long(), k_pos], cus,
            10, 0.125)
    _raises("one entry per shard", cpa.partial_attn_multi, q, q_pos, cu_q, ks, vs, kps[:1], cus, 10, 0.125)
    _raises(r"outs\[1\] has shape", cpa.partial_attn_multi, q, q_pos, cu_q, ks, vs, kps, cus, 10, 0.125,
            outs=[torch.zeros((10, 4, 64)), torch.zeros((9, 4, 64))])
    _raises("workspace must be a 1-D uint8", cpa.partial_attn_multi, q, q_pos, cu_q, ks, vs, kps, cus, 10, 0.125,
            workspace=torch.zeros(16, dtype=torch.int32))
    _raises(r"cu_ks\[1\] has shape", cpa.partial_attn_merged, q, q_pos, cu_q, ks, vs, kps, [cu_k, cu_k[:1]], 10,
            0.125)
    _raises("must be a GPU tensor", cpa.partial_attn_merged, q, q_pos, cu_q, ks, vs, kps, cus, 10, 0.125)


def test_accumulate_checks_the_running_state():
    q, q_pos, cu_q, k, v, k_pos, cu_k = _pass_kv_args()
    o_acc, lse_acc = torch.zeros((10, 4, 64)), torch.zeros((10, 4))
    _raises("must be a GPU tensor", cpa.partial_attn_accumulate, q, q_pos, cu_q, k, v, k_pos, cu_k, 10, 0.125,
            o_acc, lse_acc)
    _raises("o_acc has dtype", cpa.partial_attn_accumulate, q, q_pos, cu_q, k, v, k_pos, cu_k, 10, 0.125,
            o_acc.bfloat16(), lse_acc)
    _raises("lse_acc has shape", cpa.partial_attn_accumulate, q, q_pos, cu_q, k, v, k_pos, cu_k, 10, 0.125,
            o_acc, lse_acc[:3])


def test_paged_checks_cache_table_and_lengths():
    tq, hq, hkv, d = 6, 4, 2, 64
    q = torch.zeros((tq, hq, d), dtype=torch.bfloat16)
    q_pos = torch.arange(tq, dtype=torch.int32)
    cu_q = torch.tensor([0, 3, 6], dtype=torch.int32)
    kc = torch.zeros((8, hkv, 16, d), dtype=torch.bfloat16)
    table = torch.zeros((2, 4), dtype=torch.int32)
    lens = torch.tensor([30, 40], dtype=torch.int32)
    args = (q, q_pos, cu_q, kc, kc.clone(), table, lens, 2, 0, 8, 3, 0.125)
    _raises("must be a GPU tensor", cpa.partial_attn_paged, *args)
    _raises("block_table has dtype", cpa.partial_attn_paged, q, q_pos, cu_q, kc, kc, table.long(), lens, 2, 0, 8,
            3, 0.125)
    _raises("block_table must be", cpa.partial_attn_paged, q, q_pos, cu_q, kc, kc, table[:1], lens, 2, 0, 8, 3,
            0.125)
    _raises("local_kv_lens has dtype", cpa.partial_attn_paged, q, q_pos, cu_q, kc, kc, table, lens.long(), 2, 0, 8,
            3, 0.125)
    _raises("v_cache has shape", cpa.partial_attn_paged, q, q_pos, cu_q, kc, kc[:4], table, lens, 2, 0, 8, 3, 0.125)
    _raises(r"k_cache must be \[blocks, hkv, block_size, 64\]", cpa.partial_attn_paged, q, q_pos, cu_q, kc[0], kc,
            table, lens, 2, 0, 8, 3, 0.125)


def test_paged_merged_checks_the_received_parts():
    tq, hq, hkv, d = 2, 4, 2, 64
    q = torch.zeros((tq, hq, d), dtype=torch.bfloat16)
    q_pos = torch.tensor([29, 39], dtype=torch.int32)
    cu_q = torch.tensor([0, 1, 2], dtype=torch.int32)
    kc = torch.zeros((8, hkv, 16, d), dtype=torch.bfloat16)
    table = torch.zeros((2, 4), dtype=torch.int32)
    lens = torch.tensor([15, 20], dtype=torch.int32)
    o1, l1 = torch.zeros((tq, hq, d)), torch.zeros((tq, hq))
    head = (q, q_pos, cu_q, kc, kc.clone(), table, lens, 2, 0, 8)
    f = cpa.partial_attn_paged_merged
    _raises("must be a GPU tensor", f, *head, 1, 0.125, [o1], [l1])
    _raises("same number", f, *head, 1, 0.125, [o1, o1], [l1])
    _raises(r"o_parts\[1\] has dtype", f, *head, 1, 0.125, [o1, o1.bfloat16()], [l1, l1])
    _raises(r"lse_parts\[0\] has shape", f, *head, 1, 0.125, [o1], [l1[:1]])
    _raises("own_out has dtype", f, *head, 1, 0.125, [o1], [l1], own_out=o1.bfloat16())
    _raises("block_table has dtype", f, q, q_pos, cu_q, kc, kc, table.long(), lens, 2, 0, 8, 1, 0.125, [o1], [l1])


def test_lse_merge_checks_parts_and_outputs():
    o = torch.zeros((5, 4, 64))
    l = torch.zeros((5, 4))
    _raises("must be a GPU tensor", cpa.lse_merge, [o, o], [l, l])
    _raises("same shape and dtype", cpa.lse_merge, [o, o[:4]], [l, l])
    _raises("same shape and dtype", cpa.lse_merge, [o, o], [l, l.double()])
    _raises("out has shape", cpa.lse_merge, [o, o], [l, l], out=torch.zeros((5, 4, 32)))
    _raises("lse_out must hold", cpa.lse_merge, [o, o], [l, l], lse_out=torch.zeros(7))
