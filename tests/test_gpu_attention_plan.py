"""GPU checks of attention plan reuse: hp_attention_plan runs the planning
kernels alone, and attention calls with HP_FLAG_PLANNED on the same
descriptor, query-head count and streaming setting skip theirs. One plan
serves several calls with other queries and pools (the layers of one batch);
each result must equal, bit for bit, the same call planning for itself."""
import dataclasses

import numpy as np
import pytest
import torch

import workloads
from gpu_util import OnDevice, host_bits, say
from test_gpu_attention import shared_prefix_workload

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module")
def hp():
    import block_table_gather_amd
    return block_table_gather_amd


def layer_inputs(w, group, layer):
    v = dataclasses.replace(w, seed=w.seed * 7 + 3 + 101 * layer)
    k = dataclasses.replace(w, seed=w.seed * 5 + 1 + 101 * layer)
    g = torch.Generator(device=DEV).manual_seed(7000 + layer)
    q = torch.randn((w.num_seqs, w.num_heads * group, w.head_dim), generator=g, device=DEV)
    return k.make_pool(DEV), v.make_pool(DEV), q.to(torch.bfloat16 if w.dtype != "f16"
                                                     else torch.float16)


def check_layers(hp, w, group, streaming, layers=3, checked=False):
    d = OnDevice(w)
    ws = hp.attention_plan(d.desc, w.num_heads * group, total_tokens=w.total_tokens,
                           streaming=streaming)
    for layer in range(layers):
        kp, vp, q = layer_inputs(w, group, layer)
        desc = hp.Descriptor(kp, d.bt, d.sp, d.sl)
        out = torch.full((w.num_seqs, q.shape[1], w.head_dim), float("nan"), device=DEV)
        ref = torch.full_like(out, float("nan"))
        hp.paged_attention(desc, vp, q, out, total_tokens=w.total_tokens, scale=0.1,
                           streaming=streaming, workspace=ws, planned=True, checked=checked)
        hp.paged_attention(desc, vp, q, ref, total_tokens=w.total_tokens, scale=0.1,
                           streaming=streaming)
        torch.cuda.synchronize()
        assert np.array_equal(host_bits(out), host_bits(ref)), f"layer {layer}"


def test_plan_reuse_shared_prefix(hp):
    """Cached loads over runs of sequences sharing pages: the comparison and
    the shared-prefix plan run once."""
    w = shared_prefix_workload(7100, 16, 4, 128, "bf16", np.uint32,
                               [(12, 512, (16, 200)), (1, 0, (5, 300)), (6, 256, (0, 40))])
    say("plan reuse, shared prefixes", w.describe())
    check_layers(hp, w, 4, streaming=False)


def test_plan_reuse_checked(hp):
    """HP_FLAG_CHECKED with a reused plan: the validator's words sit before
    the plan in the workspace and do not disturb it."""
    w = shared_prefix_workload(7110, 16, 2, 64, "f16", np.uint32, [(9, 300, (1, 60))])
    say("plan reuse, checked", w.describe())
    check_layers(hp, w, 8, streaming=False, checked=True)


def test_plan_reuse_many_sequences(hp):
    """More than 4,096 sequences: the unit plan runs once."""
    rng = np.random.default_rng(7120)
    S, P = 4600, 4
    lens = rng.integers(0, 24, size=S).astype(np.uint32)
    counts = (lens + P - 1) // P
    K = int(counts.sum())
    bt = rng.permutation(K + 7)[:K].astype(np.uint32)
    sp = np.concatenate([[0], np.cumsum(counts)]).astype(np.uint32)
    w = workloads.Workload("plan", "bf16", P, 2, 64, K + 7, np.uint32, bt, sp, lens, seed=7120)
    say("plan reuse, many sequences", w.describe())
    check_layers(hp, w, 2, streaming=False, layers=2)


@pytest.mark.parametrize("group", [1, 4])
def test_plan_reuse_no_plan_needed(hp, group):
    """A decode-style batch with streaming loads: no planning kernel exists;
    the planned calls behave as the others."""
    w = workloads.random_small(7130 + group, max_seqs=12, max_len=300, page_sizes=(16,),
                               heads=(4,), dims=(128,), dtypes=("f16",), alias=False)
    say("plan reuse, none needed", group, w.describe())
    check_layers(hp, w, group, streaming=True, layers=2)


def test_plan_reuse_int8(hp):
    """hp_paged_attention_q8 on a shared-prefix batch reuses its plan."""
    w = shared_prefix_workload(7140, 16, 4, 128, "i8", np.uint32,
                               [(10, 512, (1, 100)), (3, 64, (0, 20))])
    w = dataclasses.replace(w, values="int8", with_scales=True)
    say("plan reuse, int8", w.describe())
    d = OnDevice(w)
    ws = hp.attention_plan(d.desc, 16, total_tokens=w.total_tokens)
    for layer in range(2):
        vw = dataclasses.replace(w, seed=w.seed + 11 * (layer + 1))
        vp, vs = vw.make_pool(DEV), vw.make_scales(DEV)
        g = torch.Generator(device=DEV).manual_seed(7150 + layer)
        q = torch.randn((w.num_seqs, 16, 128), generator=g, device=DEV).to(torch.bfloat16)
        out = torch.full((w.num_seqs, 16, 128), float("nan"), device=DEV)
        ref = torch.full_like(out, float("nan"))
        hp.paged_attention_q8(d.desc, vp, vs, q, out, total_tokens=w.total_tokens,
                              workspace=ws, planned=True)
        hp.paged_attention_q8(d.desc, vp, vs, q, ref, total_tokens=w.total_tokens)
        torch.cuda.synchronize()
        assert np.array_equal(host_bits(out), host_bits(ref)), f"layer {layer}"
