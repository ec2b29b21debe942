"""Value tier with a resident hot buffer (psd_value_tier_stage + psd_sparse_decode_tiered),
V in pinned host memory, and the KV tier (psd_kv_tier_stage + psd_sparse_decode_kv_tiered),
K and V in pinned host memory, over consecutive decode steps whose queries drift: outputs
are the same bits as the attention reading K and V straight from where they live, and the
oracle's; every resident slot holds its slice's rows (K and V for the KV tier); the counts
add up; with no slots every entry reads from host, with few slots the overflow reads from
host."""
import dataclasses

import numpy as np
import pytest
import torch

import synth
from gpu_util import check_workload, make_step, meta_f64

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


CASES = {
    # 256 units: whole-unit attention
    "whole_unit": synth.small_spec(name="tier_whole_unit", batch=32, num_q_heads=32,
                                   num_kv_heads=8, seq_lens=(), len_range=(1500, 9000),
                                   budget_percent=6, max_len=9000),
    # few units: split-K attention and its merge
    "split_k": synth.small_spec(name="tier_split_k", batch=3, num_q_heads=16, num_kv_heads=2,
                                seq_lens=(4000, 700, 6100), budget_pages=30, max_len=6200),
    "f32_d64": synth.small_spec(name="tier_f32_d64", batch=6, num_q_heads=8, num_kv_heads=2,
                                head_dim=64, head_dim_v=64, dtype="f32",
                                seq_lens=(3000, 1200, 5000, 64, 17, 2500), budget_pages=24,
                                max_len=5000),
}


def _drifted_q(w: synth.Workload, t: int) -> np.ndarray:
    """Step t's queries: step 0's plus a small seeded drift, in the workload's dtype."""
    q = synth.to_f64(w.q, w.spec.dtype).astype(np.float32)
    if t:
        q = q + np.float32(0.12 * t) * np.random.default_rng(1000 + t).standard_normal(
            q.shape).astype(np.float32)
    return synth.f32_to_bf16_bits(q) if w.spec.dtype == "bf16" else q


def _q_tensor(raw: np.ndarray, dtype: str, dev) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(raw))
    return t.view(torch.int16).to(dev).view(torch.bfloat16) if dtype == "bf16" else t.to(dev)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("tier", ["v", "kv"])
@pytest.mark.parametrize("mode", ["ample", "tight", "none"])
@pytest.mark.parametrize("name", list(CASES))
def test_value_tier_over_steps(name, mode, tier):
    w = synth.make_workload(CASES[name])
    kv = tier == "kv"
    print(f"[gpu] {tier} tier {name} {mode}", flush=True)
    step, bands = make_step(w, v_host=True, guard=False, kv_host=kv)
    step.build_meta()
    step.select()
    kept = int(step.sel_count.clamp(min=0).sum())
    slots = {"ample": 2 * kept, "tight": max(1, kept // 3), "none": 0}[mode]
    step.enable_tier(slots, kv=kv)
    v_host = step.v  # pinned host V pool [NB, 16, H_kv, D_v]
    k_host = step.k  # the K pool: pinned host memory for the KV tier
    Hkv = w.spec.num_kv_heads
    for t in range(3):
        q_raw = _drifted_q(w, t)
        step.q.copy_(_q_tensor(q_raw, w.spec.dtype, step.q.device))
        step.select()
        step.tier_stage()
        step.sparse_tiered()
        torch.cuda.synchronize()
        out_tier = step.out.clone()
        step.out.fill_(123.0)
        step.sparse()  # V (and K for the KV tier) straight from host memory
        torch.cuda.synchronize()
        assert torch.equal(out_tier.view(torch.int32), step.out.view(torch.int32)), f"step {t}"
        cnt = step.sel_count.cpu().numpy().clip(min=0)
        kept = int(cnt.sum())
        c = step.tier_counts()
        vslot = step.tier_vslot.cpu().numpy()
        sel = step.sel_pages.cpu().numpy()
        entries = [(s, g, e) for s in range(w.spec.batch) for g in range(Hkv)
                   for e in range(int(cnt[s, g]))]
        assert c["hits"] + c["misses"] == kept, (c, kept)
        assert c["copied"] <= c["misses"]
        from_host = sum(1 for s, g, e in entries if vslot[s, g, e] < 0)
        assert c["from_host"] == from_host, (c, from_host)
        if mode == "none":
            assert c["hits"] == 0 and c["copied"] == 0 and from_host == kept
        if mode == "ample":
            assert from_host == 0
            if t:
                assert c["hits"] > 0, c  # the drifted step keeps some of the last step's pages
        if mode == "tight" and t == 0:
            assert from_host > 0
        # every slot an entry reads holds that entry's slice (its block's rows of head g)
        if slots:
            hot = step.tier_hot.cpu()
            hot_k = step.tier_hot_k.cpu() if kv else None
            used = {}
            for s, g, e in entries:
                slot = int(vslot[s, g, e])
                if slot < 0:
                    continue
                blk = int(w.block_table[s, sel[s, g, e]])
                assert used.setdefault(slot, (blk, g)) == (blk, g), "one slot, two slices"
                bits = torch.int16 if w.spec.dtype == "bf16" else torch.int32  # NaN rows too
                assert torch.equal(hot[slot].view(bits), v_host[blk, :, g, :].view(bits)), \
                    (s, g, e, slot)
                if kv:
                    assert torch.equal(hot_k[slot].view(bits), k_host[blk, :, g, :].view(bits)), \
                        ("K", s, g, e, slot)
        if t in (0, 2):  # the oracle on the drifted queries
            wt = dataclasses.replace(w, q=q_raw)
            seqs = range(w.spec.batch) if w.spec.batch <= 8 else range(0, w.spec.batch, 5)
            check_workload(wt, dict(meta=meta_f64(step, w.spec.dtype),
                                    sel=step.sel_pages.cpu().numpy(), cnt=step.sel_count.cpu().numpy(),
                                    out=out_tier.cpu().numpy().astype(np.float64),
                                    b_max=step.b_max), seqs=seqs, dense_seqs=[])
    del step
    torch.cuda.empty_cache()
