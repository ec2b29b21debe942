"""psd_decode_step_noalloc (the decode step on the library's static scratch, for callers
that cannot allocate) against psd_decode_step with a caller workspace: statistics, rows,
counts and outputs bit for bit, over consecutive calls in one process where each call
runs over the scratch contents the previous one left, the second with a smaller input."""
import numpy as np
import pytest
import torch

import synth
from gpu_util import check_guards, make_step

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _same(a, b):
    return torch.equal(a.view(torch.int32), b.view(torch.int32))


# Chunked selection and split-K attention (candidates and partials in the scratch), then a
# smaller batch, then a batch whose one-launch step needs almost no scratch, then the first
# again.
CASES = [
    synth.small_spec("noalloc_chunked", batch=8, num_q_heads=32, num_kv_heads=8, seq_lens=(),
                     len_range=(16 * 2500, 16 * 3000), budget_pages=50, max_len=16 * 3000),
    synth.small_spec("noalloc_small", batch=2, seq_lens=(16 * 700 - 3, 4000), budget_pages=40,
                     max_len=16 * 700),
    synth.small_spec("noalloc_fused", batch=64, num_q_heads=32, num_kv_heads=8, seq_lens=(),
                     len_range=(3000, 9000), budget_percent=5, max_len=9008),
    synth.small_spec("noalloc_certified", batch=2, num_q_heads=64, num_kv_heads=2,
                     seq_lens=(9000, 3000), budget_percent=5, max_len=9008),
    synth.small_spec("noalloc_latent", batch=4, num_q_heads=128, num_kv_heads=1, head_dim=576,
                     head_dim_v=512, latent=True, seq_lens=(16 * 700 - 5, 1500, 333, 16 * 300),
                     budget_percent=5, max_len=16 * 700),
]


def _one(spec):
    w = synth.make_workload(spec)
    print(f"[gpu] noalloc {spec.name}: B={w.spec.batch} G={w.spec.group}", flush=True)
    ref_step, bands_r = make_step(w)
    ref_step.build_meta()
    stale = ref_step.meta.clone()
    ref_step.step()
    check_guards(bands_r, f"{spec.name} decode_step")
    ref = [t.clone() for t in (ref_step.meta, ref_step.sel_pages, ref_step.sel_count, ref_step.out)]
    step, bands = make_step(w)
    step.meta.copy_(stale)
    step.sel_pages.fill_(-7)
    step.sel_count.fill_(-7)
    step.out.fill_(123.0)
    step.step_noalloc()
    check_guards(bands, f"{spec.name} decode_step_noalloc")
    got = (step.meta, step.sel_pages, step.sel_count, step.out)
    for what, a, b in zip(("statistics", "rows", "counts", "outputs"), got, ref):
        assert _same(a, b), f"{spec.name}: {what} differ"
    print(f"[ok] noalloc {spec.name}: bit-identical to psd_decode_step", flush=True)
    del step, ref_step, bands, bands_r
    torch.cuda.empty_cache()


def test_noalloc_matches_decode_step_over_consecutive_calls():
    for spec in CASES + CASES[:1]:
        _one(spec)


def test_noalloc_rejects_a_step_beyond_the_scratch():
    from page_selected_sparse_amd import api

    spec = synth.small_spec("noalloc_too_big", batch=2, num_q_heads=128, num_kv_heads=1,
                            head_dim=576, head_dim_v=512, latent=True, seq_lens=(16, 16),
                            budget_pages=4, max_len=16)
    w = synth.make_workload(spec)
    step, _ = make_step(w, guard=False)
    big = api.make_shape(step.q, step.k, step.v, step.block_table, 512)
    big.batch, big.max_pages_per_seq = 128, 4096  # host-side check only: nothing launches
    with pytest.raises(api.PsdError) as e:
        api.decode_step_noalloc(big, step.q, step.meta, step.k, step.v, step.block_table,
                                step.seq_lens, step.budgets, 2048, step.scale, step.sel_pages,
                                step.sel_count, step.out)
    assert e.value.status == -6
