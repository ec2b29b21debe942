"""The diagnostic memory walks (psd_diag_walk) read exactly the bytes the decode step reads:
the XOR of the per-unit words they write equals the XOR of the same words picked on the host
from the raw caches (kind 0: each kept page's K and V rows per unit; kind 1: each candidate
page's statistics record), for bf16 and fp32 caches at D = 64 and 128 and a latent cache."""
import numpy as np
import pytest
import torch

import synth
from gpu_util import make_step

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


CASES = {
    "bf16_d128": synth.small_spec(name="walk_bf16_d128", batch=5, num_q_heads=16,
                                  num_kv_heads=4, seq_lens=(3000, 17, 900, 4096, 33),
                                  budget_pages=12, max_len=4096),
    "bf16_d64": synth.small_spec(name="walk_bf16_d64", head_dim=64, head_dim_v=64),
    "f32_d64": synth.small_spec(name="walk_f32_d64", head_dim=64, head_dim_v=64, dtype="f32"),
    "f32_d128": synth.small_spec(name="walk_f32_d128", dtype="f32", seq_lens=(500, 37, 1200),
                                 max_len=1200),
    "latent576": synth.small_spec(name="walk_latent", batch=2, num_q_heads=16, num_kv_heads=1,
                                  head_dim=576, head_dim_v=512, latent=True,
                                  seq_lens=(1500, 333), max_len=1504),
}


def _xor32(a: np.ndarray) -> int:
    return int(np.bitwise_xor.reduce(np.ascontiguousarray(a).view(np.uint32).ravel(),
                                     initial=np.uint32(0)))


@pytest.mark.parametrize("name", list(CASES))
def test_walks_read_the_steps_bytes(name):
    w = synth.make_workload(CASES[name])
    sp = w.spec
    print(f"[gpu] walk {name}", flush=True)
    step, _ = make_step(w, guard=False)
    step.build_meta()
    step.select()
    sel = step.sel_pages.cpu().numpy()
    cnt = step.sel_count.cpu().numpy()
    meta = step.meta.cpu()
    meta = meta.view(torch.int16).numpy() if sp.dtype == "bf16" else meta.numpy()
    k = w.k_raw  # [NB, 16, H_kv, D]
    v = None if sp.latent else w.v_raw
    n = (w.seq_lens.astype(np.int64) + 15) // 16
    units = sp.batch * sp.num_kv_heads
    want_kv, want_stats = np.zeros(units, np.uint32), np.zeros(units, np.uint32)
    for s in range(sp.batch):
        for g in range(sp.num_kv_heads):
            u = s * sp.num_kv_heads + g
            c = max(0, min(int(cnt[s, g]), step.b_max))
            for e in range(c):
                lp = min(max(int(sel[s, g, e]), 0), int(n[s]) - 1)
                blk = int(w.block_table[s, lp])
                want_kv[u] ^= _xor32(k[blk, :, g, :])
                if v is not None:
                    want_kv[u] ^= _xor32(v[blk, :, g, :])
            for p in range(1, int(n[s]) - 1):
                want_stats[u] ^= _xor32(meta[int(w.block_table[s, p]), g])
    for kind, want in ((0, want_kv), (1, want_stats)):
        step.walk_checksum = torch.full((units,), -1, dtype=torch.int32,
                                        device=step.q.device)  # every word must be written
        step.walk(kind)
        torch.cuda.synchronize()
        got = step.walk_checksum.cpu().numpy().view(np.uint32)
        assert np.array_equal(got, want), (kind, np.nonzero(got != want)[0][:8])
    del step
    torch.cuda.empty_cache()
