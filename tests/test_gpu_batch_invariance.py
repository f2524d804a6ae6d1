"""GPU: batch invariance of the decode step.

ctol.digital commentary, CTOL House Review (batch-invariant deterministic
kernels): a sequence's output must not depend on the other sequences it is
batched with.  With HybridAttention(batch_invariant=True) every split of a
source covers a fixed range of a row's keys and the split counts depend on
the layer alone, so each sequence of a variable-length batch (planted
indexer-key ties included) must give the same output bits as the sequence
decoded alone, with the same appends; and two runs must agree bit for bit.
"""
import pytest
import torch

import lca_inputs as li
from oracle import compress as ocmp

from gpu_util import layer_for, tdtype

pytestmark = pytest.mark.gpu


def _decode(layer, cfg, d, lens, device="cuda"):
    """One decode step with appends for the sequences in d (packed raw
    streams, one query row each); returns the output."""
    caches = layer.alloc_caches(lens, device, tdtype(cfg))
    done_h = [L - 1 for L in lens]
    done = torch.tensor(done_h, dtype=torch.int64, device=device)
    # the caches as they were before the newest token (what the step appends
    # is computed by the step itself)
    layer.compress(caches, d, d["tok_off"], done_len=None)
    qmax = max(lens)
    bufs = layer.decode_buffers(len(lens), ocmp.n_entries(qmax, cfg.m, cfg.w), ocmp.n_entries(qmax, cfg.m2, cfg.w2),
                                device, tdtype(cfg))
    out = layer.decode_step(caches, d, d["tok_off"], d["q"], d["p"], d["omega"], d["sigma"], d["q_pos"], bufs,
                            done_len=done, done_h=done_h)
    torch.cuda.synchronize()
    return out.clone(), bufs["idx"].clone()


def _alone(d, b):
    """Sequence b's inputs as a batch of one (the same bits)."""
    off = d["tok_off"].cpu().tolist()
    one = {}
    for k, t in d.items():
        if k in ("tok_off", "q_pos", "sigma"):
            continue
        if k in ("q", "p", "omega"):
            one[k] = t[b:b + 1].contiguous()
        else:
            one[k] = t[off[b]:off[b + 1]].contiguous()
    one["tok_off"] = torch.tensor([0, off[b + 1] - off[b]], dtype=torch.int64, device=t.device)
    one["q_pos"] = d["q_pos"][b:b + 1].contiguous()
    one["sigma"] = d["sigma"]
    return one


@pytest.mark.parametrize("H,k,options", [(128, 1024, {}), (64, 512, {}), (128, 1024, dict(rope=64, sepv=True))])
def test_decode_step_batch_invariant(H, k, options):
    lens = (70001, 16384, 40960, 5003, 262144, 23456)
    cfg = li.small("inv", 161, lens, H=H, D=512, k=k, plant=32, **options)
    print(f"[batch invariance] H={H} k={k} {options} lens={lens}", flush=True)
    d = li.make_raw_torch(cfg, 0, "cuda")
    layer = layer_for(cfg, batch_invariant=True, max_context=1 << 20)
    out_b, idx_b = _decode(layer, cfg, d, list(lens))
    out_b2, _ = _decode(layer, cfg, d, list(lens))
    assert torch.equal(out_b, out_b2), "two runs of the batch differ"
    for b, L in enumerate(lens):
        out_1, idx_1 = _decode(layer, cfg, _alone(d, b), [L])
        assert torch.equal(idx_1[0], idx_b[b]), f"sequence {b}: selection differs alone"
        assert torch.equal(out_1[0], out_b[b]), (
            f"sequence {b} (L={L}): output bits differ alone and in the batch "
            f"(max abs {(out_1[0].float() - out_b[b].float()).abs().max().item():.3e})")
