"""The seeded input generator: shapes, determinism and the heavy-key recipe."""
import torch

from workloads import WORKLOADS, generate, heavy_positions, sample_units


def test_shapes_and_determinism():
    w = WORKLOADS[1]
    a = generate(w, seed=0)
    b = generate(w, seed=0)
    c = generate(w, seed=1)
    assert a["q_prompt"].shape == (1, 4, 64, 64) and a["q_prompt"].dtype == torch.float32
    assert a["q_dec"].shape == (64, 1, 4, 64)
    for k in a:
        assert torch.equal(a[k], b[k])
        assert a[k].is_contiguous()
    assert not torch.equal(a["q_prompt"], c["q_prompt"])


def test_heavy_keys_follow_the_mean_query_direction():
    w = WORKLOADS[4].scaled(batch=2, heads=3, prompt=40, steps=20)
    x = generate(w, seed=0)
    sel = heavy_positions(w, seed=0)
    assert int(sel[0, 4:].sum()) <= round(0.05 * 60) <= int(sel[0].sum())
    assert bool(sel[:, :4].all())                               # sinks
    q = torch.cat([x["q_prompt"].permute(2, 0, 1, 3), x["q_dec"]]).double()   # [N,B,H,d]
    k = torch.cat([x["k_prompt"].permute(2, 0, 1, 3), x["k_dec"]]).double()
    u = q.sum(0)
    u = u / u.norm(dim=-1, keepdim=True)
    cos = (k * u).sum(-1) / k.norm(dim=-1)                      # [N,B,H]
    heavy = sel.t()[:, :, None].expand_as(cos)
    assert float(cos[heavy].min()) > 0.999                      # along u (fp16 rounding)
    assert float(cos[~heavy].abs().max()) < 0.6                 # random keys are not
    assert float(k.norm(dim=-1)[heavy].mean()) > 3 * float(k.norm(dim=-1)[~heavy].mean())


def test_sample_units_keeps_ends():
    s = sample_units(896, 16, seed=0)
    assert s[0] == 0 and s[-1] == 895 and len(s) == 16 and s == sorted(set(s))
    assert sample_units(4, 16) == [0, 1, 2, 3]
