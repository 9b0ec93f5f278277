"""Artifact prefetch (segmla_prefetch): while layer l runs, the next layer's cached rows are
staged into device buffers on the library's own stream; the next layer's forward, ordered
after the transfers by a device event, must see exactly the staged rows (RedKnot-MLA paper,
TP8 fast-path paragraph)."""
import numpy as np
import pytest
import torch

from segmented_attention_amd import segmla as S
from segmented_attention_amd.segmla import Plan
from tests.gpu_common import run_gpu, say
from workload import SMALL_CONFIGS, make_inputs

pytestmark = pytest.mark.gpu


def _bits(x):
    return x.view(torch.int16) if x.dtype == torch.bfloat16 else x.view(torch.int32)


def _same(a, b):
    return a.shape == b.shape and torch.equal(_bits(a), _bits(b))


ARTIFACTS = {"bf16": ("kv", "z_cached"), "e4m3": ("kv", "kv_scale", "kv_rope", "z_cached")}


@pytest.mark.parametrize("cfg", [SMALL_CONFIGS[1], SMALL_CONFIGS[4]], ids=lambda c: c["name"])
def test_prefetch_next_layer_from_pinned_host(cfg):
    """Layer B's artifacts come from pinned host memory; their transfers are issued before
    layer A's forward and overlap it; B's forward after prefetch_wait equals B's forward on the
    original device tensors bit for bit, and A is unaffected."""
    say("case prefetch %s" % cfg["name"])
    inp_a = make_inputs(cfg, "cuda")
    inp_b = make_inputs(dict(cfg, seed=cfg["seed"] + 100), "cuda")
    _, oa_ref, za_ref, _ = run_gpu(inp_a)
    _, ob_ref, zb_ref, _ = run_gpu(inp_b)
    names = ARTIFACTS[cfg["kv_dtype"]]
    host = {k: inp_b[k].cpu().pin_memory() for k in names}
    staged = {k: torch.full_like(inp_b[k], 0x7F if inp_b[k].dtype == torch.uint8 else float("nan"))
              for k in names}
    plan_a = Plan.for_inputs(inp_a)
    plan_a.build(inp_a["scores"])
    plan_b = Plan.for_inputs(inp_b)
    plan_b.build(inp_b["scores"])
    torch.cuda.synchronize()
    pf = S.Prefetcher()
    pf.prefetch([(host[k], staged[k]) for k in names])
    T, H = inp_a["T"], cfg["n_heads"]
    oa = torch.full_like(oa_ref, float("nan"))  # Local heads outside A are never written
    za = torch.full_like(za_ref, float("nan"))
    plan_a.forward(inp_a, oa, za)          # runs beside the transfers
    pf.wait()
    ob = torch.full_like(ob_ref, float("nan"))
    zb = torch.full_like(zb_ref, float("nan"))
    plan_b.forward(dict(inp_b, **staged), ob, zb)
    torch.cuda.synchronize()
    ms = pf.elapsed_ms()
    nbytes = sum(host[k].numel() * host[k].element_size() for k in names)
    say("  staged %.1f MB in %.3f ms (%.1f GB/s)" % (nbytes / 1e6, ms, nbytes / ms / 1e6))
    for k in names:
        assert _same(staged[k], inp_b[k]), k
    assert _same(oa.nan_to_num(7), oa_ref.nan_to_num(7)) and _same(za, za_ref)
    assert _same(ob.nan_to_num(7), ob_ref.nan_to_num(7)) and _same(zb, zb_ref)
    pf.close()
    plan_a.close()
    plan_b.close()


def test_prefetch_segment_ranges_into_a_device_pool():
    """Only some segments' rows are staged (device to device, per-segment ranges with row
    strides): the other rows of the destination pool hold NaN until then, and the forward that
    waits on the prefetch reads the staged segments exactly."""
    cfg = SMALL_CONFIGS[1]
    say("case prefetch segment ranges %s" % cfg["name"])
    inp = make_inputs(cfg, "cuda")
    _, o_ref, z_ref, _ = run_gpu(inp)
    pool = {k: inp[k].clone() for k in ("kv", "z_cached")}
    segs = [1, 3]  # two documents: their latent rows and cached state arrive by prefetch
    for i in segs:
        a, n = int(inp["pool_rows"][i]), int(inp["lens"][i])
        for k in pool:
            pool[k][a:a + n] = float("nan")
    pf = S.Prefetcher()
    pairs = []
    for i in segs:
        a, n = int(inp["pool_rows"][i]), int(inp["lens"][i])
        for k in pool:
            pairs.append((inp[k][a:a + n], pool[k][a:a + n]))
    plan = Plan.for_inputs(inp)
    plan.build(inp["scores"])
    pf.prefetch(pairs)
    pf.wait()
    out = torch.full_like(o_ref, float("nan"))
    z = torch.full_like(z_ref, float("nan"))
    plan.forward(dict(inp, **pool), out, z)
    torch.cuda.synchronize()
    assert _same(out.nan_to_num(7), o_ref.nan_to_num(7)) and _same(z, z_ref)
    with pytest.raises(ValueError):
        pf.prefetch([(inp["kv"][:4].cpu(), pool["kv"][:4])])  # pageable host memory
    with pytest.raises(ValueError):
        pf.prefetch([(inp["kv"][:4], pool["kv"][:5])])
    bad = S.CopyRange(inp["kv"].data_ptr(), pool["kv"].data_ptr(), 2, 16, 8, 16)  # stride < row
    assert S.lib().segmla_prefetch(pf.handle, bad, 1, None) == S.SEGMLA_E_SHAPE
    pf.close()
    plan.close()
