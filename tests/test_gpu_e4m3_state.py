"""GPU parity of the grouped projected state emitted as 1x128 E4M3 blocks (layer z_e4m3 = 1).

The library quantizes the bf16 grouped state z it would otherwise return ("Reading notes on
DeepSeek-V4 serving in TensorRT-LLM", Part I, FP8 dataflow bullet: E4M3 codes with one fp32
scale per block of 128 channels, for the next projection). Both sides take the quantization
decision in the same precision: the oracle's quantizer (fp32 scale amax / 448, fp32 quotient,
nearest-even E4M3 code) applied to the library's own bf16 state from the same plan with
z_e4m3 = 0 must give the library's codes and scales bit for bit, on every row. The decoded
state must also match the fp64 oracle's grouped state within the E4M3 bound (6e-2 relative
per (row, group), the latent format's tolerance). Whole requests, a chunk with key splits and a
decode row (the matrix-vector projection and the group sums) are covered.
"""
import numpy as np
import pytest
import torch

from oracle import segmla_oracle as O
from segmented_attention_amd.segmla import Plan
from tests.gpu_common import oracle_inputs, say
from workload import make_inputs
from workload.configs import GROUPED_CONFIGS

pytestmark = pytest.mark.gpu

E4M3_TOL = 6e-2


def _run(inp, cfg, q_range, split_keys=0):
    T, H = inp["T"], cfg["n_heads"]
    q0, q1 = q_range if q_range is not None else (0, T)
    n, slots, ds = q1 - q0, H // cfg["group_heads"], cfg["d_state"]
    plan = Plan.for_inputs(dict(inp, cfg=cfg), split_keys, q_range=q_range)
    plan.build(inp["scores"])
    out = torch.full((n, H, inp["d_v"]), float("nan"), dtype=inp["q"].dtype, device="cuda")
    if cfg.get("z_e4m3", 0):
        z = torch.full((n, slots, ds), 0x7F, dtype=torch.uint8, device="cuda")  # E4M3 NaN code
        zs = torch.full((n, slots, ds // 128), float("nan"), dtype=torch.float32, device="cuda")
        plan.forward(inp, out, z, z_scale=zs)
    else:
        z = torch.full((n, slots, ds), float("nan"), dtype=inp["q"].dtype, device="cuda")
        zs = None
        plan.forward(inp, out, z)
    torch.cuda.synchronize()
    plan.close()
    return out, z, zs


CASES = [(GROUPED_CONFIGS[1], None, 0), (GROUPED_CONFIGS[1], (200, 520), 128),
         (GROUPED_CONFIGS[1], "last", 0), (GROUPED_CONFIGS[2], None, 0),
         (GROUPED_CONFIGS[2], "last", 256)]


@pytest.mark.parametrize("cfg,window,split", CASES,
                         ids=["%s-%s-%d" % (c[0]["name"], c[1], c[2]) for c in CASES])
def test_e4m3_state_matches_quantizer_and_oracle(cfg, window, split):
    inp = make_inputs(cfg, "cuda")
    T = inp["T"]
    q_range = (T - 1, T) if window == "last" else window
    q0, q1 = q_range if q_range is not None else (0, T)
    say("case e4m3 state %s window %s split %d" % (cfg["name"], (q0, q1), split))
    out_b, z_b, _ = _run(inp, cfg, q_range, split)
    out_e, codes, scales = _run(inp, dict(cfg, z_e4m3=1), q_range, split)
    # the attention outputs are the same computation
    assert torch.equal(out_b.view(torch.int16), out_e.view(torch.int16))
    # quantization decision: the library's bf16 state through the oracle's quantizer
    want_c, want_s = O.quantize_e4m3_b128_fp32(z_b.float().cpu().numpy())
    got_c, got_s = codes.cpu().numpy(), scales.cpu().numpy()
    np.testing.assert_array_equal(got_s.view(np.uint32), want_s.view(np.uint32))
    np.testing.assert_array_equal(got_c, want_c)
    # the decoded state against the fp64 grouped oracle
    deq = O.e4m3_decode(got_c).reshape(*got_c.shape[:-1], -1, 128) * got_s[..., None].astype(np.float64)
    deq = deq.reshape(got_c.shape)
    ref = O.layer_forward_grouped(oracle_inputs(inp), rows=np.arange(q0, q1))
    e = O.rel_err_rows(deq.reshape(-1, deq.shape[-1]), ref["Z"].reshape(-1, deq.shape[-1]))
    say("  decoded state max rel err %.3g" % e.max())
    assert e.max() <= E4M3_TOL, "decoded E4M3 state rel err %.3g" % e.max()


def test_e4m3_state_full_size_32k():
    """The 32K Flash-like layer in groups of 8, whole request: codes and scales bit for bit
    against the oracle's quantizer on every row, the decoded state against the fp64 oracle on
    sampled rows (the first and last row of every segment and 64 seeded rows)."""
    cfg = [c for c in GROUPED_CONFIGS if c["name"] == "flash_32k_grouped_bf16"][0]
    inp = make_inputs(cfg, "cuda")
    T = inp["T"]
    say("case e4m3 state %s" % cfg["name"])
    _, z_b, _ = _run(inp, cfg, None)
    _, codes, scales = _run(inp, dict(cfg, z_e4m3=1), None)
    got_c, got_s = codes.cpu().numpy(), scales.cpu().numpy()
    for r0 in range(0, T, 4096):  # in slices: the oracle's quantizer works in fp64 temporaries
        want_c, want_s = O.quantize_e4m3_b128_fp32(z_b[r0:r0 + 4096].float().cpu().numpy())
        np.testing.assert_array_equal(got_s[r0:r0 + 4096].view(np.uint32), want_s.view(np.uint32))
        np.testing.assert_array_equal(got_c[r0:r0 + 4096], want_c)
    offs = np.asarray(inp["offsets"], dtype=np.int64)
    lens = np.asarray(inp["lens"], dtype=np.int64)
    rng = np.random.default_rng(cfg["seed"])
    rows = np.unique(np.concatenate([offs, offs + lens - 1, rng.integers(0, T, 64)]))
    ref = O.layer_forward_grouped(oracle_inputs(inp, lazy=True), rows=rows)
    sel = got_c[rows]
    deq = (O.e4m3_decode(sel).reshape(*sel.shape[:-1], -1, 128) *
           got_s[rows][..., None].astype(np.float64)).reshape(sel.shape)
    e = O.rel_err_rows(deq.reshape(-1, deq.shape[-1]), ref["Z"].reshape(-1, deq.shape[-1]))
    say("  decoded state max rel err %.3g over %d rows" % (e.max(), rows.size))
    assert e.max() <= E4M3_TOL
