"""A decode step's GEMV sequence captured in one HIP graph and replayed.

The entry points allocate nothing, never synchronise and leave the argmax
workspace counters zero after every call, so a captured sequence can be
replayed any number of times (the graph-replay decode loop of memra-engine
decode.rs, `decode_step_dc_cap`).  Each replay is checked bit for bit against
the same calls made eagerly on the same inputs, with the inputs changed and
other GPU work done between replays, so the graph is known to read its inputs
live and to reset its own state.
"""
import numpy as np
import pytest

import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gemv_q4k_q6k_amd as gq
    gq.lib()
    return torch.device("cuda:0")


def up(a, dev):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def test_decode_step_graph_replays(dev):
    import gemv_q4k_q6k_amd as gq
    r = synth.rng_for(2024)
    shapes = {"attn": (4096, 2560), "lm": (20_000, 1024), "ffn": (2048, 2560), "q8": (3000, 8192)}
    Wa = up(synth.q4k_weights(r, *shapes["attn"]), dev)
    Wl = up(synth.q6k_weights(r, *shapes["lm"]), dev)
    Wg = up(synth.q4k_weights(r, *shapes["ffn"]), dev)
    Wu = up(synth.q4k_weights(r, *shapes["ffn"]), dev)
    Wd = up(synth.q6k_weights(r, shapes["ffn"][1], shapes["ffn"][0]), dev)
    W8 = up(synth.q4k_weights(r, *shapes["q8"]), dev)
    N_lm, K_lm = shapes["lm"]
    mask_bits = np.random.default_rng(3).random(N_lm) < 0.5
    mask = up(np.packbits(np.concatenate([mask_bits, np.zeros((-N_lm) % 32, bool)]),
                          bitorder="little").view(np.int32), dev)

    xa = torch.empty(shapes["attn"][1], device=dev)
    xl = torch.empty(K_lm, device=dev)
    xf = torch.empty(shapes["ffn"][1], device=dev)
    x8 = torch.empty(shapes["q8"][1], device=dev)

    def new_inputs(seed):
        g = torch.Generator(device="cpu").manual_seed(seed)
        for t in (xa, xl, xf, x8):
            t.copy_(torch.randn(t.numel(), generator=g))

    def outputs():
        return {
            "ya": torch.empty(shapes["attn"][0], device=dev),
            "idx": torch.empty(1, dtype=torch.int32, device=dev),
            "vmax": torch.empty(1, device=dev),
            "midx": torch.empty(1, dtype=torch.int32, device=dev),
            "h": torch.empty(shapes["ffn"][0], device=dev),
            "yd": torch.empty(shapes["ffn"][1], device=dev),
            "xq": torch.empty(shapes["q8"][1], dtype=torch.int8, device=dev),
            "xd": torch.empty(shapes["q8"][1] // 32, dtype=torch.int16, device=dev),
            "y8": torch.empty(shapes["q8"][0], device=dev),
        }

    ws = torch.zeros(gq.lm_head_argmax_ws_bytes(N_lm, K_lm), dtype=torch.uint8, device=dev)
    ws2 = torch.zeros_like(ws)

    def step(o, ws_, ws_m):
        gq.q4k_gemv(Wa, xa, *shapes["attn"], y=o["ya"])
        gq.lm_head_argmax(Wl, xl, N_lm, K_lm, ws_, out_idx=o["idx"], out_max=o["vmax"])
        gq.lm_head_argmax_masked(Wl, xl, mask, N_lm, K_lm, ws_m, out_idx=o["midx"])
        gq.swiglu_gemv(Wg, Wu, xf, *shapes["ffn"], h=o["h"])
        gq.q6k_gemv(Wd, o["h"], shapes["ffn"][1], shapes["ffn"][0], y=o["yd"])
        gq.q8_quantize(x8, xq=o["xq"], xd=o["xd"])
        gq.q4k_q8_gemv(W8, o["xq"], o["xd"], *shapes["q8"], y=o["y8"])

    # eager warm-up (fills the library's per-device caches outside capture)
    new_inputs(0)
    og = outputs()
    step(og, ws, ws2)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(og, ws, ws2)

    ref_ws = torch.zeros_like(ws)
    ref_ws2 = torch.zeros_like(ws)
    for rep in range(4):
        new_inputs(100 + rep)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        oe = outputs()
        step(oe, ref_ws, ref_ws2)                 # the same calls, eagerly
        junk = torch.randn(1 << 20, device=dev)   # unrelated GPU work between replays
        (junk * 2).sum().item()
        torch.cuda.synchronize()
        for k in og:
            assert torch.equal(og[k], oe[k]), (rep, k)
        for w in (ws, ws2):
            assert int(torch.count_nonzero(w[:4096]).item()) == 0, rep
