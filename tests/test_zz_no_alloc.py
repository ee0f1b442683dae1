"""lm_head_argmax_noalloc -- the entry point that allocates nothing (its
workspace is the library's own per-GPU device array) -- against
lm_head_argmax with a caller workspace, through the C ABI: two calls in a
row, the second on a smaller input, each bit-exact in index and value.  The
first call in a fresh process also covers the one-time set-up (symbol
address lookup and the counter clear)."""
import numpy as np
import pytest

import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def test_noalloc_matches_caller_workspace():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gemv_q4k_q6k_amd as gq
    L = gq.lib()
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream().cuda_stream
    K = 1024
    for N, seed in ((248_320, 31), (20_000, 32)):          # the second input is smaller
        W, x = synth.c3_inputs(seed, N=N)
        # a planted exact tie: the last row repeats row N // 3
        W = W.reshape(N, -1).copy()
        W[N - 1] = W[N // 3]
        dW = torch.from_numpy(W.reshape(-1)).to(dev)
        dx = torch.from_numpy(x).to(dev)
        ws = torch.zeros(gq.lm_head_argmax_ws_bytes(N, K), dtype=torch.uint8, device=dev)
        idx = torch.full((1,), -1, dtype=torch.int32, device=dev)
        mx = torch.full((1,), float("nan"), dtype=torch.float32, device=dev)
        idx_ref = torch.full((1,), -2, dtype=torch.int32, device=dev)
        mx_ref = torch.full((1,), float("nan"), dtype=torch.float32, device=dev)
        torch.cuda.synchronize()
        print(f"lm_head_argmax_noalloc N={N} K={K} seed={seed}", flush=True)
        held = torch.cuda.memory_allocated()
        rc = L.lm_head_argmax_noalloc(dW.data_ptr(), dx.data_ptr(), idx.data_ptr(), mx.data_ptr(), N, K, stream)
        assert rc == gq.OK, gq.strerror(rc)
        rc = L.lm_head_argmax(dW.data_ptr(), dx.data_ptr(), idx_ref.data_ptr(), mx_ref.data_ptr(), ws.data_ptr(),
                              ws.numel(), N, K, stream)
        assert rc == gq.OK, gq.strerror(rc)
        torch.cuda.synchronize()
        assert torch.cuda.memory_allocated() == held
        assert int(idx.item()) == int(idx_ref.item()), (N, int(idx.item()), int(idx_ref.item()))
        assert mx.cpu().numpy().view(np.uint32)[0] == mx_ref.cpu().numpy().view(np.uint32)[0]
        assert 0 <= int(idx.item()) < N
        # the caller workspace's counters are back at zero (the library's own
        # are checked by the second, smaller call agreeing as well)
        assert int(torch.count_nonzero(ws[:4096]).item()) == 0
