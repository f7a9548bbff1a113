"""greedy_accept_noalloc (the entry point that allocates nothing) against greedy_accept.

Through the C ABI: two calls in a row on the shared device scratch, the second with a
smaller batch and vocabulary, each bit-identical to greedy_accept with its own workspace
(accepted counts, next tokens, per-row argmax); a batch whose scratch would exceed the fixed
array is refused before any launch.
"""
import ctypes

import pytest
import torch

from dsa_sparse_attention_amd import _lib, api, synth, workloads

pytestmark = pytest.mark.gpu

W = workloads


def _inputs(base, batch, vocab, K, dtype):
    w = W.replace(base, batch=batch, vocab=vocab, rows=K + 1, logits_dtype=dtype)
    a = synth.accept_inputs(w)
    return a["logits"].cuda(), a["draft"].cuda()


def _both(logits, draft, K):
    ref = api.greedy_accept(logits, draft, K, argmax=True)
    B = logits.shape[0] // (K + 1)
    am = torch.full((B, K + 1), -7, dtype=torch.int32, device=logits.device)
    got = api.greedy_accept_noalloc(logits, draft, K, argmax=am)
    torch.cuda.synchronize()
    return ref, got


def test_noalloc_matches_greedy_accept_on_two_calls():
    print("noalloc: 32 x 6 x 151552 bf16, then 7 x 5 x 5000 f32", flush=True)
    lg, dr = _inputs(W.MTP5_VERIFY, 32, 151552, 5, "bf16")
    lg[3, 100] = lg[3].max()  # planted exact tie: the lower index wins in both
    lg[3, 7] = lg[3, 100]
    ref, got = _both(lg, dr, 5)
    for r, g in zip(ref, got):
        assert torch.equal(r, g)
    lg2, dr2 = _inputs(W.TINY, 7, 5000, 4, "f32")
    ref2, got2 = _both(lg2, dr2, 4)
    for r, g in zip(ref2, got2):
        assert torch.equal(r, g)


def test_noalloc_refuses_batches_beyond_its_scratch():
    print("noalloc: oversized batch refused before launch", flush=True)
    lib = _lib.load()
    B, K, V = 1200, 2, 151552  # 3600 rows x 37 slices x 8 bytes > 1 MiB
    assert lib.greedy_accept_workspace_size(B, K, V) > api.NOALLOC_SCRATCH_BYTES
    tiny = torch.zeros(16, dtype=torch.int32, device="cuda")
    p = ctypes.c_void_p(tiny.data_ptr())
    st = lib.greedy_accept_noalloc(p, api.DSA_BF16, V, p, B, K, V, p, p, None,
                                   ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 3  # DSA_ERR_WORKSPACE_TOO_SMALL, before any launch
    assert b"scratch" in lib.dsa_last_error()
