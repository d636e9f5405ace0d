"""Head reordering on the GPU: the block permutation of projection weights against the
oracle's reordering (bit-exact: it is a copy), the gates-to-weights pipeline, and a cache
run in the reordered head order giving the same outputs as in native order (explainer,
"Head Reordering Preprocessing": heads are permutation-invariant)."""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import duo_oracle as O

import head_split_kv_amd as hsk
from gpu_util import to_dev

pytestmark = pytest.mark.gpu


def _bits(rng, *shape):
    """Random 16-bit patterns (bf16 weights as raw bits, any value)."""
    return rng.integers(-(1 << 15), 1 << 15, size=shape, dtype=np.int16)


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


@pytest.mark.parametrize("Hkv,G,d,hidden", [(8, 4, 128, 4096), (32, 1, 128, 4096),
                                            (3, 2, 64, 200)])
def test_projection_reorder_matches_oracle(Hkv, G, d, hidden):
    """Q, K, V rows and output-projection columns of one layer (the first two shapes are
    the Llama-3-8B and Llama-2-7B layers)."""
    rng = np.random.default_rng(71 + Hkv)
    mask = (rng.random(Hkv) < 0.5).astype(np.uint8)
    kv_order, q_order = hsk.duo_head_order(mask, G)
    Hq = Hkv * G
    wq, wk, wo = _bits(rng, Hq * d, hidden), _bits(rng, Hkv * d, hidden), _bits(rng, hidden, Hq * d)
    got_q = hsk.reorder_output_rows(_dev(wq), q_order, d).cpu().numpy()
    got_k = hsk.reorder_output_rows(_dev(wk), kv_order, d).cpu().numpy()
    got_o = hsk.reorder_input_cols(_dev(wo), q_order, d).cpu().numpy()
    assert np.array_equal(got_q, O.reorder_output_rows(wq, O.query_head_order(O.head_order(mask), G), d))
    assert np.array_equal(got_k, O.reorder_output_rows(wk, O.head_order(mask), d))
    assert np.array_equal(got_o, O.reorder_input_cols(wo, O.query_head_order(O.head_order(mask), G), d))


@pytest.mark.parametrize("outer,n_blocks,block_bytes", [
    (1, 1, 16), (1, 1024, 16), (7, 5, 48), (1000, 3, 16), (3, 17, 4096), (1, 2, 16 * 1031),
    (4096, 32, 256)])
def test_permute_blocks_shapes(outer, n_blocks, block_bytes):
    """Block sizes from one 16-byte chunk up, up to 1,024 blocks, chunk counts that leave a
    ragged last grid step."""
    rng = np.random.default_rng(outer * 31 + n_blocks)
    order = rng.permutation(n_blocks).astype(np.int32)
    src = rng.integers(0, 256, size=(outer, n_blocks, block_bytes), dtype=np.uint8)
    dst = torch.full((outer, n_blocks, block_bytes), 0xAB, dtype=torch.uint8, device="cuda")
    hsk.duo_permute_blocks(_dev(src), dst, outer, n_blocks, block_bytes, order)
    assert np.array_equal(dst.cpu().numpy(), src[:, order, :])


def test_gates_to_weights_pipeline():
    """Trained-looking gates of a 4-layer GQA model at 50 % binarized by the library, equal
    to the oracle's mask, then every layer's K projection reordered so that the layer's
    retrieval heads come first."""
    rng = np.random.default_rng(77)
    L, Hkv, G, d, hidden = 4, 8, 4, 128, 512
    alpha = np.clip(rng.normal(0.3, 0.3, (L, Hkv)), 0, 1).astype(np.float32)
    mask, tau, n = hsk.duo_binarize_gates(alpha, 0.5)
    want, want_tau = O.binarize_gates(alpha.astype(np.float64), 0.5)
    assert np.array_equal(mask, want) and tau == want_tau and n == L * Hkv // 2
    for layer in range(L):
        kv_order, _ = hsk.duo_head_order(mask[layer], G)
        wk = _bits(rng, Hkv * d, hidden)
        got = hsk.reorder_output_rows(_dev(wk), kv_order, d).cpu().numpy()
        assert np.array_equal(got, O.reorder_output_rows(wk, O.head_order(want[layer]), d))
        hr = int(mask[layer].sum())
        assert mask[layer][kv_order].tolist() == [1] * hr + [0] * (Hkv - hr)


def test_reordered_cache_gives_permuted_outputs():
    """A cache whose heads are in the reordered layout (retrieval first), fed the permuted
    q, k, v, returns exactly the permuted outputs of the native-order cache: prefill of a
    300-token prompt in chunks, then decode steps."""
    w = W.Workload("reorder-invariance", 1, 2, 16, 4, 128, "bf16", 4, 32, 0, 0, 2,
                   fixed_mask=((1, 3),), seed=79)
    mask = W.retrieval_mask(w)[0]
    kv_order, q_order = hsk.duo_head_order(mask, w.group)
    caches = []
    for m in (mask, mask[kv_order]):
        caches.append(hsk.DuoCache(num_layers=1, batch=2, num_q_heads=16, num_kv_heads=4,
                                   head_dim=128, sink=4, recent=32, capacity=400,
                                   retrieval_mask=[m], dtype=torch.bfloat16,
                                   out_dtype=torch.float32))
    n, chunk = 300, 128

    def toks(kind, c0, c1):
        return np.stack([W.tokens(w, kind, 0, b, c0, c1) for b in range(2)])

    for c0 in range(0, n, chunk):
        c1 = min(n, c0 + chunk)
        q, k, v = toks("q", c0, c1), toks("k", c0, c1), toks("v", c0, c1)
        outs = []
        for ci, (qo, ko) in enumerate(((np.arange(16), np.arange(4)), (q_order, kv_order))):
            dq, dk, dv = (to_dev(x, torch.bfloat16) for x in (q[:, :, qo], k[:, :, ko], v[:, :, ko]))
            outs.append(caches[ci].attn_prefill(0, dq, dk, dv).cpu().numpy())
            caches[ci].kv_append(0, dk, dv)
        assert np.array_equal(outs[1], outs[0][:, :, q_order]), c0
    for p in range(n, n + 3):
        q, k, v = (toks(kind, p, p + 1)[:, 0] for kind in ("q", "k", "v"))  # [B, heads, d]
        outs = []
        for ci, (qo, ko) in enumerate(((np.arange(16), np.arange(4)), (q_order, kv_order))):
            dq, dk, dv = (to_dev(x, torch.bfloat16) for x in (q[:, qo], k[:, ko], v[:, ko]))
            outs.append(caches[ci].decode_step(0, dq, dk, dv).cpu().numpy())
        assert np.array_equal(outs[1], outs[0][:, q_order]), p
