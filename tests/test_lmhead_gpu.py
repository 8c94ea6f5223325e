"""GPU parity of the fused lm_head -> greedy verification against the
oracle, through the C ABI (SSD guide sec. 6 compute_logits and sec. 7
temperature 0; the 2.16x EAGLE blog sec. 5 tree and sec. 6 classification
matmul).

The GPU accumulates bfloat16 products in float32 on the matrix cores; the
oracle computes the logits exactly in float64.  Rule, per row: the GPU's
argmax must be an admissible id -- one whose exact logit is within
EPS * (|h||w| of it + |h||w| of the exact argmax) of the exact maximum --
and equal to the exact argmax when that is the only admissible id; its
reported maximum must be within EPS * |h||w| of that id's exact logit.  The
chain / tree outputs must equal the oracle's rules applied to the GPU's
argmaxes, and equal the exact oracle wherever every row has one admissible
id."""
import numpy as np
import pytest

from draft_token_verification_07_amd import synth
from helpers import to_dev

pytestmark = pytest.mark.gpu

EPS = 2.0 ** -18


@pytest.fixture(scope="module", autouse=True)
def _gpu(oracle_mod):
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _say(*a):
    print("[lmhead]", *a, flush=True)


def _check_rows(oracle_mod, hidden, W, gpu_g, gpu_max, rows):
    """Rows `rows` of the flattened batch against the float64 logits."""
    z, za = oracle_mod.lmhead_logits(hidden.reshape(-1, hidden.shape[-1])[rows], W)
    g, adm = oracle_mod.lmhead_admissible(z, za, EPS)
    gg = gpu_g.reshape(-1)[rows]
    gm = gpu_max.reshape(-1)[rows]
    ok = adm[np.arange(len(rows)), gg]
    assert ok.all(), "inadmissible argmax at rows %s" % np.asarray(rows)[~ok][:5]
    single = adm.sum(axis=1) == 1
    np.testing.assert_array_equal(gg[single], g[single])
    zg = z[np.arange(len(rows)), gg]
    assert np.all(np.abs(gm - zg) <= EPS * za[np.arange(len(rows)), gg] + 1e-30)
    return g, single


def _run_chain(w):
    import torch
    import draft_token_verification_07_amd as sv
    B, R, d = w["hidden"].shape
    toks, n, gmax, mx, st = sv.spec_lmhead_verify_greedy(to_dev(w["hidden"]), to_dev(w["W"]),
                                                         to_dev(w["tokens"]) if R > 1 else None)
    torch.cuda.synchronize()
    return dict(tokens=toks.cpu().numpy(), accept_len=n.cpu().numpy(), argmax=gmax.cpu().numpy(),
                maxlogit=mx.cpu().numpy().astype(np.float64), status=st.cpu().numpy())


def _run_tree(w):
    import torch
    import draft_token_verification_07_amd as sv
    p, t, n, gmax, mx, st = sv.spec_lmhead_verify_tree(to_dev(w["hidden"]), to_dev(w["W"]), to_dev(w["tokens"]),
                                                       to_dev(w["parents"].astype(np.int32)))
    torch.cuda.synchronize()
    return dict(path=p.cpu().numpy(), tokens=t.cpu().numpy(), accept_len=n.cpu().numpy(), argmax=gmax.cpu().numpy(),
                maxlogit=mx.cpu().numpy().astype(np.float64), status=st.cpu().numpy())


def _compare_chain(oracle_mod, w, seqs=None):
    gpu = _run_chain(w)
    B, R, d = w["hidden"].shape
    V = w["W"].shape[0]
    seqs = np.arange(B) if seqs is None else np.asarray(seqs)
    rows = (seqs[:, None] * R + np.arange(R)[None]).reshape(-1)
    g, single = _check_rows(oracle_mod, w["hidden"], w["W"], gpu["argmax"], gpu["maxlogit"], rows)
    tok = w["tokens"][seqs]
    on_gpu = oracle_mod.greedy_from_argmax(gpu["argmax"][seqs], tok, V)
    for k in ("tokens", "accept_len", "status"):
        np.testing.assert_array_equal(gpu[k][seqs], on_gpu[k], err_msg=k)
    exact = oracle_mod.greedy_from_argmax(g.reshape(len(seqs), R), tok, V)
    clean = single.reshape(len(seqs), R).all(axis=1)
    for k in ("tokens", "accept_len"):
        np.testing.assert_array_equal(gpu[k][seqs][clean], exact[k][clean], err_msg=k)
    _say("  %d sequences, %d rows with a near-tie, mean accepted %.2f" %
         (len(seqs), int((~single).sum()), gpu["accept_len"][seqs].mean()))
    return gpu


# d a multiple of 64 takes the direct-to-LDS kernel (64-k stages), other d the
# register-staged one (32-k stages, a partial last stage for d = 72 and 8)
@pytest.mark.parametrize("B,R,d,V", [(2, 4, 64, 1000), (3, 7, 72, 5003), (1, 1, 8, 1), (5, 6, 256, 1283),
                                     (7, 5, 512, 20000), (40, 7, 128, 3000), (1, 1, 64, 1), (3, 2, 192, 7)])
def test_lmhead_chain_small(oracle_mod, B, R, d, V):
    _say("chain B=%d R=%d d=%d V=%d" % (B, R, d, V))
    _compare_chain(oracle_mod, synth.lmhead(9500 + d + V, B=B, R=R, d=d, V=V))


def test_lmhead_exact_ties_lowest_id(oracle_mod):
    """Duplicated weight rows give bit-identical logits; the lowest id wins."""
    w = synth.lmhead(9501, B=4, R=5, d=96, V=700)
    W = w["W"].copy()
    g = w["planted"].reshape(-1)
    W[(g + 257) % 700] = W[g]                  # a copy of every planted row elsewhere
    W[np.minimum(g, (g + 257) % 700)] = W[g]
    w["W"] = W
    gpu = _compare_chain(oracle_mod, w)
    z, _ = oracle_mod.lmhead_logits(w["hidden"].reshape(-1, 96), W)
    np.testing.assert_array_equal(gpu["argmax"].reshape(-1), np.argmax(z, axis=1))


@pytest.mark.parametrize("B,N,d,V", [(3, 16, 64, 999), (6, 32, 160, 4099)])
def test_lmhead_tree_small(oracle_mod, B, N, d, V):
    _say("tree B=%d N=%d d=%d V=%d" % (B, N, d, V))
    w = synth.lmhead(9600 + V, B=B, R=N, d=d, V=V, tree=True, p_match=0.8)
    gpu = _run_tree(w)
    rows = np.arange(B * N)
    g, single = _check_rows(oracle_mod, w["hidden"], w["W"], gpu["argmax"], gpu["maxlogit"], rows)
    on_gpu = oracle_mod.tree_from_argmax(gpu["argmax"], w["tokens"], w["parents"], V)
    for k in ("path", "tokens", "accept_len", "status"):
        np.testing.assert_array_equal(gpu[k], on_gpu[k], err_msg=k)


def test_lmhead_tree_smollm_size(oracle_mod):
    """The 2.16x EAGLE blog's tree at its model's lm_head size: 16 trees of
    32 nodes, d = 960, V = 49152 (every row checked)."""
    w = synth.lmhead(9700, B=16, R=32, d=960, V=49152, tree=True, p_match=0.8)
    gpu = _run_tree(w)
    g, single = _check_rows(oracle_mod, w["hidden"], w["W"], gpu["argmax"], gpu["maxlogit"], np.arange(16 * 32))
    on_gpu = oracle_mod.tree_from_argmax(gpu["argmax"], w["tokens"], w["parents"], 49152)
    for k in ("path", "tokens", "accept_len", "status"):
        np.testing.assert_array_equal(gpu[k], on_gpu[k], err_msg=k)
    exact = oracle_mod.tree_from_argmax(g.reshape(16, 32), w["tokens"], w["parents"], 49152)
    clean = single.reshape(16, 32).all(axis=1)
    np.testing.assert_array_equal(gpu["accept_len"][clean], exact["accept_len"][clean])
    _say("  smollm tree: %d near-tie rows, mean depth %.2f" % (int((~single).sum()), gpu["accept_len"].mean()))


def test_lmhead_chain_full_size_sampled(oracle_mod):
    """B=128, gamma=6, d=4096, V=128256 (a Llama-3-8B lm_head): the GPU runs the
    whole batch; eight sequences are checked row by row against float64."""
    w = synth.lmhead(9800)
    _compare_chain(oracle_mod, w, seqs=[0, 1, 17, 42, 63, 64, 100, 127])
