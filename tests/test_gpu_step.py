"""GPU parity of the Uno decode step (uno_forward, uno_decode_step, uno_ar_step) on
reduced synthetic stacks against the oracle's composition (oracle/step.py).

* Forward logits: fp32 results of bf16 products; per row, ||z - z_ref|| <=
  2e-2 ||z_ref|| (the products' tolerance; the measured error is far smaller).
* Greedy steps: every token is the argmax of one logit row, so a token can differ
  from the oracle's only where that row's top two oracle logits are within twice
  the row's largest |z - z_ref|. Such a slot is counted as a near-tie and excuses
  its sequence from that slot on; every other draft, decision, token, accept
  length and resample must be equal, at least one sequence must be compared whole
  and at least half of all decisive slots compared. The looped stack drafts with
  one loop and verifies with two; a perturbed-identity stack keeps 1 to 8 drafts
  per block, so every slot position is decided.
* Sampled steps: the step's drafts and verify outputs equal the library's own
  draft sampler and verifier run on the step's logits. Slot 0 and the AR step run
  the same frozen stack at different row counts (S*b and S), where a product may
  take different GEMM forms whose sums round in different orders: their logits
  agree within the products' tolerance, and their tokens are equal wherever the
  oracle, drawing from either logit row with the slot's uniforms, gives one token.
* A HIP graph of the step replays the eager result bit for bit, with eager steps
  of other inputs between the replays.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from helpers import to_device
from oracle import step as ostep

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import lossless_diffusion_drafted_amd as uno
    uno.load()


def _uno():
    import lossless_diffusion_drafted_amd as uno
    return uno


_MODELS = {}


def _config(name):
    """A reduced stack's sizes; small_hd64 is the small stack with 64-wide heads."""
    if name == "small_hd64":
        return dict(workloads.STEP_CONFIGS["small"], head_dim=64)
    return workloads.STEP_CONFIGS[name]


def _models(name):
    """(host model as bf16 bits, device Model) for a reduced stack."""
    if name not in _MODELS:
        c = _config(name)
        host = workloads.step_model_host(c, seed=1)
        _MODELS[name] = (host, _device_model(host, c))
    return _MODELS[name]


def _device_model(host, c, stacked=True):
    """The host stack on the device. stacked: each layer's q, k, v (and gate, up)
    weights and adapter factors back to back in one allocation, as the benchmark's
    stacks hold them, so the forward runs them as grouped products."""
    uno = _uno()
    dev = lambda a: to_device(a, DEV)

    def layer_on_device(layer):
        if not stacked:
            return [dev(t) for t in layer]

        def pack(ts):
            return list(torch.split(dev(np.concatenate(ts, axis=0)), [t.shape[0] for t in ts], dim=0))
        return pack(layer[0:3]) + [dev(layer[3])] + pack(layer[4:6]) + [dev(layer[6])]
    lora_a = [layer_on_device(t) for t in host["lora_a"]] if host["rank"] else None
    lora_b = [layer_on_device(t) for t in host["lora_b"]] if host["rank"] else None
    return uno.Model(dev(host["embed"]), dev(host["lm_head"]), [layer_on_device(t) for t in host["weights"]],
                     lora_a, lora_b, kv_width=c["kv_width"], head_dim=c["head_dim"], lora_scale=host["lora_scale"])


def _inputs(S, V, seed):
    rng = np.random.default_rng(seed)
    seed_tok = rng.integers(0, V, S).astype(np.int32)
    seq = rng.integers(0, 2**40, S).astype(np.int64)
    pos = rng.integers(0, 10000, S).astype(np.int64)
    return seed_tok, seq, pos


@pytest.mark.parametrize("name,loops,stacked,M", [("small", 1, True, 40), ("small_looped", 2, True, 40),
                                                  ("small", 1, False, 40), ("small", 1, True, 8),
                                                  ("small_hd64", 1, True, 40)])
def test_forward_matches_oracle(name, loops, stacked, M):
    """Logits of the forward against the oracle's, with the grouped q | k | v and
    gate | up products (stacked weights) and without them. The o-projection reads
    its 128-wide heads straight from v (8 rows: one-pass kernel; 40: row tiles;
    kv groups of 4 and of 1) and 64-wide heads from an expanded copy."""
    uno = _uno()
    host, model = _models(name)
    if not stacked:
        model = _device_model(host, _config(name), stacked=False)
    V = host["embed"].shape[0]
    rng = np.random.default_rng(5)
    toks = rng.integers(0, V, M).astype(np.int32)
    mask = (rng.random(M) < 0.6).astype(np.uint8)
    z = uno.uno_forward(model, to_device(toks, DEV), to_device(mask, DEV), loops=loops)
    torch.cuda.synchronize()
    z = z.cpu().numpy().astype(np.float64)
    ref = ostep.forward(host, toks, mask, loops)
    rel = np.linalg.norm(z - ref, axis=1) / np.linalg.norm(ref, axis=1)
    print(name, "max row relative error", rel.max(), "max abs", np.abs(z - ref).max())
    assert rel.max() <= 2e-2
    z0 = uno.uno_forward(model, to_device(toks, DEV), None, loops=loops).cpu().numpy()
    ref0 = ostep.forward(host, toks, None, loops)
    assert (np.linalg.norm(z0 - ref0, axis=1) / np.linalg.norm(ref0, axis=1)).max() <= 2e-2


def _top2_gap(row):
    s = np.sort(row)
    return s[-1] - s[-2]


def _perturbed_identity():
    """lm_head = embed with projection weights ~ N(0, 0.05^2): the greedy output
    usually repeats the input token but not always, so greedy blocks keep a
    spread of 1 to 8 drafts and every slot of the block is decided."""
    if "perturbed_identity" not in _MODELS:
        c = workloads.STEP_CONFIGS["small"]
        host = workloads.step_model_host(c, seed=1, weight_sigma=0.05)
        host = dict(host, lm_head=host["embed"].copy())
        _MODELS["perturbed_identity"] = (host, _device_model(host, c))
    return _MODELS["perturbed_identity"]


@pytest.mark.parametrize("name,draft_loops,verify_loops", [("small", 1, 1), ("small_looped", 1, 2),
                                                           ("small_looped", 2, 2), ("perturbed_identity", 1, 1)])
def test_greedy_step_matches_oracle(name, draft_loops, verify_loops):
    uno = _uno()
    host, model = _perturbed_identity() if name == "perturbed_identity" else _models(name)
    c = workloads.STEP_CONFIGS["small" if name == "perturbed_identity" else name]
    b, V = c["b"], host["embed"].shape[0]
    S = 64 // b
    seed_tok, seq, pos = _inputs(S, V, 7)
    r = uno.uno_decode_step(model, b, to_device(seed_tok, DEV), to_device(seq, DEV), to_device(pos, DEV),
                            temperature=0.0, seed=4, draft_loops=draft_loops, verify_loops=verify_loops,
                            want_logits=True)
    torch.cuda.synchronize()
    g = {k: v.cpu().numpy() for k, v in r.items()}
    ref = ostep.decode_step(host, seed_tok, seq, pos, b, 0.0, 50, 0.95, 4, draft_loops, verify_loops)
    zd, zv = g["draft_logits"].astype(np.float64), g["verify_logits"].astype(np.float64)
    exact, excused, compared, decisive_total = 0, [], 0, 0
    for s in range(S):
        decisive_total += min(int(ref["accept_len"][s]), b - 1) + 1
        f = None
        # decisive slots: slot 0, the oracle's kept slots and its first rejected slot
        for i in range(min(int(ref["accept_len"][s]), b - 1) + 1):
            row = s * b + i
            if i >= 1:                          # the draft of slot i: argmax of the draft row
                if _top2_gap(ref["draft_logits"][row]) <= 2 * np.abs(zd[row] - ref["draft_logits"][row]).max():
                    f = i
                    break
                assert g["draft_tokens"][s, i] == ref["drafts"][s, i], (s, i)
            # with equal drafts so far, the verify row of slot i has the same input token
            if _top2_gap(ref["verify_logits"][row]) <= 2 * np.abs(zv[row] - ref["verify_logits"][row]).max():
                f = i
                break
        if f is None:
            assert g["accept_len"][s] == ref["accept_len"][s], s
            np.testing.assert_array_equal(g["out_tokens"][s], ref["out_tokens"][s])
            assert g["resampled"][s] == ref["resampled"][s]
            exact += 1
            compared += min(int(ref["accept_len"][s]), b - 1) + 1
        else:
            np.testing.assert_array_equal(g["out_tokens"][s, :f], ref["out_tokens"][s, :f])
            excused.append((s, f))
            compared += f
    print(name, draft_loops, verify_loops, "exact", exact, "excused (sequence, slot)", excused,
          "decisive slots compared", compared, "of", decisive_total, "accept_len", g["accept_len"],
          "oracle accept_len", ref["accept_len"])
    assert exact + len(excused) == S and exact >= 1 and 2 * compared >= decisive_total


def test_identity_model_commits_the_noise_tokens():
    """lm_head = embed and zero projection weights: greedy output repeats the input
    token, so every draft is kept and the step commits the seed and the noise
    tokens, which must be the oracle's Philox draws bit for bit."""
    uno = _uno()
    c = workloads.STEP_CONFIGS["small"]
    host = workloads.step_model_host(c, seed=4)
    host = dict(host, weights=[[np.zeros_like(w) for w in layer] for layer in host["weights"]],
                lm_head=host["embed"].copy())
    model = _device_model(host, c)
    S, b, V = c["S"], c["b"], c["vocab"]
    seed_tok, seq, pos = _inputs(S, V, 8)
    r = uno.uno_decode_step(model, b, to_device(seed_tok, DEV), to_device(seq, DEV), to_device(pos, DEV),
                            temperature=0.0, seed=21, draft_loops=1, verify_loops=2)
    torch.cuda.synchronize()
    rows, _ = ostep.block_rows(seed_tok, seq, pos, b, V, 21)
    np.testing.assert_array_equal(r["out_tokens"].cpu().numpy(), rows.reshape(S, b))
    assert np.all(r["accept_len"].cpu().numpy() == b)
    tok, _ = uno.uno_ar_step(model, to_device(seed_tok, DEV), to_device(seq, DEV), to_device(pos, DEV),
                             temperature=0.0, seed=21, loops=2)
    np.testing.assert_array_equal(tok.cpu().numpy(), seed_tok)


@pytest.mark.parametrize("name,draft_loops,verify_loops", [("small", 1, 1), ("small_looped", 1, 2)])
def test_sampled_step_composition(name, draft_loops, verify_loops):
    uno = _uno()
    host, model = _models(name)
    c = workloads.STEP_CONFIGS[name]
    S, b, V = c["S"], c["b"], host["embed"].shape[0]
    seed_tok, seq, pos = (to_device(a, DEV) for a in _inputs(S, V, 9))
    sp = dict(temperature=1.0, top_k=50, top_p=0.95, seed=12)
    r = uno.uno_decode_step(model, b, seed_tok, seq, pos, draft_loops=draft_loops, verify_loops=verify_loops,
                            want_logits=True, **sp)
    q = r["draft_logits"].view(S, b, V)
    p = r["verify_logits"].view(S, b, V)
    d, _ = uno.uno_draft_sample(q, seq, pos, **sp)
    v = uno.uno_verify_block(p, q, r["draft_tokens"], seq, pos, **sp)
    tok, z_ar = uno.uno_ar_step(model, seed_tok, seq, pos, loops=verify_loops, want_logits=True, **sp)
    torch.cuda.synchronize()
    assert torch.equal(d[:, 1:], r["draft_tokens"][:, 1:])
    for k in ("out_tokens", "accept_len", "resampled"):
        assert torch.equal(v[k], r[k]), k
    # The AR step's rows and the step's slot-0 verify rows: the same frozen stack
    # at S and S*b rows.
    za = z_ar.double().cpu().numpy()
    zb = p[:, 0].double().cpu().numpy()
    for i in range(S):
        assert np.linalg.norm(za[i] - zb[i]) <= 2e-2 * np.linalg.norm(za[i])
    seq_h, pos_h = seq.cpu().numpy(), pos.cpu().numpy()
    nodraft = np.zeros((S, 1), np.int32)
    ta = oracle.verify_block(za.astype(np.float32)[:, None], za.astype(np.float32)[:, None], nodraft,
                             seq_h, pos_h, dtype="f32", **sp)["out_tokens"][:, 0]
    tb = oracle.verify_block(zb.astype(np.float32)[:, None], zb.astype(np.float32)[:, None], nodraft,
                             seq_h, pos_h, dtype="f32", **sp)["out_tokens"][:, 0]
    same = ta == tb
    assert same.sum() >= S // 2
    np.testing.assert_array_equal(tok.cpu().numpy()[same], r["out_tokens"][:, 0].cpu().numpy()[same])
    L = r["accept_len"].cpu().numpy()
    assert np.all((L >= 1) & (L <= b))
    print(name, "accept_len", L)


def test_step_graph_replay():
    """The step recorded in a HIP graph (every kernel on one stream, workspaces made
    beforehand) replays the eager result, with eager steps of other inputs between."""
    uno = _uno()
    host, model = _models("small_looped")
    c = workloads.STEP_CONFIGS["small_looped"]
    S, b, V = c["S"], c["b"], host["embed"].shape[0]
    sp = dict(temperature=1.0, top_k=50, top_p=0.95, seed=3)
    ins = [tuple(to_device(a, DEV) for a in _inputs(S, V, k)) for k in range(3)]
    static_in = tuple(t.clone() for t in ins[0])
    out = {k: torch.empty((S, b) if k in ("out_tokens", "draft_tokens") else (S,), dtype=torch.int32, device=DEV)
           for k in ("out_tokens", "accept_len", "resampled", "draft_tokens")}
    eager = [uno.uno_decode_step(model, b, *x, draft_loops=1, verify_loops=2, **sp) for x in ins]
    torch.cuda.synchronize()
    eager = [{k: v.clone() for k, v in e.items()} for e in eager]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        uno.uno_decode_step(model, b, *static_in, draft_loops=1, verify_loops=2, out=out, **sp)   # warm-up
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        uno.uno_decode_step(model, b, *static_in, draft_loops=1, verify_loops=2, out=out, **sp)
    for rep in range(3):
        k = rep % 3
        for dst, src in zip(static_in, ins[k]):
            dst.copy_(src)
        graph.replay()
        torch.cuda.synchronize()
        for key in out:
            assert torch.equal(out[key], eager[k][key]), (rep, key)
        other = uno.uno_decode_step(model, b, *ins[(k + 1) % 3], draft_loops=1, verify_loops=2, **sp)
        torch.cuda.synchronize()
        assert torch.equal(other["out_tokens"], eager[(k + 1) % 3]["out_tokens"])


def test_step_argument_errors():
    uno = _uno()
    _, model = _models("small")
    z = torch.zeros(9, dtype=torch.int32, device=DEV)
    i64 = torch.zeros(9, dtype=torch.int64, device=DEV)
    with pytest.raises(uno.UnoError) as e:
        uno.uno_decode_step(model, 8, z, i64, i64)           # 72 rows > 64
    assert e.value.status == "UNO_ERR_UNSUPPORTED"
    with pytest.raises(uno.UnoError) as e:
        uno.uno_decode_step(model, 4, z[:2], i64[:2], i64[:2], draft_loops=0)
    assert e.value.status == "UNO_ERR_INVALID_ARG"
