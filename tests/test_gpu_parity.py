"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the
same seeded inputs.  Marked gpu; run on an MI355X.

Sizes: the tiny F32 model (several GEMV tiles per matrix, a ragged 16-row
prompt against 32-row prefill chunks), a reduced model at the full 1024/3072
widths, and the full 28-layer BF16 / Q8 / Q4 models at their real shapes."""
import dataclasses
import sys

import numpy as np
import pytest

from autoregressive_codebook_tts_frame_amd import synth
from parity import assert_near_ties_only, code_mismatches, margin, rel_l2, tol_for

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("needs a GPU", allow_module_level=True)

from autoregressive_codebook_tts_frame_amd import qt  # noqa: E402
from oracle import Oracle  # noqa: E402
from oracle.oracle import sample_scores  # noqa: E402


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _forced_run(m, w, wl, nframes, batch=1, dump_hidden=False, prompts=None, sampler=None, flags=0, pool_rows=0,
                order=None):
    """Oracle free run, then the GPU teacher-forced with the oracle's codes
    (one frame per call, dumps read after each) and free-running.
    sampler: (temperature, seed) set on both sides before the prefill.
    pool_rows: a paged ring of that many rows; order: the GPU's prefill order."""
    prompts = prompts or [synth.make_prompt(wl, b) for b in range(batch)]
    ov = synth.make_overlays(wl, nframes, batch)
    o = Oracle(m, w, batch, pcap=max(len(p[1]) for p in prompts) + nframes + 1)
    if sampler:
        o.set_sampler(*sampler)
    pre_logits = []
    for b, (c, t) in enumerate(prompts):
        pre_logits.append(o.prefill(b, c, t, dump=True)["logits"])
    ostate = [o.get_state(b) for b in range(batch)]
    oout = o.decode(nframes, ov, dump=True, hidden=dump_hidden)

    d = qt.Decoder(m, w, batch, flags=qt.QT_F_DUMP | flags, pool_rows=pool_rows)
    if sampler:
        d.set_sampler(*sampler)
    for b in (order or range(batch)):
        d.prefill(b, *prompts[b])
    gstate = [d.get_state(b) for b in range(batch)]
    gpre = d.dump(qt.QT_DUMP_TALKER_LOGITS)
    g = {k: [] for k in ("codes", "talker_logits", "pred_logits", "bridge", "x0", "gather", "tpos", "hidden")}
    for f in range(nframes):
        g["codes"].append(d.decode(1, ov[f:f + 1], forced=oout["codes"][f:f + 1])[0])
        g["talker_logits"].append(d.dump(qt.QT_DUMP_TALKER_LOGITS))
        g["pred_logits"].append(d.dump(qt.QT_DUMP_PRED_LOGITS).transpose(1, 0, 2))
        g["bridge"].append(d.dump(qt.QT_DUMP_BRIDGE))
        g["x0"].append(d.dump(qt.QT_DUMP_X0))
        g["gather"].append(d.dump(qt.QT_DUMP_GATHER))
        g["tpos"].append(d.dump(qt.QT_DUMP_TPOS))
        if dump_hidden:
            g["hidden"].append(d.dump(qt.QT_DUMP_HIDDEN).transpose(1, 0, 2))
    g = {k: np.stack(v) for k, v in g.items() if v}
    return dict(o=o, d=d, ov=ov, prompts=prompts, pre_logits=pre_logits, ostate=ostate,
                oout=oout, gstate=gstate, gpre=gpre, g=g, sampler=sampler, flags=flags,
                q0=[len(t) for _, t in prompts], pool_rows=pool_rows)


def _read_state(d, b, length):
    """Slot b's decode state after a GPU prefill: talker K/V of positions
    [0, length) as float32 [Lt][length][nkv][hd] (the oracle's layout), and
    (pos, c0, bridge)."""
    m = d.m
    ring = d.talker_ring()[b, :, :, :, :length, :].cpu().numpy()  # [Lt][2][nkv][L][hd]
    if m.kv_bf16:
        ring = synth.bf16_bits_to_f32(ring.view(np.uint16))
    kv = np.ascontiguousarray(ring.transpose(0, 1, 3, 2, 4))  # [Lt][2][L][nkv][hd]
    return kv, d.get_state(b)


def _prefilled_state_run(m, w, wl, nframes, prompts, sample, frames_per_replay=1):
    """The GPU prefills every stream's prompt (qt_prefill); the decode state
    of the streams in `sample` (ring rows, position, code 0, bridge) is read
    back and given to the oracle, so both sides start the decode from one
    bitwise state (the long-context and multi-stream workloads' contexts are
    prefilled from seeded prompts).  Then the oracle decodes free-running and
    the GPU decodes teacher-forced with the oracle's codes, one frame per call
    with the dumps read after each frame."""
    B = len(prompts)
    ov = synth.make_overlays(wl, nframes, B)
    d = qt.Decoder(m, w, B, frames_per_replay=frames_per_replay, flags=qt.QT_F_DUMP)
    for b, (c, t) in enumerate(prompts):
        d.prefill(b, c, t)
    torch.cuda.synchronize()
    lengths = [len(prompts[b][1]) for b in sample]
    o = Oracle(m, w, len(sample), pcap=max(lengths) + nframes + 1)
    gstate = {}
    for i, b in enumerate(sample):
        kv, (pos, c0, br) = _read_state(d, b, lengths[i])
        for layer in range(m.Lt):
            o.set_cache(i, layer, 0, kv[layer, 0], kv[layer, 1])
        o.set_state(i, pos, c0, br)
        gstate[b] = (pos, c0, br)
    oout = o.decode(nframes, ov[:, sample], dump=True)
    forced = np.zeros((nframes, B, m.G), np.int32)
    forced[:, sample] = oout["codes"]
    g = {k: [] for k in ("codes", "talker_logits", "pred_logits", "bridge", "x0", "gather", "tpos")}
    for f in range(nframes):
        g["codes"].append(d.decode(1, ov[f:f + 1], forced=forced[f:f + 1])[0][sample])
        g["talker_logits"].append(d.dump(qt.QT_DUMP_TALKER_LOGITS)[sample])
        g["pred_logits"].append(d.dump(qt.QT_DUMP_PRED_LOGITS).transpose(1, 0, 2)[sample])
        g["bridge"].append(d.dump(qt.QT_DUMP_BRIDGE)[sample])
        g["x0"].append(d.dump(qt.QT_DUMP_X0)[sample])
        g["gather"].append(d.dump(qt.QT_DUMP_GATHER)[sample])
        g["tpos"].append(d.dump(qt.QT_DUMP_TPOS)[sample])
    g = {k: np.stack(v) for k, v in g.items()}
    return dict(o=o, d=d, ov=ov, prompts=[None] * len(sample), pre_logits=None, oout=oout, g=g,
                sample=sample, pstate=gstate, lengths=lengths)


def _check(r, m, label, free_run=True):
    tol = tol_for(m)
    oout, g = r["oout"], r["g"]
    B = len(r["prompts"])
    worst = {}
    for b in range(B if r["pre_logits"] is not None else 0):
        # prefill: position, bridge, logits
        assert r["gstate"][b][0] == r["ostate"][b][0]
        worst["prefill_bridge"] = max(worst.get("prefill_bridge", 0), rel_l2(r["gstate"][b][2], r["ostate"][b][2]))
        worst["prefill_logits"] = max(worst.get("prefill_logits", 0), rel_l2(r["gpre"][b], r["pre_logits"][b]))
    for f in range(oout["codes"].shape[0]):
        for b in range(B):
            # one tensor per step: talker logits [Vc], bridge [H], x0 [H], and the
            # step's predictor logits [G-1][Vc] (what the dump returns per stream)
            for key in ("talker_logits", "bridge", "x0", "pred_logits"):
                worst[key] = max(worst.get(key, 0), rel_l2(g[key][f, b], oout[key][f, b]))
            for j in range(m.G - 1):  # and each predictor head's row on its own
                worst["pred_head_row"] = max(worst.get("pred_head_row", 0),
                                             rel_l2(g["pred_logits"][f, b, j], oout["pred_logits"][f, b, j]))
            if "hidden" in g:
                for l in range(m.Lt):
                    worst["hidden"] = max(worst.get("hidden", 0), rel_l2(g["hidden"][f, b, l], oout["hidden"][f, b, l]))
    say(f"[{label}] worst rel-L2 (tol {tol}):", {k: f"{v:.2e}" for k, v in worst.items()})
    for k, v in worst.items():
        assert v <= tol, f"{label}: {k} rel-L2 {v} > {tol}"
    # integer work is bit-exact: gather indices and K/V write positions
    assert np.array_equal(g["gather"], oout["gather"])
    assert np.array_equal(g["tpos"], oout["tpos"])

    # (code 0 of the first frame comes from the prefill, or is the injected
    # state's on both sides)
    # the values a decision maximises: the logits, or under a sampler the
    # scores logits * (1/T) + Gumbel noise of the code's key
    samp = r.get("sampler")
    top_k = samp[2] if samp and len(samp) > 2 else 0

    def scores(lg, f, b, j):
        if not samp:
            return lg
        return sample_scores(lg, samp[0], samp[1], b, r["q0"][b] + f, j, top_k)

    def ref_logits(f, b, j):
        if j == 0:
            return scores(r["pre_logits"][b] if f == 0 else oout["talker_logits"][f - 1, b], f, b, j)
        return scores(oout["pred_logits"][f, b, j - 1], f, b, j)

    def gpu_logits(f, b, j):
        if j == 0:
            return scores(r["gpre"][b] if f == 0 else g["talker_logits"][f - 1, b], f, b, j)
        return scores(g["pred_logits"][f, b, j - 1], f, b, j)

    if top_k:
        # under top-k a decision may also differ where membership is a near
        # tie: the oracle's k-th and (k+1)-th logits within 4x the logit error
        raw_ref = lambda f, b, j: (r["pre_logits"][b] if f == 0 else oout["talker_logits"][f - 1, b]) if j == 0 \
            else oout["pred_logits"][f, b, j - 1]
        raw_gpu = lambda f, b, j: (r["gpre"][b] if f == 0 else g["talker_logits"][f - 1, b]) if j == 0 \
            else g["pred_logits"][f, b, j - 1]
        diff = list(zip(*np.nonzero(g["codes"] != oout["codes"])))
        say(f"[{label}] teacher-forced decisions differing: {len(diff)} of {g['codes'].size}")
        for f, b, j in diff:
            rl, gl = np.asarray(raw_ref(f, b, j), np.float64), np.asarray(raw_gpu(f, b, j), np.float64)
            dl = float(np.max(np.abs(rl - gl)))
            srt = np.sort(rl)[::-1]
            s_ref, s_gpu = scores(raw_ref(f, b, j), f, b, j), scores(raw_gpu(f, b, j), f, b, j)
            both = np.isfinite(s_ref) & np.isfinite(s_gpu)
            ds = float(np.max(np.abs(s_ref[both] - s_gpu[both]))) if both.any() else np.inf
            boundary = srt[top_k - 1] - srt[top_k]
            mg = margin(s_ref[np.isfinite(s_ref)])
            say(f"[{label}] code flip frame {f} stream {b} code {j}: score margin {mg:.3e} (err {ds:.3e}), "
                f"k-th gap {boundary:.3e} (logit err {dl:.3e})")
            assert boundary <= 4 * dl or mg <= 4 * ds, f"{label}: top-k decision differs away from a near tie"
        bad = diff
    else:
        bad = code_mismatches(g["codes"], oout["codes"], ref_logits, gpu_logits)
        say(f"[{label}] teacher-forced decisions differing: {len(bad)} of {g['codes'].size}")
        assert_near_ties_only(bad, label)
    if free_run and not bad and "pstate" in r:
        # free running from the same prefilled state reproduces the oracle's
        # codes (the sampled streams restart from their state; the ring rows
        # past it are rewritten at the same positions before they are read)
        d2 = r["d"]
        for b, st in r["pstate"].items():
            d2.set_state(b, *st)
        n = oout["codes"].shape[0]
        codes = d2.decode(n, r["ov"])[:, r["sample"]]
        assert np.array_equal(codes, oout["codes"]), f"{label}: free-run codes differ"
    elif free_run and not bad:
        # free running from the same prefill reproduces the oracle's codes
        d2 = qt.Decoder(m, r["d"].dw, B, flags=r.get("flags", 0), pool_rows=r.get("pool_rows", 0))
        if r.get("sampler"):
            d2.set_sampler(*r["sampler"])
        for b, (c, t) in enumerate(r["prompts"]):
            d2.prefill(b, c, t)
        n = oout["codes"].shape[0]
        codes = d2.decode(n, r["ov"])
        assert np.array_equal(codes, oout["codes"]), f"{label}: free-run codes differ"
        d2.close()


# ----------------------------------------------------------------- tiny F32


@pytest.fixture(scope="module")
def tiny():
    m = synth.TINY
    wl = synth.WORKLOADS["tiny_f32_b1"]
    w = synth.make_weights(m)
    say("[tiny] running oracle + GPU, 8 frames")
    return m, w, wl, _forced_run(m, w, wl, 8, dump_hidden=True)


def test_tiny_f32_parity(tiny):
    m, w, wl, r = tiny
    assert r["d"].path == qt.QT_PATH_FRAME  # one stream: the persistent kernel
    _check(r, m, "tiny_f32")
    # F32: the oracle's codes come out free-running with no near ties
    assert np.array_equal(r["g"]["codes"], r["oout"]["codes"])


def test_tiny_traced_kernel_equals_plain():
    # the QT_F_TRACE instantiation of the persistent kernel (phase stamps
    # compiled in) decodes the same bits as the one without them, and stamps
    # one row per GEMV phase of the call's first frame, in order
    m = synth.TINY
    w = synth.make_weights(m)
    wl = synth.WORKLOADS["tiny_f32_b1"]
    codes, text = synth.make_prompt(wl, 0)
    ov = synth.make_overlays(wl, 4)
    out, tr = {}, None
    for trace in (False, True):
        say(f"[tiny traced] trace {trace}")
        d = qt.Decoder(m, w, 1, flags=qt.QT_F_DUMP | (qt.QT_F_TRACE if trace else 0))
        assert d.path == qt.QT_PATH_FRAME
        d.prefill(0, codes, text)
        out[trace] = (d.decode(4, ov), d.dump(qt.QT_DUMP_TALKER_LOGITS), d.dump(qt.QT_DUMP_PRED_LOGITS),
                      d.dump(qt.QT_DUMP_BRIDGE))
        if trace:
            tr = d.dump(qt.QT_DUMP_TRACE).astype(np.int64)
        d.close()
    assert np.array_equal(out[False][0], out[True][0])
    for a, b in zip(out[False][1:], out[True][1:]):
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    n = next(i for i in range(768) if tr[i, 0] == 255)
    assert n == (m.G - 1) * (4 * m.Lp + 1) + 4 * m.Lt + 1  # predictor steps, then the talker step
    assert np.all(np.diff(tr[:n, 1]) > 0)  # phase starts in order
    assert np.all(tr[:n, 2] >= tr[:n, 1]) and np.all(tr[:n, 3] >= tr[:n, 2])


def test_tiny_graph_equals_eager_bitwise(tiny):
    m, w, wl, r = tiny
    c, t = r["prompts"][0]
    outs = []
    for flags in (qt.QT_F_DUMP | qt.QT_F_OPS, qt.QT_F_DUMP | qt.QT_F_EAGER):
        d = qt.Decoder(m, r["d"].dw, 1, flags=flags)
        assert d.path == (qt.QT_PATH_GRAPH if flags & qt.QT_F_OPS else qt.QT_PATH_EAGER)
        d.prefill(0, c, t)
        codes = d.decode(8, r["ov"])
        outs.append((codes, d.dump(qt.QT_DUMP_TALKER_LOGITS), d.dump(qt.QT_DUMP_PRED_LOGITS),
                     d.get_state(0)[2]))
        d.close()
    for a, b in zip(*outs):
        assert np.array_equal(a.view(np.uint32) if a.dtype == np.float32 else a,
                              b.view(np.uint32) if b.dtype == np.float32 else b)


def test_tiny_repeat_runs_identical_and_multi_frame_call(tiny):
    m, w, wl, r = tiny
    c, t = r["prompts"][0]
    runs = []
    for _ in range(2):
        d = qt.Decoder(m, r["d"].dw, 1)
        d.prefill(0, c, t)
        runs.append(d.decode(8, r["ov"]))
        d.close()
    assert np.array_equal(runs[0], runs[1])
    assert np.array_equal(runs[0], r["oout"]["codes"])


def test_tiny_adaptive_k_any_frame_count(tiny):
    # four frames per graph replay, calls of 1, 3 and 6 frames (one 1-frame
    # graph replay, three, then a 4-frame replay and two 1-frame ones): the
    # codes of one 10-frame call with one frame per replay, bit for bit
    m, w, wl, r = tiny
    ov = synth.make_overlays(wl, 10)
    prompt = synth.make_prompt(wl, 0)
    d1 = qt.Decoder(m, r["d"].dw, 1, flags=qt.QT_F_OPS)
    d1.prefill(0, *prompt)
    ref = d1.decode(10, ov)
    d4 = qt.Decoder(m, r["d"].dw, 1, frames_per_replay=4, max_frames_per_call=8, flags=qt.QT_F_OPS)
    d4.prefill(0, *prompt)
    got = np.concatenate([d4.decode(1, ov[:1]), d4.decode(3, ov[1:4]), d4.decode(6, ov[4:])])
    say("[tiny adaptive K] calls of 1, 3, 6 frames at K = 4 (6 = a 4-frame replay + 2 single ones)")
    assert np.array_equal(got, ref)
    d1.close()
    d4.close()


def test_tiny_batched_equals_per_stream_and_permutation(tiny):
    m, w, wl, r = tiny
    wl3 = dataclasses.replace(wl, batch=3)
    prompts = [synth.make_prompt(wl3, b, T=9 + 5 * b) for b in range(3)]
    ov = synth.make_overlays(wl3, 4)
    d = qt.Decoder(m, r["d"].dw, 3, flags=qt.QT_F_DUMP)
    for b, (c, t) in enumerate(prompts):
        d.prefill(b, c, t)
    cb = d.decode(4, ov)
    lb = d.dump(qt.QT_DUMP_PRED_LOGITS)
    # permuted slots give permuted outputs, bit for bit
    perm = [2, 0, 1]
    dp = qt.Decoder(m, r["d"].dw, 3, flags=qt.QT_F_DUMP)
    for s, b in enumerate(perm):
        dp.prefill(s, *prompts[b])
    cp = dp.decode(4, ov[:, perm])
    assert np.array_equal(cp, cb[:, perm])
    assert np.array_equal(dp.dump(qt.QT_DUMP_PRED_LOGITS).view(np.uint32), lb[:, perm].view(np.uint32))
    for b in range(3):
        # the same per-op kernels at batch 1 (the persistent kernel orders
        # its reductions differently, so it is compared to the oracle instead)
        d1 = qt.Decoder(m, r["d"].dw, 1, flags=qt.QT_F_DUMP | qt.QT_F_OPS)
        d1.prefill(0, *prompts[b])
        c1 = d1.decode(4, ov[:, b:b + 1])
        assert np.array_equal(c1[:, 0], cb[:, b])
        assert np.array_equal(d1.dump(qt.QT_DUMP_PRED_LOGITS)[:, 0].view(np.uint32), lb[:, b].view(np.uint32))
        d1.close()
    # and the oracle agrees on every stream
    o = Oracle(m, w, 3)
    for b, (c, t) in enumerate(prompts):
        o.prefill(b, c, t)
    assert np.array_equal(o.decode(4, ov)["codes"], cb)


def test_tiny_frame_kernel_equals_op_graph_codes(tiny):
    m, w, wl, r = tiny
    c, t = r["prompts"][0]
    out = {}
    for flags in (0, qt.QT_F_OPS):
        d = qt.Decoder(m, r["d"].dw, 1, flags=flags)
        d.prefill(0, c, t)
        out[flags] = (d.decode(8, r["ov"]), d.get_state(0))
        d.close()
    assert np.array_equal(out[0][0], out[qt.QT_F_OPS][0])
    assert out[0][1][:2] == out[qt.QT_F_OPS][1][:2]
    assert rel_l2(out[0][1][2], out[qt.QT_F_OPS][1][2]) < 1e-5


def test_tiny_poisoned_ring_tail_and_predictor_cache(tiny):
    m, w, wl, r = tiny
    c, t = r["prompts"][0]
    d = qt.Decoder(m, r["d"].dw, 1)
    d.prefill(0, c, t)
    tr = d.talker_ring()
    tr[0, :, :, :, len(t):, :] = float("nan")   # positions past the context
    d.predictor_ring()[...] = float("nan")      # stale predictor rows
    torch.cuda.synchronize()
    assert np.array_equal(d.decode(8, r["ov"]), r["oout"]["codes"])


def test_tiny_errors_leave_state_unchanged(tiny):
    m, w, wl, r = tiny
    c, t = r["prompts"][0]
    d = qt.Decoder(m, r["d"].dw, 1)
    with pytest.raises(qt.QtError) as e:
        d.decode(1, r["ov"][:1])
    assert e.value.code == qt.QT_E_STATE
    d.prefill(0, c, t)
    bad = r["ov"][:1].copy()
    bad[0, 0] = m.Vt
    with pytest.raises(qt.QtError) as e:
        d.decode(1, bad)
    assert e.value.code == qt.QT_E_RANGE
    with pytest.raises(qt.QtError) as e:
        d.decode(m.P, np.zeros((m.P, 1), np.int32))
    assert e.value.code == qt.QT_E_CONTEXT_FULL
    # empty calls and a prompt longer than the ring are refused before any launch
    with pytest.raises(qt.QtError) as e:
        d.decode(0, np.zeros((0, 1), np.int32))
    assert e.value.code == qt.QT_E_ARG
    with pytest.raises(qt.QtError) as e:
        d.prefill(0, np.zeros((0, m.G), np.int32), np.zeros((0,), np.int32))
    assert e.value.code == qt.QT_E_ARG
    with pytest.raises(qt.QtError) as e:
        d.prefill(0, np.zeros((m.P + 1, m.G), np.int32), np.zeros((m.P + 1,), np.int32))
    assert e.value.code == qt.QT_E_CONTEXT_FULL
    assert d.get_state(0)[0] == len(t)
    assert np.array_equal(d.decode(8, r["ov"]), r["oout"]["codes"])


# ----------------------------------------------------------------- sampling


@pytest.mark.parametrize("flags", [0, qt.QT_F_OPS])
def test_tiny_sampled_parity(tiny, flags):
    # temperature sampling in the persistent kernel and the per-op graph: F32
    # codes equal the oracle's free-running, teacher-forced values in tolerance
    m, w, wl, r = tiny
    say(f"[tiny sampled] flags {flags}, 8 frames, T = 1.0")
    rs = _forced_run(m, w, wl, 8, sampler=(1.0, 77), flags=flags)
    assert rs["d"].path == (qt.QT_PATH_GRAPH if flags else qt.QT_PATH_FRAME)
    _check(rs, m, "tiny_sampled")
    assert np.array_equal(rs["g"]["codes"], rs["oout"]["codes"])
    # sampling at T = 1 on these logits is not the greedy decode
    assert np.mean(rs["oout"]["codes"] != r["oout"]["codes"]) > 0.5


@pytest.mark.parametrize("flags", [0, qt.QT_F_OPS], ids=["frame", "ops"])
@pytest.mark.parametrize("top_k", [1, 5, 200, 255])
def test_tiny_top_k_parity(tiny, top_k, flags):
    # top-k on the persistent kernel (every workgroup polls the head's logits
    # and runs the radix select) and on the per-op path (radix select in the
    # argmax kernel): F32 codes equal the oracle's free-running; top_k = 1 is
    # the greedy decode, 255 drops one logit of 256
    m, w, wl, r = tiny
    say(f"[tiny top-k] flags {flags}, k = {top_k}, 8 frames, T = 1.0")
    rs = _forced_run(m, w, wl, 8, sampler=(1.0, 31, top_k), flags=flags)
    assert rs["d"].path == (qt.QT_PATH_GRAPH if flags else qt.QT_PATH_FRAME)
    _check(rs, m, f"tiny_top{top_k}")
    assert np.array_equal(rs["g"]["codes"], rs["oout"]["codes"])
    if top_k == 1:
        assert np.array_equal(rs["oout"]["codes"], r["oout"]["codes"])


def test_tiny_sampled_batched_keys_by_slot(tiny):
    m, w, wl, r = tiny
    wl3 = dataclasses.replace(wl, batch=3)
    prompts = [synth.make_prompt(wl3, 0, T=12)] * 3  # one prompt in every slot
    ov = np.repeat(synth.make_overlays(wl3, 4)[:, :1], 3, axis=1)
    d = qt.Decoder(m, r["d"].dw, 3)
    d.set_sampler(0.7, 5)
    for b, (c, t) in enumerate(prompts):
        d.prefill(b, c, t)
    cb = d.decode(4, ov)
    o = Oracle(m, w, 3)
    o.set_sampler(0.7, 5)
    for b, (c, t) in enumerate(prompts):
        o.prefill(b, c, t)
    assert np.array_equal(o.decode(4, ov)["codes"], cb)
    # identical inputs, different slots: different draws
    assert not np.array_equal(cb[:, 0], cb[:, 1])
    with pytest.raises(qt.QtError) as e:
        d.set_sampler(-1.0, 0)
    assert e.value.code == qt.QT_E_ARG
    with pytest.raises(qt.QtError) as e:
        d.set_sampler(float("nan"), 0)
    assert e.value.code == qt.QT_E_ARG


# ----------------------------------------------------------------- BF16 / Q8


def _reduced(base, **kw):
    return dataclasses.replace(base, Lt=2, Lp=1, Vt=4096, P=512, model_id=base.model_id + 20, **kw)


def test_reduced_bf16_full_width_parity():
    m = _reduced(synth.BIG)
    w = synth.make_weights(m)
    # a 358-row prompt: one prompt chunk (a 512-row bucket) whose last 64-row
    # GEMM block is ragged at 38 rows; decode over 2 attention tiles
    wl = dataclasses.replace(synth.WORKLOADS["bf16_b1"], model=m, prompt=358)
    say("[reduced bf16] prompt 358, 6 frames")
    _check(_forced_run(m, w, wl, 6, dump_hidden=True), m, "reduced_bf16")


@pytest.mark.parametrize("nq,nkv,hd", [(8, 8, 128), (16, 4, 64)], ids=["group1_hd128", "group4_hd64"])
def test_gqa_groups_parity(nq, nkv, hd):
    # GQA groups other than the persistent kernel's (2): the per-op path with
    # one query head per KV head (prompt chunks on the MFMA prompt attention)
    # and four per KV head at head dim 64 (prompt chunks on the decode tiles);
    # two streams, a 300-row and a 77-row prompt, 3 frames
    m = dataclasses.replace(synth.BIG, Lt=2, Lp=1, Vt=4096, P=512, model_id=synth.BIG.model_id + 60 + nkv,
                            nq=nq, nkv=nkv, hd=hd)
    w = synth.make_weights(m)
    wl = dataclasses.replace(synth.WORKLOADS["bf16_b1"], model=m)
    prompts = [synth.make_prompt(wl, 0, T=300), synth.make_prompt(wl, 1, T=77)]
    say(f"[gqa nq={nq} nkv={nkv} hd={hd}] prompts 300 and 77, 3 frames")
    r = _forced_run(m, w, wl, 3, batch=2, prompts=prompts)
    assert r["d"].path == qt.QT_PATH_GRAPH
    _check(r, m, f"gqa_{nq}_{nkv}_{hd}")
    r["d"].close()


def test_reduced_bf16_sampled_parity():
    # full widths, one stream (persistent kernel) and eight (MFMA GEMM path)
    m = _reduced(synth.BIG)
    w = synth.make_weights(m)
    wl = dataclasses.replace(synth.WORKLOADS["q8_b8"], model=m, prompt=40)
    for batch in (1, 8):
        say(f"[reduced bf16 sampled] 4 frames, batch {batch}, T = 0.8")
        _check(_forced_run(m, w, wl, 4, batch=batch, sampler=(0.8, 2024)), m, f"reduced_bf16_sampled_b{batch}")
    for batch in (1, 8):
        say(f"[reduced bf16 top-k] 4 frames, batch {batch}, T = 0.8, k = 50")
        _check(_forced_run(m, w, wl, 4, batch=batch, sampler=(0.8, 2024, 50)), m, f"reduced_bf16_top50_b{batch}")


def test_reduced_q8_random_scales_parity():
    # one stream on the persistent kernel (its loader waves widen the int8
    # rows to bf16 in LDS), two on the per-op GEMV
    m = _reduced(synth.BIG_Q8)
    w = synth.make_weights(m, random_q8_scales=True)
    wl = dataclasses.replace(synth.WORKLOADS["q8_b1"], model=m, prompt=40)
    for batch in (1, 2):
        say(f"[reduced q8 random scales] 4 frames, batch {batch}")
        r = _forced_run(m, w, wl, 4, batch=batch)
        assert r["d"].path == (qt.QT_PATH_FRAME if batch == 1 else qt.QT_PATH_GRAPH)
        _check(r, m, f"reduced_q8_b{batch}")


def test_reduced_bf16_batched_parity():
    # eight streams: the projections run on the batched MFMA GEMM (8- and
    # 16-row predictor steps, 8-row talker steps, 32-row prefill chunks)
    m = _reduced(synth.BIG)
    w = synth.make_weights(m)
    wl = dataclasses.replace(synth.WORKLOADS["q8_b8"], model=m, prompt=40)
    say("[reduced bf16 batched] 4 frames, batch 8")
    _check(_forced_run(m, w, wl, 4, batch=8), m, "reduced_bf16_b8")


def test_reduced_q8_batched_parity():
    m = _reduced(synth.BIG_Q8)
    w = synth.make_weights(m, random_q8_scales=True)
    wl = dataclasses.replace(synth.WORKLOADS["q8_b8"], model=m, prompt=40)
    say("[reduced q8 batched] 3 frames, batch 8")
    _check(_forced_run(m, w, wl, 3, batch=8), m, "reduced_q8_b8")


@pytest.mark.parametrize("flags", [0, qt.QT_F_OPS], ids=["frame", "ops"])
def test_reduced_q4_parity(flags):
    # 4-bit blocks: one stream on the persistent kernel (4-bit rows widened
    # in LDS) or, with the per-op flag, on the GEMV; two streams on the GEMV;
    # a 358-row prompt's prefill chunks (128, 128, 102 rows) on the MFMA GEMM
    m = _reduced(synth.BIG_Q4)
    w = synth.make_weights(m, random_q8_scales=True)
    wl = dataclasses.replace(synth.WORKLOADS["q4_b1"], model=m, prompt=358)
    for batch in (1, 2):
        say(f"[reduced q4 random scales] flags {flags}, prompt 358, 4 frames, batch {batch}")
        r = _forced_run(m, w, wl, 4, batch=batch, flags=flags)
        assert r["d"].path == (qt.QT_PATH_FRAME if batch == 1 and not flags else qt.QT_PATH_GRAPH)
        _check(r, m, f"reduced_q4_b{batch}")


def test_reduced_q4_batched_parity():
    m = _reduced(synth.BIG_Q4)
    w = synth.make_weights(m, random_q8_scales=True)
    wl = dataclasses.replace(synth.WORKLOADS["q4_b8"], model=m, prompt=40)
    say("[reduced q4 batched] 3 frames, batch 8")
    _check(_forced_run(m, w, wl, 3, batch=8), m, "reduced_q4_b8")
    say("[reduced q4 batched sampled] 3 frames, batch 8, T = 0.8")
    _check(_forced_run(m, w, wl, 3, batch=8, sampler=(0.8, 7)), m, "reduced_q4_b8_sampled")


@pytest.mark.parametrize("base", [synth.BIG, synth.BIG_Q8, synth.BIG_Q4], ids=["bf16", "q8", "q4"])
def test_gemv_widths_parity(base):
    # hidden 320 and ffn 960 (not multiples of the GEMM's 256-wide K slice):
    # every projection over them runs on the GEMV, the O projection
    # (K = 2,048) on the GEMM, at one and two streams; the persistent kernel
    # does not take 640-byte rows, so the per-op path decodes
    m = dataclasses.replace(base, Lt=2, Lp=1, Vt=4096, P=512, model_id=base.model_id + 30, H=320, F=960)
    w = synth.make_weights(m, random_q8_scales=True)
    wl = dataclasses.replace(synth.WORKLOADS["q8_b1"], model=m, prompt=40)
    for batch in (1, 2):
        say(f"[gemv widths {base.name}] H 320, F 960, prompt 40, 3 frames, batch {batch}")
        r = _forced_run(m, w, wl, 3, batch=batch)
        assert r["d"].path == qt.QT_PATH_GRAPH
        _check(r, m, f"gemv_widths_{base.name}_b{batch}")


@pytest.mark.timeout(900)
def test_full_q4_b1_parity():
    m = synth.BIG_Q4
    wl = synth.WORKLOADS["q4_b1"]
    say("[q4_b1] weights")
    w = synth.make_weights(m)
    say("[q4_b1] prefill 128 + 4 frames")
    r = _forced_run(m, w, wl, 4)
    assert r["d"].path == qt.QT_PATH_FRAME
    _check(r, m, "q4_b1")


@pytest.mark.timeout(900)
def test_full_bf16_b1_parity():
    m = synth.BIG
    wl = synth.WORKLOADS["bf16_b1"]
    say("[bf16_b1] weights")
    w = synth.make_weights(m)
    say("[bf16_b1] prefill 128 + 6 frames")
    _check(_forced_run(m, w, wl, 6), m, "bf16_b1")


@pytest.mark.timeout(900)
def test_full_bf16_b1_sampled_parity():
    m = synth.BIG
    wl = synth.WORKLOADS["bf16_b1"]
    w = synth.make_weights(m)
    say("[bf16_b1 sampled] prefill 128 + 4 frames, T = 0.9")
    r = _forced_run(m, w, wl, 4, sampler=(0.9, 99))
    assert r["d"].path == qt.QT_PATH_FRAME
    _check(r, m, "bf16_b1_sampled")


@pytest.mark.timeout(900)
def test_full_q8_b1_parity():
    m = synth.BIG_Q8
    wl = synth.WORKLOADS["q8_b1"]
    say("[q8_b1] weights")
    w = synth.make_weights(m)
    say("[q8_b1] prefill 128 + 4 frames")
    r = _forced_run(m, w, wl, 4)
    assert r["d"].path == qt.QT_PATH_FRAME
    _check(r, m, "q8_b1")


@pytest.mark.timeout(900)
def test_full_bf16_long_context_parity():
    # the long-context workload as configured: a seeded 2,048-row prompt
    # prefilled through the 28-layer model on the GPU, its state handed to
    # the oracle, then decoding across position 2,048 -- the window grows from
    # 2,048 to 2,304 positions (9 attention tiles) at the first frame; the
    # frame kernel runs 72 attention workgroups with one weight slot
    m = synth.BIG
    wl = synth.WORKLOADS["bf16_long_b1"]
    w = synth.make_weights(m)
    say("[bf16_long] GPU prefill of 2048 rows, oracle from its state, 6 frames")
    r = _prefilled_state_run(m, w, wl, 6, [synth.make_prompt(wl, 0)], [0])
    assert r["d"].path == qt.QT_PATH_FRAME
    assert r["lengths"] == [2048]
    _check(r, m, "bf16_long")


@pytest.mark.timeout(900)
def test_full_bf16_max_context_parity():
    # the ring's last positions: a 4,088-row prompt prefilled on the GPU,
    # decoded to position 4,093 of 4,096; the frame kernel runs 128
    # attention workgroups (16 tiles per head) beside 128 GEMV workgroups
    m = synth.BIG
    wl = synth.WORKLOADS["bf16_long_b1"]
    w = synth.make_weights(m)
    say("[bf16_max_context] GPU prefill of 4088 rows, oracle from its state, 6 frames")
    r = _prefilled_state_run(m, w, wl, 6, [synth.make_prompt(wl, 0, T=4088)], [0])
    assert r["d"].path == qt.QT_PATH_FRAME
    _check(r, m, "bf16_max_context")
    # one more frame than the ring holds is refused before any launch
    d = r["d"]
    d.set_state(0, *r["pstate"][0])
    with pytest.raises(qt.QtError) as e:
        d.decode(9, r["ov"][:1].repeat(9, axis=0))
    assert e.value.code == qt.QT_E_CONTEXT_FULL
    d.close()


@pytest.mark.timeout(900)
def test_full_bf16_b32_parity():
    # the multi-stream workload as the bench runs it: 32 streams whose seeded
    # prompts have the ragged context lengths (uniform in [64, 2048]), each
    # prefilled through the model on the GPU; six streams' states go to the
    # oracle and every frame of those streams is compared (teacher-forced,
    # one frame per call), then the free run
    m = synth.BIG
    wl = synth.WORKLOADS["bf16_b32"]
    w = synth.make_weights(m)
    lens = synth.make_context_lengths(wl)
    prompts = [synth.make_prompt(wl, b, T=int(lens[b])) for b in range(wl.batch)]
    sample = [0, 5, 9, 22, 27, 31]
    say("[bf16_b32] contexts", lens.tolist(), "checking streams", sample)
    r = _prefilled_state_run(m, w, wl, 4, prompts, sample)
    assert r["d"].path == qt.QT_PATH_GRAPH
    _check(r, m, "bf16_b32")
    r["d"].close()


@pytest.mark.timeout(900)
def test_full_bf16_b32_replay_of_four_frames_equals_one_and_adaptive_k():
    # four frames per graph replay (as the bench times the workload) decode
    # the same codes and last-frame logits as one frame per replay, bit for bit
    m = synth.BIG
    wl = synth.WORKLOADS["bf16_b32"]
    w = synth.make_weights(m)
    lens = synth.make_context_lengths(wl)
    prompts = [synth.make_prompt(wl, b, T=int(lens[b])) for b in range(wl.batch)]
    ov = synth.make_overlays(wl, 8)
    dw = qt.DeviceWeights(m, w, "cuda")
    out = {}
    for K, calls in ((1, [8]), (4, [8]), (4, [1, 2, 5])):
        # (K = 4 in calls of 1, 2 and 5 frames: adaptive K replays the 1-frame
        # graph for the frames past each call's last whole block)
        say(f"[bf16_b32 replay] K = {K}: 32 prefills, calls of {calls} frames")
        d = qt.Decoder(m, dw, wl.batch, frames_per_replay=K, flags=qt.QT_F_DUMP)
        for b, (c, t) in enumerate(prompts):
            d.prefill(b, c, t)
        codes, f0 = [], 0
        for n in calls:
            codes.append(d.decode(n, ov[f0:f0 + n]))
            f0 += n
        out[(K, len(calls))] = (np.concatenate(codes), d.dump(qt.QT_DUMP_TALKER_LOGITS),
                                d.dump(qt.QT_DUMP_PRED_LOGITS))
        d.close()
    ref = out[(1, 1)]
    for key in ((4, 1), (4, 3)):
        assert np.array_equal(ref[0], out[key][0])
        assert np.array_equal(ref[1].view(np.uint32), out[key][1].view(np.uint32))
        assert np.array_equal(ref[2].view(np.uint32), out[key][2].view(np.uint32))


@pytest.mark.timeout(900)
def test_reduced_long_prefill_parity():
    # the 2,048-row prefill itself against the oracle's own prefill, on the
    # full widths with two talker layers: 4 prompt chunks of 512 rows, causal
    # tiles across 8 attention tiles; last-row logits, bridge, code 0 and
    # every cached K/V row
    m = dataclasses.replace(_reduced(synth.BIG), P=4096)
    w = synth.make_weights(m)
    wl = dataclasses.replace(synth.WORKLOADS["bf16_long_b1"], model=m)
    codes, text = synth.make_prompt(wl, 0)
    say("[reduced long prefill] oracle prefill of 2048 rows (2 layers)")
    o = Oracle(m, w, 1, pcap=2048 + 1)
    pre = o.prefill(0, codes, text, dump=True)
    opos, oc0, obr = o.get_state(0)
    d = qt.Decoder(m, w, 1, flags=qt.QT_F_DUMP)
    d.prefill(0, codes, text)
    pos, c0, br = d.get_state(0)
    gl = d.dump(qt.QT_DUMP_TALKER_LOGITS)[0]
    kv, _ = _read_state(d, 0, 2048)
    worst = {"logits": rel_l2(gl, pre["logits"]), "bridge": rel_l2(br, obr)}
    for layer in range(m.Lt):
        ok, ov_ = o.get_cache(0, layer, 0, 2048)
        worst[f"k{layer}"] = rel_l2(kv[layer, 0], ok)
        worst[f"v{layer}"] = rel_l2(kv[layer, 1], ov_)
    say("[reduced long prefill] rel-L2:", {k: f"{v:.2e}" for k, v in worst.items()})
    assert pos == opos == 2048
    for k, v in worst.items():
        assert v <= 1e-2, f"reduced long prefill: {k} rel-L2 {v}"
    if c0 != oc0:  # only at a near tie of the last row's logits
        assert margin(pre["logits"]) <= 4 * float(np.max(np.abs(gl - pre["logits"])))


@pytest.mark.parametrize("base", [synth.BIG, synth.BIG_Q8], ids=["bf16", "q8"])
def test_ffn_width_not_multiple_of_256_parity(base):
    # hidden 1,024 but FFN 2,080: the model takes the GEMV for every
    # projection (the GEMM's row norms need sums of squares that only its own
    # residual epilogue writes), at one and two streams on the per-op path
    m = dataclasses.replace(base, Lt=2, Lp=1, Vt=4096, P=512, model_id=base.model_id + 40, F=2080)
    w = synth.make_weights(m, random_q8_scales=True)
    wl = dataclasses.replace(synth.WORKLOADS["q8_b1"], model=m, prompt=40)
    for batch in (1, 2):
        say(f"[ffn 2080 {base.name}] prompt 40, 3 frames, batch {batch}")
        r = _forced_run(m, w, wl, 3, batch=batch)
        assert r["d"].path == qt.QT_PATH_GRAPH
        _check(r, m, f"ffn2080_{base.name}_b{batch}")


def _tied_heads(m, w, wl, prompt):
    """Weights whose heads tie exactly at the decisions of the oracle's first
    frame: row 0 of each head becomes a copy of the row the oracle picked
    there (when that row is not 0).  Decoded with the first frame's codes fed
    back (teacher forcing), every head then sees the inputs it saw before, so
    each of those logits is the maximum twice -- at 0 and at a row that the
    persistent kernel gives another workgroup -- and the lowest index must
    win.  Returns the weights, the first frame's codes (code 0 from the
    prefill) and the indices of the tied decisions."""
    o = Oracle(m, w, 1)
    o.prefill(0, *prompt)
    ov = synth.make_overlays(wl, 1, 1)
    codes = o.decode(1, ov)["codes"]
    w2 = dict(w)
    w2["t_head"] = w["t_head"].copy()
    w2["p_heads"] = [h.copy() for h in w["p_heads"]]
    tied = []
    for j in range(m.G):
        c = int(codes[0, 0, j])
        if c:
            tab = w2["t_head"] if j == 0 else w2["p_heads"][j - 1]
            tab[0] = (w["t_head"] if j == 0 else w["p_heads"][j - 1])[c]
            tied.append(j)
    return w2, codes, ov, tied


@pytest.mark.parametrize("sampler", [None, (1.0, 5, 1)], ids=["greedy", "top1"])
@pytest.mark.parametrize("flags", [0, qt.QT_F_OPS], ids=["frame", "ops"])
def test_exact_ties_pick_the_lowest_index(flags, sampler):
    # greedy, and top-k sampling with k = 1: of two equal largest logits only
    # the lower index is a member, whatever the noise
    m = synth.TINY
    wl = synth.WORKLOADS["tiny_f32_b1"]
    w = synth.make_weights(m)
    prompt = synth.make_prompt(wl, 0)
    w2, codes, ov, tied = _tied_heads(m, w, wl, prompt)
    assert len(tied) >= 8
    o = Oracle(m, w2, 1)
    d = qt.Decoder(m, w2, 1, flags=flags)
    if sampler:
        o.set_sampler(*sampler)
        d.set_sampler(sampler[0], sampler[1], top_k=sampler[2])
    o.prefill(0, *prompt)
    oc = o.decode(1, ov, forced=codes)["codes"]
    assert d.path == (qt.QT_PATH_GRAPH if flags else qt.QT_PATH_FRAME)
    d.prefill(0, *prompt)
    gc = d.decode(1, ov, forced=codes)
    say(f"[ties {flags} {sampler}] tied decisions {tied}; codes", gc[0, 0].tolist())
    assert all(oc[0, 0, j] == 0 for j in tied)  # the oracle's rule: lowest index
    assert np.array_equal(gc, oc)                # F32: every decision equal
    d.close()


def test_exact_ties_bf16_full_width():
    # the same on the 1,024-wide bf16 model: 2,048-way heads spread over the
    # persistent kernel's workgroups (one stream), and the MFMA GEMM + argmax
    # kernel (two streams); the tied decisions must be 0 exactly, the others
    # may differ from the oracle only at a near tie
    m = _reduced(synth.BIG)
    wl = dataclasses.replace(synth.WORKLOADS["bf16_b1"], model=m, prompt=40)
    w = synth.make_weights(m)
    prompt = synth.make_prompt(wl, 0)
    w2, codes, ov, tied = _tied_heads(m, w, wl, prompt)
    assert len(tied) >= 8
    o = Oracle(m, w2, 1)
    o.prefill(0, *prompt)
    oout = o.decode(1, ov, forced=codes, dump=True)
    for batch in (1, 2):
        d = qt.Decoder(m, w2, batch, flags=qt.QT_F_DUMP)
        for b in range(batch):
            d.prefill(b, *prompt)
        gc = d.decode(1, np.repeat(ov, batch, axis=1), forced=np.repeat(codes, batch, axis=1))
        gl = d.dump(qt.QT_DUMP_PRED_LOGITS)
        say(f"[ties bf16 b{batch}] tied {tied}; codes", gc[0, 0].tolist())
        for b in range(batch):
            assert all(gc[0, b, j] == 0 for j in tied), "a tie went to a higher index"
            for j in range(1, m.G):
                if gc[0, b, j] != oout["codes"][0, 0, j]:
                    rl = oout["pred_logits"][0, 0, j - 1]
                    err = float(np.max(np.abs(gl[j - 1, b] - rl)))
                    assert margin(rl) <= 4 * err, f"code {j} differs away from a near tie"
        d.close()


# ----------------------------------------------------------------- paged ring


def _paged_vs_dense(m, w, prompts, frames, pool_rows, order, wl, sampler=None):
    """A dense and a paged context decode the same prompts: the outputs must be
    bitwise equal (the paged ring only moves rows).  Slots are prefilled in
    `order`, so each slot's rows are scattered through the pool."""
    B = len(prompts)
    dd = qt.Decoder(m, w, B, flags=qt.QT_F_DUMP)
    dp = qt.Decoder(m, dd.dw, B, flags=qt.QT_F_DUMP, pool_rows=pool_rows)
    assert dd.path == dp.path == qt.QT_PATH_GRAPH
    for d in (dd, dp):
        if sampler:
            d.set_sampler(*sampler)
        for b in order:
            d.prefill(b, *prompts[b])
    return dd, dp


def _same_outputs(dd, dp, n, ov):
    cd = dd.decode(n, ov)
    cp = dp.decode(n, ov)
    assert np.array_equal(cd, cp)
    for kind in (qt.QT_DUMP_TALKER_LOGITS, qt.QT_DUMP_PRED_LOGITS, qt.QT_DUMP_BRIDGE):
        assert np.array_equal(dd.dump(kind).view(np.uint32), dp.dump(kind).view(np.uint32))
    return cd


@pytest.mark.parametrize("sampler", [None, (0.9, 11, 50)], ids=["greedy", "top50"])
def test_paged_ring_equals_dense(sampler):
    # four ragged streams (40 to 460 rows: one to two 256-position tiles),
    # prefilled out of order, decoded in calls of 8, 4 and 4 frames; then one
    # slot re-prefilled with a shorter prompt (its rows go back to the pool
    # and are reused) and decoded again; the pool holds exactly what the
    # streams need, so one more frame is refused
    m = _reduced(synth.BIG)
    w = synth.make_weights(m)
    wl = dataclasses.replace(synth.WORKLOADS["q8_b8"], model=m, prompt=40)
    lens = [40, 300, 130, 460]
    prompts = [synth.make_prompt(wl, b, T=t) for b, t in enumerate(lens)]
    short = synth.make_prompt(wl, 7, T=70)
    n = 16
    pool = sum(lens) + len(lens) * n
    say(f"[paged {sampler}] prompts {lens}, pool {pool} rows")
    dd, dp = _paged_vs_dense(m, w, prompts, n, pool, [2, 0, 3, 1], wl, sampler)
    ov = synth.make_overlays(wl, n, len(lens))
    _same_outputs(dd, dp, 8, ov[:8])
    _same_outputs(dd, dp, 4, ov[8:12])
    for d in (dd, dp):  # slot 3 restarts: 460 rows back to the pool, 70 taken
        d.prefill(3, *short)
    _same_outputs(dd, dp, 4, ov[12:16])
    # 4 x 16 frames + the prompts fill the pool but for what slot 3 gave back
    st = [dp.get_state(b) for b in range(len(lens))]
    free = pool - (lens[0] + lens[1] + lens[2] + 3 * n) - (70 + 4)
    assert free == 460 + 12 - 70
    # frames until the pool runs out: every slot needs a row per frame
    k = free // len(lens)
    _same_outputs(dd, dp, k, np.repeat(ov[:1], k, axis=0))
    with pytest.raises(qt.QtError) as e:
        dp.decode(len(lens), np.repeat(ov[:1], len(lens), axis=0))
    assert e.value.code == qt.QT_E_CONTEXT_FULL
    # refused before any launch: the state did not move
    assert [dp.get_state(b)[0] for b in range(len(lens))] == [s[0] + k for s in st]
    # a restored position needs the slot's rows to exist
    with pytest.raises(qt.QtError) as e:
        dp.set_state(0, st[0][0] + k + 1, *st[0][1:])
    assert e.value.code == qt.QT_E_STATE
    dd.close()
    dp.close()


def test_paged_ring_oracle_parity():
    # the paged ring against the oracle, at the 1e-2 gates: three ragged
    # streams (60, 270, 150 rows) prefilled out of order, so each stream's
    # rows are scattered through the pool (its exact size)
    m = _reduced(synth.BIG)
    w = synth.make_weights(m)
    wl = dataclasses.replace(synth.WORKLOADS["q8_b8"], model=m, prompt=40)
    lens = [60, 270, 150]
    prompts = [synth.make_prompt(wl, b, T=t) for b, t in enumerate(lens)]
    say(f"[paged oracle] prompts {lens}, 4 frames")
    r = _forced_run(m, w, wl, 4, batch=3, prompts=prompts, pool_rows=sum(lens) + 3 * 4, order=[1, 2, 0])
    assert r["d"].path == qt.QT_PATH_GRAPH and r["d"].pool_rows
    _check(r, m, "paged_b3")


# ----------------------------------------------------------------- prompts of several streams in one call


def _ring_bytes(d, b, T):
    return d.talker_ring()[b, :, :, :, :T, :].cpu().numpy().copy().view(np.uint8)


@pytest.mark.parametrize("base,sampler", [("tiny", None), ("reduced_bf16", None), ("reduced_bf16", (0.8, 5, 40))],
                         ids=["tiny", "reduced_bf16", "reduced_bf16_top40"])
def test_prefill_rows_equals_per_stream(base, sampler, tiny):
    # several streams' prompts in one qt_prefill_rows call (chunks of the same
    # positions of every stream still going, ragged prompts padded and ending
    # in different chunks, the chunk size growing as streams finish) leave
    # every slot as its own qt_prefill does, bit for bit: ring rows, bridge,
    # c0, position and the head's logits; the graph replays equal the eager
    # launches of the same chunks; a paged ring decodes the same codes
    if base == "tiny":
        m, w, wl = tiny[0], tiny[3]["d"].dw, tiny[2]
        lens, slots = [5, 37, 100, 16], [3, 0, 2, 1]
    else:
        m = _reduced(synth.BIG)
        w = synth.make_weights(m)
        wl = dataclasses.replace(synth.WORKLOADS["q8_b8"], model=m, prompt=40)
        lens, slots = [300, 40, 129], [1, 2, 0]
    B = len(lens)
    wlb = dataclasses.replace(wl, batch=B)
    prompts = [synth.make_prompt(wlb, 20 + i, T=t) for i, t in enumerate(lens)]
    ov = synth.make_overlays(wlb, 3)
    say(f"[prefill rows {base}] prompts {lens} into slots {slots}, sampler {sampler}")
    d_each = qt.Decoder(m, w, B, flags=qt.QT_F_DUMP | qt.QT_F_OPS)
    if sampler:  # the first codes are drawn inside the prefill call
        d_each.set_sampler(*sampler)
    for b, (c, t) in zip(slots, prompts):
        d_each.prefill(b, c, t)
    lg_each = d_each.dump(qt.QT_DUMP_TALKER_LOGITS)
    outs = {}
    for name, flags in (("graph", qt.QT_F_DUMP | qt.QT_F_OPS), ("eager", qt.QT_F_DUMP | qt.QT_F_EAGER)):
        d = qt.Decoder(m, w, B, flags=flags)
        if sampler:
            d.set_sampler(*sampler)
        d.prefill_rows(slots, [c for c, _ in prompts], [t for _, t in prompts])
        for b, T in zip(slots, lens):
            se, sr = d_each.get_state(b), d.get_state(b)
            assert se[:2] == sr[:2], (name, b)
            assert np.array_equal(se[2].view(np.uint32), sr[2].view(np.uint32)), (name, b)
            assert np.array_equal(_ring_bytes(d_each, b, T), _ring_bytes(d, b, T)), (name, b)
        assert np.array_equal(d.dump(qt.QT_DUMP_TALKER_LOGITS).view(np.uint32), lg_each.view(np.uint32)), name
        outs[name] = d.decode(3, ov)
        d.close()
    ref = d_each.decode(3, ov)
    assert np.array_equal(outs["graph"], ref) and np.array_equal(outs["eager"], ref)
    dp = qt.Decoder(m, w, B, flags=qt.QT_F_OPS, pool_rows=sum(lens) + 3 * B)
    if sampler:
        dp.set_sampler(*sampler)
    dp.prefill_rows(slots, [c for c, _ in prompts], [t for _, t in prompts])
    assert np.array_equal(dp.decode(3, ov), ref)
    dp.close()
    d_each.close()
    if base == "tiny":  # F32: the oracle's codes exactly
        o = Oracle(m, tiny[1], B)
        for b, (c, t) in zip(slots, prompts):
            o.prefill(b, c, t)
        assert np.array_equal(o.decode(3, ov)["codes"], ref)


def test_prefill_rows_refusals_leave_state(tiny):
    m, w, wl = tiny[0], tiny[3]["d"].dw, tiny[2]
    wl2 = dataclasses.replace(wl, batch=2)
    prompts = [synth.make_prompt(wl2, b, T=12 + b) for b in range(2)]
    ov = synth.make_overlays(wl2, 2)
    d = qt.Decoder(m, w, 2, flags=qt.QT_F_OPS)
    d.prefill_rows([0, 1], [c for c, _ in prompts], [t for _, t in prompts])
    st = [d.get_state(b) for b in range(2)]
    c, t = prompts[0]
    cases = [([0, 0], [c, c], [t, t], qt.QT_E_ARG),            # a slot twice
             ([0, 2], [c, c], [t, t], qt.QT_E_ARG),            # a slot outside [0, B)
             ([0, 1, 0, 1, 0], [c] * 5, [t] * 5, qt.QT_E_ARG),  # more than 4 streams
             ([1], [np.zeros((m.P + 1, m.G), np.int32)], [np.zeros(m.P + 1, np.int32)], qt.QT_E_CONTEXT_FULL),
             ([1], [c], [np.full(len(t), m.Vt, np.int32)], qt.QT_E_RANGE)]
    for sl, cs, ts, code in cases:
        with pytest.raises(qt.QtError) as e:
            d.prefill_rows(sl, cs, ts)
        assert e.value.code == code, (sl, e.value.code)
    assert qt.lib.qt_prefill_rows(d.ctx, 0, None, None, None, None) == qt.QT_E_ARG
    assert [d.get_state(b)[:2] for b in range(2)] == [s[:2] for s in st]
    ref = qt.Decoder(m, w, 2, flags=qt.QT_F_OPS)
    for b, (c, t) in enumerate(prompts):
        ref.prefill(b, c, t)
    assert np.array_equal(d.decode(2, ov), ref.decode(2, ov))
    d.close()
    ref.close()
