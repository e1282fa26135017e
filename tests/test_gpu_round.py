"""End-to-end verify rounds on the GPU against the oracle.

* single-linear workload: 2048x2048 8-bit projection and 8192x2048 head over
  6 rows, greedy accept of 5 drafts whose first 3 equal the oracle's tokens;
* batched verify: 4 requests x 6 rows = 24 rows through the 151936x4096 head
  in one launch, per-request greedy accept with match rates 0.3/0.5/0.7/0.9.
"""
import numpy as np
import pytest

import oracle
from speculative_decoding_verify_dspk_amd import inputs
from gpuutil import assert_argmax_parity, assert_rows_close, oracle_logits_chunked, run_lmhead, run_qgemm
from test_gpu_accept import gpu_greedy

pytestmark = pytest.mark.gpu


def test_single_linear_round():
    m, k, n, v = 6, 2048, 2048, 8192
    w = inputs.make_qweight(n, k, 8, "round1", "linear")
    x = inputs.make_activations(m, k, "round1", "x")
    y = run_qgemm(w, x, m)
    assert_rows_close(y, oracle.qlinear(x, w.codes, w.scales, w.biases, 8, n, k), what="linear")
    head = inputs.make_qweight(v, k, 8, "round1", "head")
    h = inputs.make_activations(m, k, "round1", "h")
    ids, z = run_lmhead(head, h, m)
    zref = oracle.qlinear(h, head.codes, head.scales, head.biases, 8, v, k)
    t_ref, near = assert_argmax_parity(ids, zref, what="head")
    d = inputs.drafts_first_equal(t_ref, 3, v, "round1", "drafts")
    al, com = gpu_greedy(ids[None, :].astype(np.int32), d[None, :])
    ral, rcom = oracle.accept_greedy(t_ref[None, :], d[None, :])
    if not near.any():
        assert al[0] == ral[0] and np.array_equal(com, rcom)
    assert al[0] >= 4          # three drafts equal the target's tokens, plus the target's own


def test_batched_four_requests():
    b, rows, hid, v = 4, 6, 4096, 151936
    m = b * rows
    head = inputs.make_qweight(v, hid, 8, "round5", "head")
    h = inputs.make_activations(m, hid, "round5", "h")
    ids, z = run_lmhead(head, h, m, want_logits=True)
    zref = oracle_logits_chunked(head, h)
    assert_rows_close(z, zref, what="batched logits")
    t_ref, near = assert_argmax_parity(ids, zref, what="batched head")
    t = t_ref.reshape(b, rows)
    d = inputs.drafts_match_rate(t, np.array([0.3, 0.5, 0.7, 0.9]), v, "round5")
    al, com = gpu_greedy(ids.reshape(b, rows).astype(np.int32), d)
    ral, rcom = oracle.accept_greedy(t, d)
    ok_req = ~near.reshape(b, rows).any(axis=1)
    assert np.array_equal(al[ok_req], ral[ok_req]) and np.array_equal(com[ok_req], rcom[ok_req])


@pytest.mark.parametrize("b,rows", [(1, 1), (1, 6), (1, 17), (4, 6), (2, 16), (32, 1)])
def test_fused_head_accept_equals_separate_calls(b, rows):
    """dspk_lmhead_argmax_accept_greedy gives exactly the ids of
    dspk_lmhead_argmax and the acceptance of dspk_accept_greedy on them, and
    the acceptance matches the oracle's greedy rule on the oracle's ids."""
    import torch
    from speculative_decoding_verify_dspk_amd import binding
    from gpuutil import dev_act
    m, k, v = b * rows, 2048, 8192
    head = inputs.make_qweight(v, k, 8, "fused", b, rows)
    h_bits = inputs.make_activations(m, k, "fused", "h", b, rows)
    dw = binding.DeviceQWeight.upload(head)
    h = dev_act(h_bits)
    ids_sep, _ = run_lmhead(head, h_bits, m, want_logits=False, dw=dw)
    zref = oracle.qlinear(h_bits, head.codes, head.scales, head.biases, 8, v, k)
    t_ref, near = assert_argmax_parity(ids_sep, zref, what="fused head")
    t = t_ref.reshape(b, rows)
    d = inputs.drafts_match_rate(t, np.full(b, 0.7), v, "fused", b, rows) if rows > 1 else None
    al_sep, com_sep = gpu_greedy(ids_sep.reshape(b, rows).astype(np.int32), d)
    ws = binding.alloc_workspace(binding.lmhead_workspace_bytes(v, m))
    am = torch.full((m,), -7, dtype=torch.int32, device="cuda")
    al = torch.full((b,), -7, dtype=torch.int32, device="cuda")
    com = torch.full((b, rows), -7, dtype=torch.int32, device="cuda")
    dd = torch.from_numpy(np.ascontiguousarray(d, dtype=np.int32)).cuda() if d is not None else None
    for _ in range(2):      # the workspace is left zeroed: a second call gives the same results
        binding.lmhead_argmax_accept_greedy(dw, h, b, rows, am, dd, al, com, workspace=ws)
        torch.cuda.synchronize()
        assert np.array_equal(am.cpu().numpy(), ids_sep)
        assert np.array_equal(al.cpu().numpy(), al_sep) and np.array_equal(com.cpu().numpy(), com_sep)
    if d is not None:
        ral, rcom = oracle.accept_greedy(t, d)
        ok = ~near.reshape(b, rows).any(axis=1)
        assert np.array_equal(al_sep[ok], ral[ok]) and np.array_equal(com_sep[ok], rcom[ok])
    else:
        assert np.all(al_sep == 1) and np.array_equal(com_sep[:, 0], ids_sep)


def test_results_written_to_pinned_host_memory():
    """The acceptance outputs may be pinned host memory mapped for the device:
    the fused greedy head and the sampling accept write there exactly what
    they write to device memory, with no copy launch."""
    import torch
    from speculative_decoding_verify_dspk_amd import binding
    from gpuutil import dev_act
    b, rows, k, v = 2, 6, 2048, 8192
    m = b * rows
    head = inputs.make_qweight(v, k, 8, "pinned", "head")
    h_bits = inputs.make_activations(m, k, "pinned", "h")
    dw = binding.DeviceQWeight.upload(head)
    h = dev_act(h_bits)
    ids, z = run_lmhead(head, h_bits, m, want_logits=True, dw=dw)
    d = inputs.drafts_match_rate(ids.reshape(b, rows), np.full(b, 0.7), v, "pinned", "d")
    dd = torch.from_numpy(np.ascontiguousarray(d, dtype=np.int32)).cuda()
    ws = binding.alloc_workspace(binding.lmhead_workspace_bytes(v, m))
    am = torch.empty((m,), dtype=torch.int32, device="cuda")
    q, ds = inputs.draft_distribution(z[:rows], 1.0, 0.5, "pinned", "q")
    u = inputs.make_uniforms(rows, "pinned", "u")
    zt = torch.from_numpy(np.ascontiguousarray(z[:rows])).cuda()
    qt = torch.from_numpy(np.ascontiguousarray(q)).cuda()
    dst = torch.from_numpy(ds).cuda()
    ut = torch.from_numpy(u).cuda()
    sws = binding.alloc_workspace(binding.sample_workspace_bytes(v, rows))
    got = {}
    for where in ("device", "pinned"):
        kw = dict(device="cuda") if where == "device" else dict(pin_memory=True)
        al = torch.full((b,), -7, dtype=torch.int32, **kw)
        com = torch.full((b, rows), -7, dtype=torch.int32, **kw)
        binding.lmhead_argmax_accept_greedy(dw, h, b, rows, am, dd, al, com, workspace=ws)
        sal = torch.full((1,), -7, dtype=torch.int32, **kw)
        scom = torch.full((rows,), -7, dtype=torch.int32, **kw)
        binding.accept_sample(zt, qt, dst, ut, rows, v, 1.0, sal, scom, sws)
        torch.cuda.synchronize()
        got[where] = [x.cpu().numpy().copy() for x in (al, com, sal, scom)]
    for a, c in zip(got["device"], got["pinned"]):
        assert np.array_equal(a, c)
    assert np.all(got["pinned"][0] >= 1) and 1 <= got["pinned"][2][0] <= rows


def test_graph_replays_match_eager_round():
    """A round captured into HIP graphs (layers, head, accept) and replayed
    several times, with eager work and synchronisations in between, gives
    the eager round's results bit for bit on every replay (the kernels are
    deterministic and leave their workspaces zeroed for the next call)."""
    import torch
    from speculative_decoding_verify_dspk_amd import binding
    from speculative_decoding_verify_dspk_amd.verify_round import VerifyStack
    m = 8
    st = VerifyStack("qwen3-4b", 1, 8, m)
    st.launch_head(m)
    torch.cuda.synchronize()
    t = st.argmax[:m].cpu().numpy()[None, :]
    d = torch.from_numpy(inputs.drafts_match_rate(t, 0.7, st.vocab, "graph-test")).cuda()
    alen = torch.empty((1,), dtype=torch.int32, device="cuda")
    com = torch.empty((1, m), dtype=torch.int32, device="cuda")

    def outputs():
        return [y.clone() for y in st.y_qkv + [st.y_o] + st.y_gu + [st.y_down]] + \
               [st.argmax.clone(), alen.clone(), com.clone()]

    st.launch_layers(m)
    st.launch_head(m)
    binding.accept_greedy(st.argmax, d, 1, m, alen, com)
    torch.cuda.synchronize()
    ref = outputs()
    graphs = st.capture_round(m, 0, d, alen, com)
    for rep in range(3):
        for y in st.y_qkv + [st.y_o] + st.y_gu + [st.y_down]:
            y.fill_(float("nan"))
        st.argmax.fill_(-5)
        alen.fill_(-5)
        com.fill_(-5)
        torch.cuda.synchronize()
        for g in graphs:
            g.replay()
        torch.cuda.synchronize()
        got = outputs()
        for a, b in zip(ref, got):
            assert torch.equal(a, b), f"replay {rep} differs from the eager round"
        # eager work between replays: an unrelated eager call on the same workspaces
        st.launch_head(m)
        torch.cuda.synchronize()


def test_measured_curve_drives_the_cap_policy(tmp_path):
    """The verify-cost curve measured on this GPU (cached on disk) feeds the
    cap controller: costs are positive, and a perfect drafter is never parked."""
    from speculative_decoding_verify_dspk_amd import binding, calibration
    from speculative_decoding_verify_dspk_amd.verify_round import VerifyStack
    st = VerifyStack("qwen3-4b", 1, 8, 8)
    key = calibration.cache_key("qwen3-4b", 8)
    curve = calibration.load_or_measure(str(tmp_path / "c.json"), key,
                                        lambda: calibration.measure_verify_curve(st, range(1, 9), reps=3))
    assert len(curve) == 8 and all(t > 0 for t in curve)
    cap, rate = binding.choose_cap(curve, None, 1.0)
    assert cap >= 1 and rate > 1.0 / curve[0]
    assert binding.choose_cap(curve, None, 0.0)[0] == 0
    # the library's choice on the curve this device measured is the oracle's
    drafter = [0.0] + [2.0 + 0.5 * i for i in range(1, len(curve))]
    for a in np.linspace(0.0, 1.0, 21):
        for dr in (None, drafter):
            got = binding.choose_cap(curve, dr, float(a))
            want = oracle.choose_cap(curve, dr, float(a))
            assert got[0] == want[0], (a, dr is not None, got, want, curve)
            assert abs(got[1] - want[1]) <= 1e-12 * max(1.0, abs(want[1]))


def _sampled_columns(g, n, count=96):
    return np.unique(np.concatenate([[0, 1, 63, 64, n - 1], g.choice(n, count, replace=False)]))


def test_dense27b_sampled_round_on_one_workspace():
    """A 27B-shaped round at M = 17 (anchor + 16 drafts): two layers' projections
    (q/k/v grouped, o, gate/up grouped, down; independent N(0, 1) inputs per
    launch), the 151936 x 5120 head with logits, then speculative sampling at
    T = 1 against drafts drawn from q = softmax(z + N(0, 0.5)) built from the
    oracle's logits.  Every projection and head launch shares ONE workspace
    (different shapes, grouped and single, head last), as the workspace
    contract allows.  Projections: sampled columns against the oracle; head:
    full logits and ids; acceptance: equal to the oracle's on the oracle's
    logits, except decisions within the band the logit difference opens."""
    import torch
    from speculative_decoding_verify_dspk_amd import binding
    from gpuutil import dev_act, dev_f32, dev_i32, oracle_columns
    from test_gpu_accept import exempt
    m, T = 17, 1.0
    s = inputs.LAYER_SHAPES["dense-27b"]
    H, Q, KV, F, V = s["hidden"], s["q"], s["kv"], s["inter"], s["vocab"]
    need = max(binding.qgemm_workspace_bytes(Q, H, m) * 3, binding.qgemm_workspace_bytes(F, H, m) * 2,
               binding.lmhead_workspace_bytes(V, m))
    ws = binding.alloc_workspace(need)
    g = np.random.default_rng(27)
    f32 = dict(dtype=torch.float32, device="cuda")
    for layer in range(2):
        mk = lambda n, k, name: inputs.make_qweight(n, k, 8, "c4round", layer, name)   # noqa: E731
        groups = [([mk(Q, H, "q"), mk(KV, H, "k"), mk(KV, H, "v")], H, "attn_in"),
                  ([mk(H, Q, "o")], Q, "o_in"),
                  ([mk(F, H, "gate"), mk(F, H, "up")], H, "mlp_in"),
                  ([mk(H, F, "down")], F, "down_in")]
        for ws_, k, src in groups:
            print(f"27B layer {layer} {src}: {[w.n for w in ws_]} x {k}", flush=True)
            x = inputs.make_activations(m, k, "c4round", layer, src)
            dws = [binding.DeviceQWeight.upload(w) for w in ws_]
            ys = [torch.full((m, w.n), float("nan"), **f32) for w in ws_]
            if len(ws_) == 1:
                binding.qgemm_verify(dws[0], dev_act(x), m, ys[0], ws)
            else:
                binding.qgemm_verify_grouped(dws, dev_act(x), m, ys, ws)
            torch.cuda.synchronize()
            for w, y in zip(ws_, ys):
                got = y.cpu().numpy()
                assert np.isfinite(got).all()
                cols = _sampled_columns(g, w.n)
                ref = oracle_columns(w, x, cols)
                assert_rows_close(got[:, cols], ref, what=f"layer {layer} n={w.n}")
            del dws
    head = inputs.make_qweight(V, H, 8, "c4round", "lm_head")
    h = inputs.make_activations(m, H, "c4round", "final_h")
    dh = binding.DeviceQWeight.upload(head)
    am = torch.full((m,), -7, dtype=torch.int32, device="cuda")
    z = torch.empty((m, V), **f32)
    binding.lmhead_argmax(dh, dev_act(h), m, am, z, ws)
    torch.cuda.synchronize()
    assert int(ws[:512].count_nonzero()) == 0, "head words not returned to zero"
    print("oracle logits of the 27B-shaped head", flush=True)
    zref = oracle_logits_chunked(head, h)
    zg = z.cpu().numpy()
    assert_rows_close(zg, zref, what="27B head logits")
    assert_argmax_parity(am.cpu().numpy(), zref, what="27B head")
    q, d = inputs.draft_distribution(zref, T, 0.5, "c4round", "drafter")
    u = inputs.make_uniforms(m, "c4round", "uniforms")
    al = torch.full((1,), -9, dtype=torch.int32, device="cuda")
    com = torch.full((m,), -9, dtype=torch.int32, device="cuda")
    sws = binding.alloc_workspace(binding.sample_workspace_bytes(V, m))
    binding.accept_sample(z, dev_f32(q), dev_i32(d), dev_f32(u), m, V, T, al, com, sws)
    torch.cuda.synchronize()
    ral, rcom = oracle.accept_sample(zref, q, d, u, T)
    got_al, got_com = int(al.cpu()[0]), com.cpu().numpy()
    dz = float(np.abs(zg - zref).max())
    print(f"27B round: accepted {got_al} (oracle {ral}); max |dz| = {dz:.2e}")
    if got_al != ral or not np.array_equal(got_com, rcom):
        band = max(1e-5, 4.0 * dz / T)
        assert exempt(zref, q.astype(np.float64), d, u.astype(np.float64), T, band=band), \
            f"gpu ({got_al}, {got_com}) != oracle ({ral}, {rcom})"
        print(f"27B round: exempt within band {band:.1e}")


def test_projections_chain_through_bf16_rows():
    """The boundary chains: a projection's bf16 output rows (row-major
    [m][n]) are the next projection's input as they are -- Qwen3-4B q then o
    shapes, no relayout between the two calls."""
    import torch
    from speculative_decoding_verify_dspk_amd import binding
    from gpuutil import dev_act
    m, H, Q = 8, 2560, 4096
    w1 = inputs.make_qweight(Q, H, 8, "chain", "q")
    w2 = inputs.make_qweight(H, Q, 8, "chain", "o")
    x = inputs.make_activations(m, H, "chain", "x")
    d1, d2 = binding.DeviceQWeight.upload(w1), binding.DeviceQWeight.upload(w2)
    ws = binding.alloc_workspace(binding.qgemm_workspace_bytes(Q, H, m))
    y1 = torch.empty((m, Q), dtype=torch.int16, device="cuda")        # bf16 bit patterns
    y2 = torch.empty((m, H), dtype=torch.float32, device="cuda")
    binding.qgemm_verify(d1, dev_act(x), m, y1, ws)
    binding.qgemm_verify(d2, y1, m, y2, ws)                            # y1 is x of the second call
    torch.cuda.synchronize()
    # the oracle's chain: its own fp64 first stage rounded to bf16 rows, then the second stage
    r1 = oracle.qlinear(x, w1.codes, w1.scales, w1.biases, 8, Q, H)
    r1_bits = inputs.f32_to_bf16_bits(r1.astype(np.float32))
    g1 = y1.cpu().numpy().view(np.uint16)
    diff = np.abs(inputs.bf16_bits_to_f32(g1).astype(np.float64) - inputs.bf16_bits_to_f32(r1_bits))
    ulp = np.abs(inputs.bf16_bits_to_f32(r1_bits)).astype(np.float64) * 2.0 ** -7
    assert (diff <= ulp + 1e-30).all(), "first stage off by more than one bf16 ulp"
    assert (g1 != r1_bits).mean() < 0.01, "first-stage rounding differs too often"
    r2 = oracle.qlinear(r1_bits, w2.codes, w2.scales, w2.biases, 8, H, Q)
    # the two chains round their first stage to bf16 separately (a few
    # one-ulp differences), so only the contract tolerance applies here
    worst = assert_rows_close(y2.cpu().numpy(), r2, what="chained second projection", design=None)
    print(f"chain: {int((g1 != r1_bits).sum())} first-stage bf16 roundings differ; second stage {worst:.2e}")
