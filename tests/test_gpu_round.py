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
