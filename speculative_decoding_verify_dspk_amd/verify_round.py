"""One verify round on the GPU, composed from the C-ABI calls.

A round ("mlx-dspark" wiki summary, "Architecture"): every projection of the
target over the M rows (anchor + drafts, or B requests x rows), the vocabulary
head with the row argmax (or logits for sampling), and the acceptance step,
whose few result words the caller may have written straight into pinned host
memory ("mlx-dspark releases", v0.2.0 notes: at most one device sync per
round).

Weights and activations are seeded synthetic tensors of the workload's shapes
(``inputs.LAYER_SHAPES``).  Each decoder layer contributes four launches, as a
real layer's dependencies allow: q/k/v grouped (they read the same rows), o,
gate/up grouped, down.  The four inputs of a layer are independent N(0, 1)
rows; attention, norms and the activation function are outside this path.

A round's launches can be captured once into HIP graphs (``capture_round``)
and replayed every round: the kernels take no host-side work between calls
(their workspaces come back zeroed), so a replay is the whole round in one
submission, without host launch gaps between its kernels.
"""
from __future__ import annotations

from dataclasses import dataclass, field

from . import binding, inputs


@dataclass
class Layer:
    qkv: list
    o: binding.DeviceQWeight
    gateup: list
    down: binding.DeviceQWeight


@dataclass
class VerifyStack:
    model: str
    n_layers: int
    bits: int
    max_m: int
    copies: int = 1
    seed: str = "stack"
    layers: list = field(default_factory=list)   # [copy][layer] -> Layer
    heads: list = field(default_factory=list)    # [copy] -> DeviceQWeight

    def __post_init__(self):
        import torch
        s = inputs.LAYER_SHAPES[self.model]
        self.hidden, self.qdim, self.kvdim, self.inter, self.vocab = (s["hidden"], s["q"], s["kv"], s["inter"],
                                                                      s["vocab"])
        H, Q, KV, F, V = self.hidden, self.qdim, self.kvdim, self.inter, self.vocab

        def mk(n, k, *lab):
            c, sc, bi = inputs.make_qweight_device(n, k, self.bits, self.model, self.seed, *lab)
            return binding.DeviceQWeight(n, k, self.bits, c, sc, bi)

        for cp in range(self.copies):
            ls = []
            for li in range(self.n_layers):
                ls.append(Layer(qkv=[mk(Q, H, cp, li, "q"), mk(KV, H, cp, li, "k"), mk(KV, H, cp, li, "v")],
                                o=mk(H, Q, cp, li, "o"),
                                gateup=[mk(F, H, cp, li, "gate"), mk(F, H, cp, li, "up")],
                                down=mk(H, F, cp, li, "down")))
            self.layers.append(ls)
            self.heads.append(mk(V, H, cp, "lm_head"))
        M = self.max_m
        act = lambda k, name: inputs.make_activations_device(M, k, self.model, self.seed, name)
        self.x_attn, self.x_o, self.x_mlp, self.x_down = act(H, "attn_in"), act(Q, "o_in"), act(H, "mlp_in"), \
            act(F, "down_in")
        self.h = act(H, "final_h")
        f32 = dict(dtype=torch.float32, device="cuda")
        self.y_qkv = [torch.empty((M, Q), **f32), torch.empty((M, KV), **f32), torch.empty((M, KV), **f32)]
        self.y_o = torch.empty((M, H), **f32)
        self.y_gu = [torch.empty((M, F), **f32), torch.empty((M, F), **f32)]
        self.y_down = torch.empty((M, H), **f32)
        self.argmax = torch.empty((M,), dtype=torch.int32, device="cuda")
        self.logits = torch.empty((M, V), **f32)
        # one workspace per launch shape (their split-K layouts differ)
        wsb = binding.qgemm_workspace_bytes
        self.ws_qkv = binding.alloc_workspace(wsb(Q, H, M) + 2 * wsb(KV, H, M))
        self.ws_o = binding.alloc_workspace(wsb(H, Q, M))
        self.ws_gu = binding.alloc_workspace(2 * wsb(F, H, M))
        self.ws_down = binding.alloc_workspace(wsb(H, F, M))
        self.ws_head = binding.alloc_workspace(binding.lmhead_workspace_bytes(V, M))

    # ------------------------------------------------------------------ sizes
    def layer_weight_bytes(self) -> int:
        L = self.layers[0][0]
        return sum(w.nbytes for w in L.qkv + [L.o] + L.gateup + [L.down])

    def head_weight_bytes(self) -> int:
        return self.heads[0].nbytes

    def round_weight_bytes(self) -> int:
        return self.n_layers * self.layer_weight_bytes() + self.head_weight_bytes()

    # ---------------------------------------------------------------- launches
    def launch_layers(self, m: int, copy: int = 0, stream=None) -> None:
        for L in self.layers[copy]:
            binding.qgemm_verify_grouped(L.qkv, self.x_attn, m, self.y_qkv, self.ws_qkv, stream)
            binding.qgemm_verify(L.o, self.x_o, m, self.y_o, self.ws_o, stream)
            binding.qgemm_verify_grouped(L.gateup, self.x_mlp, m, self.y_gu, self.ws_gu, stream)
            binding.qgemm_verify(L.down, self.x_down, m, self.y_down, self.ws_down, stream)

    def launch_head(self, m: int, copy: int = 0, want_logits: bool = False, stream=None) -> None:
        binding.lmhead_argmax(self.heads[copy], self.h, m, self.argmax, self.logits if want_logits else None,
                              self.ws_head, stream)

    def prepare_round(self, m: int, copy: int, want_logits: bool = False, stream=None):
        """The round's projection and head calls at width m on weight copy
        ``copy`` with their arguments marshalled once: (layer calls, head call)."""
        layers = []
        for L in self.layers[copy]:
            layers += [binding.prepare_qgemm_grouped(L.qkv, self.x_attn, m, self.y_qkv, self.ws_qkv, stream),
                       binding.prepare_qgemm(L.o, self.x_o, m, self.y_o, self.ws_o, stream),
                       binding.prepare_qgemm_grouped(L.gateup, self.x_mlp, m, self.y_gu, self.ws_gu, stream),
                       binding.prepare_qgemm(L.down, self.x_down, m, self.y_down, self.ws_down, stream)]
        head = binding.prepare_lmhead(self.heads[copy], self.h, m, self.argmax, self.logits if want_logits else None,
                                      self.ws_head, stream)
        return layers, head

    def capture_calls(self, m: int, copy: int, accept, want_logits: bool = False):
        """HIP graphs (layers, head, accept) of one round at width m on weight
        copy ``copy``; ``accept`` launches the acceptance step.  Replay them in
        that order on one stream."""
        import torch
        fns = (lambda: self.launch_layers(m, copy),
               lambda: self.launch_head(m, copy, want_logits=want_logits),
               accept)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):          # one eager pass before capture
            for f in fns:
                f()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graphs = []
        for f in fns:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                f()
            graphs.append(g)
        return graphs

    def capture_round(self, m: int, copy: int, draft_ids, accept_len, committed):
        """HIP graphs (layers, head, accept) of one greedy round at width m."""
        return self.capture_calls(m, copy, lambda: binding.accept_greedy(self.argmax, draft_ids, 1, m, accept_len,
                                                                          committed))
