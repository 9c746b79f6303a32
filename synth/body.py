"""A synthetic transformer forward pass as a body: a let-list with the type
of every let and the values read outside it, for the partition and the
dispatch count.  The shape of a GPT forward pass (token embedding, L
pre-norm blocks of causal attention and a GELU feed-forward, a final layer
normalization, the logits and a cross-entropy loss); contractions, the
embedding gather, head reshapes and the loss's mean are boundaries.  It is
not the pages' corpus program, which is not available: its counts are its
own.  No arithmetic of the method lives here."""
from typing import List, Sequence, Tuple

from .dag import Node

F32 = "f32"


class Body:
    def __init__(self):
        self.nodes: List[Node] = []
        self.types: List[Tuple[Tuple[int, ...], str]] = []
        self.outputs: List[bool] = []
        self.n_inputs = 0

    def _add(self, node: Node, shape: Sequence[int], dtype: str = F32) -> int:
        self.nodes.append(node)
        self.types.append((tuple(int(s) for s in shape), dtype))
        self.outputs.append(False)
        return len(self.nodes) - 1

    def input(self, shape, dtype=F32) -> int:
        k = self.n_inputs
        self.n_inputs += 1
        return self._add(Node("input", (), None, k), shape, dtype)

    def const(self, value: float) -> int:
        return self._add(Node("const", (), float(value)), ())

    def op(self, name: str, args: Sequence[int], shape, iparam=None) -> int:
        return self._add(Node(name, tuple(args), None, iparam), shape)

    def shape(self, i: int) -> Tuple[int, ...]:
        return self.types[i][0]


def layernorm(b: Body, x: int, gamma: int, beta: int, eps: int) -> int:
    s = b.shape(x)
    row = s[:-1] + (1,)
    mu = b.op("row_mean", [x], row)
    d = b.op("sub", [x, mu], s)
    var = b.op("row_mean", [b.op("pow2", [d], s)], row)
    den = b.op("sqrt", [b.op("add", [var, eps], row)], row)
    return b.op("add", [b.op("mul", [b.op("div", [d, den], s), gamma], s), beta], s)


def softmax_causal(b: Body, scores: int, scale: int, T: int) -> int:
    s = b.shape(scores)
    row = s[:-1] + (1,)
    y = b.op("causal_mask", [b.op("mul", [scores, scale], s)], s, iparam=T)
    z = b.op("sub", [y, b.op("row_max", [y], row)], s)
    e = b.op("exp", [z], s)
    return b.op("div", [e, b.op("row_sum", [e], row)], s)


def gpt_forward(V: int = 92, D: int = 64, H: int = 2, L: int = 2, B: int = 2, T: int = 32) -> Body:
    """Loss of a GPT of L blocks over a batch of B sequences of T tokens."""
    b = Body()
    N, HD = B * T, D // H
    tokens = b.input((N,), F32)
    table = b.input((V, D))
    pos = b.input((T, D))
    eps = b.const(1e-5)
    x = b.op("add", [b.op("opaque", [tokens, table], (N, D)), pos], (N, D))
    scale = b.const(1.0 / HD ** 0.5)
    for _ in range(L):
        g1, b1, g2, b2 = b.input((D,)), b.input((D,)), b.input((D,)), b.input((D,))
        wqkv, wo, w1, w2 = b.input((D, 3 * D)), b.input((D, D)), b.input((D, 4 * D)), b.input((4 * D, D))
        bo, bb1, bb2 = b.input((D,)), b.input((4 * D,)), b.input((D,))
        h = layernorm(b, x, g1, b1, eps)
        qkv = b.op("matmul", [h, wqkv], (N, 3 * D))
        q = b.op("opaque", [qkv], (B * H * T, HD))          # split heads
        k = b.op("opaque", [qkv], (B * H * HD, T))          # split heads, transposed
        v = b.op("opaque", [qkv], (B * H * T, HD))
        p = softmax_causal(b, b.op("matmul", [q, k], (B * H * T, T)), scale, T)
        a = b.op("opaque", [b.op("matmul", [p, v], (B * H * T, HD))], (N, D))   # merge heads
        x = b.op("add", [x, b.op("add", [b.op("matmul", [a, wo], (N, D)), bo], (N, D))], (N, D))
        h = layernorm(b, x, g2, b2, eps)
        f = b.op("gelu", [b.op("add", [b.op("matmul", [h, w1], (N, 4 * D)), bb1], (N, 4 * D))], (N, 4 * D))
        x = b.op("add", [x, b.op("add", [b.op("matmul", [f, w2], (N, D)), bb2], (N, D))], (N, D))
    gf, bf = b.input((D,)), b.input((D,))
    h = layernorm(b, x, gf, bf, eps)
    logits = b.op("matmul", [h, b.input((D, V))], (N, V))
    # cross entropy: log-sum-exp minus the picked logit, averaged
    m = b.op("row_max", [logits], (N, 1))
    z = b.op("sub", [logits, m], (N, V))
    lse = b.op("add", [b.op("log", [b.op("row_sum", [b.op("exp", [z], (N, V))], (N, 1))], (N, 1)), m], (N, 1))
    picked = b.op("opaque", [logits, tokens], (N, 1))     # gather of the target logit
    loss = b.op("reduce", [b.op("sub", [lse, picked], (N, 1))], ())
    b.outputs[loss] = True
    return b
