"""Seeded parity cases: inputs from gen/, expected values from oracle/.

Inputs are drawn with the generator; routing inputs are redrawn token by
token until the oracle's fp64 logits separate each token's top k+1 values by
at least 1e-3 (so the selected set and its order are decided by the data, not
by rounding).  Nothing here imports the HIP package.
"""
import numpy as np
import torch

import gen as G
import oracle as O

MIN_GAP = 1e-3

# (name, T, H, E, k, F) -- the small layer and the full-size shapes
TINY = dict(T=4, H=256, E=16, k=2, F=128)
FULL = dict(H=2048, E=512, k=10, F=768)


def rel_l2(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def assert_close_moe(y, y_ref, what=""):
    """MoE output tolerance: rel-L2 <= 2e-3 and max-abs <= 1e-2 * max|y_ref|."""
    y = np.asarray(y, np.float64)
    y_ref = np.asarray(y_ref, np.float64)
    r = rel_l2(y, y_ref)
    m = float(np.max(np.abs(y - y_ref)))
    lim = 1e-2 * float(np.max(np.abs(y_ref)))
    assert r <= 2e-3 and m <= lim, f"{what}: rel-L2 {r:.3e} (<= 2e-3), max-abs {m:.3e} (<= {lim:.3e})"
    return r, m


def x_as_f64(x):
    """fp32 or bf16 torch tensor -> exact float64 numpy."""
    return x.detach().cpu().to(torch.float64).numpy()


def router_f64(Wr_bits):
    return O.bf16_to_f64(Wr_bits.detach().cpu().numpy())


def gap_acceptor(Wr_bits, bias, k, as_bf16=False):
    """accept(x) for gen.draw_x_rejecting: True where the oracle's logits of
    token t have all top-(k+1) adjacent gaps >= MIN_GAP."""
    Wr = router_f64(Wr_bits)
    b = None if bias is None else bias.detach().cpu().double().numpy()

    def accept(x):
        xv = x.to(torch.bfloat16) if as_bf16 else x
        return O.gap_ok(O.router_logits(x_as_f64(xv), Wr, b), k, MIN_GAP)
    return accept


class LazyPool:
    """Byte view of a device pool for the oracle: copies only the slices asked for."""

    def __init__(self, pool):
        self.pool = pool

    def __getitem__(self, sl):
        return self.pool[sl].cpu().numpy()


def layer_case(seed, T, H, E, k, F, qfmt=0, bias=False, device="cpu", x_bf16=False, L=1, gap=True,
               random_bytes=False):
    """One or more layers of weights plus gap-safe tokens for layer 0."""
    li = G.make_layer_inputs(seed, L, E, H, F, qfmt=qfmt, bias=bias, device=device, random_bytes=random_bytes)
    b0 = None if li.bias is None else li.bias[0]
    acc = gap_acceptor(li.Wr[0], b0, k, as_bf16=x_bf16) if gap else (lambda x: np.ones(x.shape[0], bool))
    x, att = G.draw_x_rejecting(seed, T, H, acc, device=device)
    if x_bf16:
        x = x.to(torch.bfloat16)
    li.x = x
    li.attempts = att
    li.T, li.k = T, k
    return li


def oracle_layer(li, layer=0, x=None, tokens=None):
    """Oracle of one layer on li.x (or x); returns (y, idx, w, y_parts, logits)."""
    xx = li.x if x is None else x
    xf = x_as_f64(xx)
    if tokens is not None:
        xf = xf[tokens]
    get = O.expert_getter(LazyPool(li.pool), li.S.cpu().numpy(), layer, li.qfmt, li.H, li.F, li.R)
    b = None if li.bias is None else li.bias[layer].cpu().double().numpy()
    return O.moe_layer(xf, router_f64(li.Wr[layer]), b, li.k, get, li.E)
