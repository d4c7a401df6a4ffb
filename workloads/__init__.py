"""Seeded synthetic inputs for the block-diffusion attention step.

This module only draws inputs. It holds none of the method's arithmetic (no
attention, merge, count, similarity or selection) and is the one piece of
code shared by the HIP path's tests and benchmark and by the oracle's tests.

Randomness: every tensor comes from its own
``numpy.random.Generator(PCG64(SeedSequence([cfg_id, variant, block, step,
tag, chunk])))`` so any tensor can be regenerated alone. Values are drawn in
float32 and rounded to bfloat16 with round-to-nearest-even (the fp32 workload
keeps float32). bf16 tensors are carried as their uint16 bit patterns; their
float32 view (``bf16_to_f32``) is exact, so the oracle's float64 upcast sees
exactly the bits the GPU receives.

The five workloads (sizes are the block-diffusion shapes the method targets:
a long static prefix KV cache J_out, and a block of B queries whose tokens
are updated over denoising steps):

1. ``tiny``   fp32, 4 q heads = 4 kv heads, d 64, prefix 1024, B 4, 8 steps,
              M ~ Uniform{0..4}, tau 2.
2. ``text``   bf16, 32q/8kv, d 128, prefix 32768, B 4, 16 steps,
              M ~ Binomial(4, 0.3), tau 2.
3. ``long``   bf16, 32q/8kv, d 128, B in {8, 16}, prefix in
              {100000, 131072, 200000, 400000, 800000}, 8 steps,
              M ~ Binomial(B, 0.3), tau 4.
4. ``video``  bf16, 12 MHA heads, d 128, 4680 block queries
              (3 frames x 1560), prefix 12480 (8 frames), 4 steps; per-head
              noise scale sigma_h ~ LogUniform(1e-3, 1), block Q/K/V random
              walk X <- X + sigma_h * eps; gamma 0.95.
5. ``sparse`` bf16, 32q/8kv, d 128, prefix 65536 in 16-token pages, B 8,
              8 steps, density {0.2, 0.3, 0.4}, M ~ Binomial(8, 0.3),
              active cutoff at the 25th percentile.

Update model for text workloads: at step 0 every block token gets fresh
N(0,1) Q/K/V and a unique id; at each later step M positions, drawn
uniformly without replacement, get fresh Q/K/V and a new unique id, and the
other rows keep theirs bit for bit.
"""

from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field, replace
import math
import os

import numpy as np

PREFIX_CHUNK = 65536          # tokens per independently seeded prefix chunk

TAG_PREFIX_K, TAG_PREFIX_V = 0, 1
TAG_Q, TAG_K, TAG_V = 2, 3, 4
TAG_UPDATE = 5
TAG_SIGMA = 6


# --------------------------------------------------------------------------
# bf16 bits
# --------------------------------------------------------------------------

def bf16_bits(x):
    """float32 array -> uint16 bf16 bit patterns, round to nearest even.

    Inputs are finite; no NaN special case is needed for the workloads.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_to_f32(bits):
    """uint16 bf16 bit patterns -> float32 (exact)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def values(x, dtype):
    """Exact float32 values of a workload tensor (bf16 bits or float32)."""
    return bf16_to_f32(x) if dtype == "bf16" else np.asarray(x, np.float32)


def rng(cfg_id, variant=0, block=0, step=0, tag=0, chunk=0):
    return np.random.Generator(np.random.PCG64(
        np.random.SeedSequence([cfg_id, variant, block, step, tag, chunk])))


def _draw(g, shape, dtype, scale=1.0):
    x = g.standard_normal(shape, dtype=np.float32)
    if scale != 1.0:
        x *= np.float32(scale)
    return bf16_bits(x) if dtype == "bf16" else x


# --------------------------------------------------------------------------
# configurations
# --------------------------------------------------------------------------

@dataclass(frozen=True)
class Config:
    name: str
    cfg_id: int
    dtype: str                  # "bf16" | "f32"
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    n_prefix: int
    n_block: int                # B text queries / video block queries
    n_steps: int
    tau: int = 0
    gamma: float = 0.0
    m_dist: str = "binomial"    # "uniform" | "binomial" | "none"
    m_p: float = 0.3
    page: int = 16
    density: float = 0.0
    pct: int = 25
    q_gain: float = 1.0         # >1: peaked scores (online-softmax stress)
    extra: dict = field(default_factory=dict, compare=False, hash=False)

    @property
    def scale(self):
        return 1.0 / math.sqrt(self.head_dim)

    @property
    def k_pages(self):
        n_pages = (self.n_prefix + self.page - 1) // self.page
        return int(math.floor(self.density * n_pages + 0.5))

    def with_(self, **kw):
        return replace(self, **kw)


TINY = Config("tiny", 1, "f32", 4, 4, 64, 1024, 4, 8, tau=2,
              m_dist="uniform")
TEXT = Config("text", 2, "bf16", 32, 8, 128, 32768, 4, 16, tau=2)
LONG = Config("long", 3, "bf16", 32, 8, 128, 131072, 16, 8, tau=4)
LONG_CONTEXTS = (100000, 131072, 200000, 400000, 800000)
LONG_BLOCKS = (8, 16)
VIDEO = Config("video", 4, "bf16", 12, 12, 128, 12480, 4680, 4, gamma=0.95,
               m_dist="none")
SPARSE = Config("sparse", 5, "bf16", 32, 8, 128, 65536, 8, 8, density=0.2)
SPARSE_DENSITIES = (0.2, 0.3, 0.4)

CONFIGS = {c.name: c for c in (TINY, TEXT, LONG, VIDEO, SPARSE)}


# --------------------------------------------------------------------------
# prefix KV (static across steps)
# --------------------------------------------------------------------------

def _prefix_tensor(cfg, tag, variant, n_tok, threads):
    hkv, d = cfg.n_kv_heads, cfg.head_dim
    dt = np.uint16 if cfg.dtype == "bf16" else np.float32
    out = np.empty((n_tok, hkv, d), dtype=dt)
    n_chunks = (n_tok + PREFIX_CHUNK - 1) // PREFIX_CHUNK

    def fill(c):
        lo = c * PREFIX_CHUNK
        hi = min(n_tok, lo + PREFIX_CHUNK)
        g = rng(cfg.cfg_id, variant, 0, 0, tag, c)
        out[lo:hi] = _draw(g, (hi - lo, hkv, d), cfg.dtype)

    if threads > 1 and n_chunks > 1:
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(fill, range(n_chunks)))
    else:
        for c in range(n_chunks):
            fill(c)
    return out


def prefix_kv(cfg, n_tok=None, variant=0, threads=None):
    """Prefix K, V [n_tok, Hkv, d] (bf16 bits or float32).

    Chunk c of PREFIX_CHUNK tokens is seeded by c alone, so a shorter prefix
    is the leading part of a longer one.
    """
    n_tok = cfg.n_prefix if n_tok is None else n_tok
    threads = threads or min(8, os.cpu_count() or 1)
    k = _prefix_tensor(cfg, TAG_PREFIX_K, variant, n_tok, threads)
    v = _prefix_tensor(cfg, TAG_PREFIX_V, variant, n_tok, threads)
    return k, v


# --------------------------------------------------------------------------
# text block: token updates
# --------------------------------------------------------------------------

def _draw_m(cfg, g):
    b = cfg.n_block
    if cfg.m_dist == "uniform":
        return int(g.integers(0, b + 1))
    if cfg.m_dist == "binomial":
        return int(g.binomial(b, cfg.m_p))
    return 0


def text_steps(cfg, variant=0, block=0, m_override=None, update_variant=None):
    """Per-step block inputs: dicts with q [B,Hq,d], k, v [B,Hkv,d], ids [B].

    ``m_override`` (list, one entry per step >= 1, or None entries) fixes M
    for chosen steps; positions are still drawn from the step's seed.
    ``update_variant``: draw M and the updated positions from that variant's
    seeds instead of ``variant``'s (layers of one stack share the block's
    token updates and differ in their Q/K/V).
    """
    b, hq, hkv, d = cfg.n_block, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    steps = []
    next_id = 0
    q = k = v = ids = None
    for s in range(cfg.n_steps):
        gq = rng(cfg.cfg_id, variant, block, s, TAG_Q)
        gk = rng(cfg.cfg_id, variant, block, s, TAG_K)
        gv = rng(cfg.cfg_id, variant, block, s, TAG_V)
        fq = _draw(gq, (b, hq, d), cfg.dtype, cfg.q_gain)
        fk = _draw(gk, (b, hkv, d), cfg.dtype)
        fv = _draw(gv, (b, hkv, d), cfg.dtype)
        if s == 0:
            q, k, v = fq, fk, fv
            ids = np.arange(b, dtype=np.int32) + np.int32(next_id)
            next_id += b
            m = b
            pos = np.arange(b)
        else:
            gu = rng(cfg.cfg_id, variant if update_variant is None else update_variant, block, s,
                     TAG_UPDATE)
            m = _draw_m(cfg, gu)
            if m_override is not None and m_override[s] is not None:
                m = int(m_override[s])
            pos = np.sort(gu.choice(b, size=m, replace=False))
            q, k, v, ids = q.copy(), k.copy(), v.copy(), ids.copy()
            q[pos], k[pos], v[pos] = fq[pos], fk[pos], fv[pos]
            ids[pos] = np.arange(next_id, next_id + m, dtype=np.int32)
            next_id += m
        steps.append(dict(q=q, k=k, v=v, ids=ids, m_drawn=m, updated=pos))
    return steps


def stack_layers(cfg, n_layers, block=0, n_prefix=None):
    """A stack of n_layers synthetic layers of the text workload ``cfg``: per
    layer its own prefix K/V (variant 100 + l) and block Q/K/V per step;
    every layer sees the same token updates (M, positions and ids of
    variant 0), as the layers of one model do. Returns a list of
    (k_prefix, v_prefix, steps)."""
    out = []
    for l in range(n_layers):
        kp, vp = prefix_kv(cfg, n_tok=n_prefix, variant=100 + l)
        out.append((kp, vp, text_steps(cfg, variant=100 + l, block=block, update_variant=0)))
    return out


# --------------------------------------------------------------------------
# video block: per-head random walk
# --------------------------------------------------------------------------

def video_sigmas(cfg, variant=0):
    """sigma_h ~ LogUniform(1e-3, 1), one per head (seeded by ``variant``)."""
    g = rng(cfg.cfg_id, variant, 0, 0, TAG_SIGMA)
    return np.exp(g.uniform(math.log(1e-3), math.log(1.0), cfg.n_q_heads))


def video_steps(cfg, sigmas, variant=0, block=0):
    """Per-step block Q [Nq, Hq, d] and K/V [Nq, Hkv, d] following
    X^{s+1} = X^s + sigma_h eps, sigma_h per query head; a KV head takes the
    sigma of its group's first query head (with one query head per KV head,
    every head its own).

    The walk is kept in float32; each step's inputs are its bf16 rounding
    (the float32 workload: the walk itself).
    """
    nq, hq, hkv, d = cfg.n_block, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    sig_q = np.asarray(sigmas, dtype=np.float32)
    sigs = {"q": sig_q[None, :, None], "k": sig_q[::hq // hkv][None, :, None]}
    sigs["v"] = sigs["k"]
    state = {}
    steps = []
    for s in range(cfg.n_steps):
        cur = {}
        for name, tag in (("q", TAG_Q), ("k", TAG_K), ("v", TAG_V)):
            h = hq if name == "q" else hkv
            sig = sigs[name]
            g = rng(cfg.cfg_id, variant, block, s, tag)
            eps = g.standard_normal((nq, h, d), dtype=np.float32)
            if s == 0:
                x = eps * np.float32(cfg.q_gain) if name == "q" else eps
            else:
                x = state[name] + sig * eps
            state[name] = x
            cur[name] = bf16_bits(x) if cfg.dtype == "bf16" else x.copy()
        steps.append(cur)
    return steps


# --------------------------------------------------------------------------
# sparse block
# --------------------------------------------------------------------------

def sparse_steps(cfg, variant=0, block=0, m_override=None):
    """Same update model as ``text_steps`` (unchanged tokens keep their query
    bit for bit, so their query MSE is exactly 0)."""
    return text_steps(cfg, variant, block, m_override)


# --------------------------------------------------------------------------
# singular-proxy identifier (SPA-Cache): hidden states and a value projection
# --------------------------------------------------------------------------

TAG_FACTOR_U, TAG_FACTOR_V, TAG_HIDDEN, TAG_DRIFT = 7, 8, 9, 10


@dataclass(frozen=True)
class SpaConfig:
    """N hidden states of model width D per denoising step, a rank-r factor of
    the value projection, and the share of tokens recomputed per step."""
    name: str = "spa"
    cfg_id: int = 6
    n_tok: int = 1024
    d_model: int = 4096
    rank: int = 128
    n_steps: int = 4
    ratio: float = 0.25

    @property
    def n_select(self):
        return int(math.floor(self.ratio * self.n_tok + 0.5))

    def with_(self, **kw):
        return replace(self, **kw)


SPA = SpaConfig()


def spectrum(n):
    """Singular values of the synthetic value projection: (i + 1) ** -0.5."""
    return (np.arange(n, dtype=np.float64) + 1.0) ** -0.5


def _orthonormal(g, rows, cols):
    q, r = np.linalg.qr(g.standard_normal((rows, cols)))
    return q * np.sign(np.diag(r))[None, :]


def spa_factor(cfg, variant=0):
    """The stored rank-r factor [D, r] (bf16 bits): U_r diag(sigma_1..r) of a
    value projection W = U diag(sigma) V^T whose U has orthonormal columns
    (QR of a seeded Gaussian matrix) and sigma = ``spectrum``."""
    u = _orthonormal(rng(cfg.cfg_id, variant, 0, 0, TAG_FACTOR_U), cfg.d_model, cfg.rank)
    f = u * spectrum(cfg.rank)[None, :]
    return bf16_bits(f.astype(np.float32))


def spa_projection(cfg, variant=0):
    """A whole synthetic value projection for small D: (U [D, D], sigma [D],
    V [D, D]) in float64, W = U diag(sigma) V^T, U and V orthonormal."""
    d = cfg.d_model
    u = _orthonormal(rng(cfg.cfg_id, variant, 0, 0, TAG_FACTOR_U), d, d)
    v = _orthonormal(rng(cfg.cfg_id, variant, 0, 0, TAG_FACTOR_V), d, d)
    return u, spectrum(d), v


def spa_steps(cfg, variant=0):
    """Hidden states [N, D] (bf16 bits) per denoising step: x^0 ~ N(0, 1), then
    a random walk x^{s+1} = x^s + delta_t eps with one drift scale per token,
    delta_t ~ LogUniform(1e-3, 1) (kept in float32, rounded per step)."""
    n, d = cfg.n_tok, cfg.d_model
    delta = np.exp(rng(cfg.cfg_id, variant, 0, 0, TAG_DRIFT).uniform(
        math.log(1e-3), 0.0, n)).astype(np.float32)[:, None]
    x = None
    out = []
    for s in range(cfg.n_steps):
        eps = rng(cfg.cfg_id, variant, 0, s, TAG_HIDDEN).standard_normal((n, d), dtype=np.float32)
        x = eps if s == 0 else x + delta * eps
        out.append(bf16_bits(x))
    return out


__all__ = [
    "Config", "CONFIGS", "TINY", "TEXT", "LONG", "VIDEO", "SPARSE",
    "LONG_CONTEXTS", "LONG_BLOCKS", "SPARSE_DENSITIES", "bf16_bits",
    "bf16_to_f32", "values", "rng", "prefix_kv", "text_steps",
    "video_sigmas", "video_steps", "sparse_steps", "SpaConfig", "SPA", "spectrum",
    "spa_factor", "spa_projection", "spa_steps",
]
