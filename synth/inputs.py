"""Seeded synthetic input sets C1..C5 and their parity-only variants.

The pages measure on public benchmarks through real drafter/target models
(P2 "A 2B Drafter Made a 27B Model 3.4x Faster. Same Exact Output.",
sections "How many tokens survive" and "Throughput at batch size 1"); none
of those is used.  These inputs only take their shapes and value structure:

* drafter logits U [B, L, V] ~ N(0, sigma^2) rounded to the storage type;
* in C2..C4 each drafter row gets one planted token whose rank among the
  row follows the recall-by-position figures of P1 "DFlash 2: Block
  diffusion, wearing a drafter's coat", section "Sixteen candidates per
  position" (in the top 16 with probability 99.5% at position 1, falling
  linearly), with the top-1 share of P2's section "What a block-diffusion
  drafter is, and why it kept breaking" (85.4%);
* target logits Z [B, L+1, V] = U + N(0, noise^2), rounded; row L+1 is a
  fresh drafter-like row plus noise;
* x0 uniform over the vocabulary, E [V, r] ~ N(0, e_std^2),
  W [r, hidden] ~ N(0, 0.02^2), h [B, L, hidden] ~ N(0, 1);
* T per stream; Philox seed of stream b = (config_id << 32) | b.

All draws come from numpy.random.Generator(PCG64(SeedSequence([config_id,
set_id]))), in float32, rounded to bf16 with round-to-nearest-even.
"""

import numpy as np

# config id -> shape and value recipe (the five configurations of the
# benchmark plan; id 1 is the tiny case the oracle finishes in milliseconds)
CONFIGS = {
    1: dict(name="tiny", B=1, L=8, V=1024, K=16, r=256, hidden=256,
            logit_kind="f32", param_kind="f32", u_std=1.0, noise=0.5,
            plant="plus3", T=(0.0,)),
    2: dict(name="single-stream", B=1, L=8, V=151936, K=16, r=256, hidden=2048,
            logit_kind="bf16", param_kind="bf16", u_std=2.0, noise=1.0,
            plant="rank", recall=(0.995, 0.0195), T=(0.0,)),
    3: dict(name="concurrent-32", B=32, L=8, V=151936, K=16, r=256, hidden=2048,
            logit_kind="bf16", param_kind="bf16", u_std=2.0, noise=1.0,
            plant="rank", recall=(0.995, 0.0195), T=(1.0,)),
    4: dict(name="long-block-16", B=32, L=16, V=151936, K=16, r=256, hidden=2048,
            logit_kind="bf16", param_kind="bf16", u_std=2.0, noise=1.0,
            plant="rank", recall=(0.995, 0.013), T=(1.0,)),
    5: dict(name="large-vocab-128", B=128, L=8, V=262144, K=16, r=256, hidden=3072,
            logit_kind="bf16", param_kind="bf16", u_std=2.0, noise=1.0,
            plant=None, T=(0.0, 0.6, 1.0)),
}

TOP1_GIVEN_TOP16 = 0.854 / 0.995


def bf16_bits(x):
    """Round float32 values to bf16 (nearest, ties to even); return uint16 patterns."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (b >> np.uint32(16)) & np.uint32(1)
    return ((b + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def bf16_value(bits):
    """float32 holding the value of bf16 patterns (a representation change)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _store(x, kind):
    return bf16_bits(x) if kind == "bf16" else np.asarray(x, dtype=np.float32)


def _value(x, kind):
    return bf16_value(x) if kind == "bf16" else np.asarray(x, dtype=np.float32)


def _next_up_bf16(v):
    """Smallest bf16 value strictly above the (bf16-exact) float32 ``v``."""
    bits = int(bf16_bits(np.float32(v))[0])
    if v >= 0:
        bits = 0x0001 if bits == 0x8000 else bits + 1
    else:
        bits = 0x0000 if bits == 0x8001 else bits - 1   # -tiny -> -0 -> step to +0
    return float(bf16_value(np.uint16(bits)))


def _planted_rank(rng, recall):
    if rng.random() < recall:
        return 1 if rng.random() < TOP1_GIVEN_TOP16 else int(rng.integers(2, 17))
    return int(rng.integers(17, 65))


def _plant_row(rng, std, V, kind, recall, max_tries=200):
    """One drafter row with a token planted at a drawn rank (bf16 storage).

    The planted value is the smallest bf16 value above the row's rank-th
    largest other value; the row is re-drawn until that value also lies
    strictly below the (rank-1)-th, so that the realised rank is exact.
    """
    y = int(rng.integers(0, V))
    rank = _planted_rank(rng, recall)
    for _ in range(max_tries):
        row = _value(_store(rng.standard_normal(V, dtype=np.float32) * np.float32(std), kind), kind)
        others = np.delete(row, y)
        top = np.sort(np.partition(others, others.size - 64)[-64:])[::-1]
        x = _next_up_bf16(top[rank - 1])
        if rank == 1 or x < top[rank - 2]:
            row[y] = x
            return row, y, rank
    row[y] = top[rank - 1]                       # give up: realised as a tie
    return row, y, rank


def make(config_id, set_id=0, *, B=None, L=None, V=None, K=None, r=None,
         hidden=None, T=None, e_std=0.02, zero_E=False, ties=False,
         plant="default", cycle=None, noise=None, boost=None, shift=None):
    """Build one input set.

    Keyword overrides shrink or vary a configuration for parity cases:
    ``e_std`` (0.3 gives the strong-selector variant whose paths leave the
    top-1), ``zero_E`` (all-zero embeddings), ``ties`` (logits quantised to
    multiples of 0.5 so that rows hold many exactly equal values), ``T``
    (a scalar or a per-stream sequence), ``plant`` (None disables planted
    tokens), ``noise`` (the target's noise level; 0 makes target rows
    1..L copies of the drafter rows), ``boost`` (added to one uniformly
    chosen token of every drafter row, and so of its target row, but not to
    the extra target row L+1) and ``shift`` (a constant added to every drafter
    and target logit, for large logits at low temperature).  Returns a dict
    of numpy arrays in storage form plus the scalar dimensions.
    """
    cfg = dict(CONFIGS[config_id])
    for k, v in dict(B=B, L=L, V=V, K=K, r=r, hidden=hidden).items():
        if v is not None:
            cfg[k] = int(v)
    if plant != "default":
        cfg["plant"] = plant
    Bn, Ln, Vn, Kn, rn, Hn = (cfg[k] for k in ("B", "L", "V", "K", "r", "hidden"))
    lk, pk = cfg["logit_kind"], cfg["param_kind"]
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([config_id, set_id])))

    U = np.empty((Bn, Ln, Vn), dtype=np.uint16 if lk == "bf16" else np.float32)
    Z = np.empty((Bn, Ln + 1, Vn), dtype=U.dtype)
    planted = np.full((Bn, Ln + 1), -1, dtype=np.int64)
    planted_rank = np.zeros((Bn, Ln + 1), dtype=np.int64)
    std = np.float32(cfg["u_std"])
    noise = np.float32(cfg["noise"] if noise is None else noise)

    def drafter_row(t):
        # t: 0-based row index; row Ln is the extra target row's source
        if cfg["plant"] == "rank":
            a, slope = cfg["recall"]
            row, y, rk = _plant_row(rng, std, Vn, lk, a - slope * t)
            return row, y, rk
        row = _value(_store(rng.standard_normal(Vn, dtype=np.float32) * std, lk), lk)
        if cfg["plant"] == "plus3":
            y = int(rng.integers(0, Vn))
            row[y] = _value(_store(row[y:y + 1] + np.float32(3.0), lk), lk)[0]
            return row, y, 0
        return row, -1, 0

    for b in range(Bn):
        for t in range(Ln + 1):
            row, y, rk = drafter_row(t)
            if shift is not None:
                row = _value(_store(row + np.float32(shift), lk), lk)
            if boost is not None and t < Ln:
                yb = int(rng.integers(0, Vn))
                row[yb] = _value(_store(row[yb:yb + 1] + np.float32(boost), lk), lk)[0]
            if ties:
                row = np.round(row * np.float32(2.0)) / np.float32(2.0)
            planted[b, t], planted_rank[b, t] = y, rk
            zt = row + rng.standard_normal(Vn, dtype=np.float32) * noise
            if ties:
                zt = np.round(zt * np.float32(2.0)) / np.float32(2.0)
            Z[b, t] = _store(zt, lk)
            if t < Ln:
                U[b, t] = _store(row, lk)

    if zero_E:
        E = _store(np.zeros((Vn, rn), dtype=np.float32), pk)
    else:
        E = _store(rng.standard_normal((Vn, rn), dtype=np.float32) * np.float32(e_std), pk)
    W = _store(rng.standard_normal((rn, Hn), dtype=np.float32) * np.float32(0.02), pk)
    h = _store(rng.standard_normal((Bn, Ln, Hn), dtype=np.float32), pk)
    x0 = rng.integers(0, Vn, size=Bn).astype(np.int32)

    if T is None:
        choices = np.asarray(cfg["T"], dtype=np.float32)
        Tb = choices[rng.integers(0, len(choices), size=Bn)] if len(choices) > 1 \
            else np.full(Bn, choices[0], dtype=np.float32)
    else:
        Tb = np.broadcast_to(np.asarray(T, dtype=np.float32), (Bn,)).copy()
    seed = ((np.uint64(config_id) << np.uint64(32)) | np.arange(Bn, dtype=np.uint64)).astype(np.uint64)

    return dict(config_id=config_id, set_id=set_id, name=cfg["name"],
                B=Bn, L=Ln, V=Vn, K=Kn, r=rn, hidden=Hn,
                logit_kind=lk, param_kind=pk,
                U=U, Z=Z, x0=x0, E=E, W=W, h=h, T=Tb.astype(np.float32), seed=seed,
                cycle=int(set_id if cycle is None else cycle),
                planted=planted, planted_rank=planted_rank)


def make_conv(config_id, set_id=0, *, B=None, L=None, hidden=None, kind=None, w_std=0.02):
    """Inputs of the two-tap convolution for configuration ``config_id``:
    the block representations x [B, L, hidden] and their first predecessor
    x0 [B, hidden] (standard normal, like the gate's context vectors), and
    the tap generator Wt [2 * hidden, hidden] (normal, ``w_std``), stored in
    the configuration's parameter kind unless ``kind`` overrides it."""
    cfg = dict(CONFIGS[config_id])
    Bn = int(B if B is not None else cfg["B"])
    Ln = int(L if L is not None else cfg["L"])
    Hn = int(hidden if hidden is not None else cfg["hidden"])
    pk = kind or cfg["param_kind"]
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([config_id, set_id, 77])))
    x = _store(rng.standard_normal((Bn, Ln, Hn), dtype=np.float32), pk)
    x0 = _store(rng.standard_normal((Bn, Hn), dtype=np.float32), pk)
    Wt = _store(rng.standard_normal((2 * Hn, Hn), dtype=np.float32) * np.float32(w_std), pk)
    return dict(config_id=config_id, set_id=set_id, B=Bn, L=Ln, hidden=Hn, param_kind=pk, x=x, x0=x0, Wt=Wt)



def make_lattice(set_id=0, *, B=256, L=8, V=151936, hidden=256, T=1.0, affinity=2.8, target_p=0.8,
                 sharpen=4.0):
    """Planted lattices on which the pair selector has something to find.

    The drafter rows are those of the concurrent-32 recipe (a planted token
    per position whose rank in the row follows the recall-by-position
    figures, P1 "Sixteen candidates per position"); on top of them:

    * the drafter rows are multiplied by ``sharpen`` (a power of two, so the
      bf16 values and every rank stay exact): a drafter whose top candidates
      stand apart, as a trained one's do, instead of the nearly flat top 16
      of N(0, 2) rows;
    * the target's rows 1..L put their mode on the planted token: its logit
      is set so that at T = 1 it holds ``target_p`` of the row's mass (so at
      T = 0 it is the row's argmax), the target "agreeing" with the planted
      path;
    * each stream's planted tokens and its last verified token x0 share one
      embedding direction: E[y] = affinity * u_b (u_b a random unit vector
      of stream b), all other rows ~ N(0, 0.02); under a gate g near 1/2
      every consecutive pair of planted tokens then gets a bilinear bonus of
      about affinity^2 / 2 over a pair that leaves the planted path.

    Only value structure is drawn here: nothing of the method is computed.
    Returns the input dict of ``make`` (its ``planted`` array holds the
    planted tokens) with these Z and E.
    """
    inp = make(3, set_id, B=B, L=L, V=V, hidden=hidden, T=T)
    assert sharpen > 0 and float(np.log2(sharpen)).is_integer()
    inp["U"] = bf16_bits(bf16_value(inp["U"]) * np.float32(sharpen))
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([3, set_id, 991])))
    logit_p = np.log(target_p / (1.0 - target_p))
    for b in range(B):
        for t in range(L):
            y = int(inp["planted"][b, t])
            z = bf16_value(inp["Z"][b, t]).astype(np.float64)
            others = np.delete(z, y)
            mx = others.max()
            lse = mx + np.log(np.exp(others - mx).sum())
            inp["Z"][b, t, y] = bf16_bits(np.float32(lse + logit_p))[0]
    r = inp["r"]
    E = bf16_value(inp["E"]).copy()
    for b in range(B):
        u = rng.standard_normal(r).astype(np.float32)
        u /= np.linalg.norm(u)
        for tok in [int(inp["x0"][b])] + [int(y) for y in inp["planted"][b, :L]]:
            E[tok] = np.float32(affinity) * u
    inp["E"] = bf16_bits(E)
    inp["name"] = "planted-lattice"
    return inp
