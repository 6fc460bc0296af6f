"""CPU oracle for the routed-MoE MLP forward (NumPy, float64).

TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py may import or call this package.  The HIP
library never does, and this package imports nothing from it.

What it computes, step by step, and where each step comes from:

  S0 (ScMoE only) pre-norm of the routed input:
     ms_t = sum_i x[t,i]^2 / H,  r_t = 1/sqrt(ms_t + eps),
     xr[t,i] = bf16(x[t,i] * r_t * gamma_pre[i]).
     Source: "core.models.hybrid.shortcut_block" (Megatron-Core API docs),
     module doc and ShortcutMoEBlock._moe_router_preprocess: the shortcut
     representation is normalised before routing and dispatch.  The norm
     is an RMSNorm with eps 1e-6 (the ScMoE workload's definition).
  S1 router GEMM: l = fp32( x @ W_r^T ), bf16 activations widened exactly,
     fp32 weights.  Source: "bridge.models.beam.modeling_beam",
     beam_router_gating_linear / _BeamRouterGatingLinear / BeamTopKRouter:
     logits in the router dtype, both operands in fp32, fp32 weights.
  S2 scores and top-k: s = sigmoid(l) (fp32), s' = s + b (fp32 add),
     the k largest s' over all E experts (ties to the lower id), ids
     emitted in ascending order, w = fp32(rsf * s[ids]) -- the bias
     steers the choice only, the weight is the unbiased score, the
     scaling factor multiplies routed weights only, k <= 16.
     Source: "Module glm5next_mlp" (metrale_model_arch docs), section
     "Numerics the kernels rely on"; Constants, KERNEL_MAX_TOP_K.
  S3 permute: stable counting sort of the T*k (token, slot) pairs by
     expert id -> offsets[E+1], sorted_token[T*k], inv_pos[T*k].
     Source: "Module glm5next_mlp", Constants, MOE_MODULE (token sort /
     permute / unpermute kernels).
  S4/S5 grouped SwiGLU experts: per expert, g = A Wg^T, u = A Wu^T,
     h = bf16( silu(min(g, L)) * clamp(u, -L, L) ), y = h Wd^T (not
     rounded).  Gate rows first, then up rows, in the fused weight.
     Source: "Module glm5next_mlp", "Numerics the kernels rely on" (the
     clamp bounds gate from above only and up on both sides);
     "mstar.model.components.distributed.mlp", ParallelGatedMLP (gate/up
     fused into one projection, gate = shard 0, up = shard 1).
  S6 shared expert: the same SwiGLU FFN with its own width, same clamp,
     on all rows, added unscaled.  Source: "Module glm5next_mlp", Modules
     (forward: the dense SwiGLU FFN also serves as the shared expert) and
     "Numerics the kernels rely on"; shortcut_block._moe_shared_experts
     (ScMoE: the shared expert sees the current layer's input).
  S7 combine: z[t] = sum_j w[t,j] * y[inv_pos[t*k+j]] + ys[t];
     out = bf16(z), or for ScMoE out = bf16(z * r_z * gamma_post) with
     r_z = 1/sqrt(mean(z^2) + eps).  Source: "Module glm5next_mlp",
     section "One all-reduce for both EP and TP" (shared output and routed
     slots added in one combine); shortcut_block module doc and
     ShortcutMoEBlock._postprocess (post-norm of the merged sum).
  S8 (optional) finish: the residual add that closes the layer,
     out = bf16(bf16(o * c0) + bf16(res * c1)) on the layer output o
     (after the post-norm, which a plain layer may also ask for: Beam's
     sandwich norm on the MLP output).  Source:
     "bridge.models.beam.modeling_beam", _beam_bda (bias -> post norm ->
     dropout -> depth-scaled residual add) and scaled_residual_add (the
     output times coefs[0] plus the residual times coefs[1], in the
     residual's dtype); "core.models.hybrid.shortcut_block",
     ShortcutMoEBlock._postprocess (finish residual/BDA): c0 = c1 = 1.
  Router backward (training; optional): for l = x W_r^T (+ bias) in fp32,
     grad_x = bf16(fp32(dL W_r)), grad_W = fp32(dL^T x), grad_b =
     fp32(sum_t dL[t]).  Source: "bridge.models.beam.modeling_beam",
     _BeamRouterGatingLinear (both GEMM operands in the router dtype, fp32;
     saved activations keep their dtype, bf16; an expanded stride-0
     gradient must be read correctly).

Readings where the pages are silent (each also listed in the design
notes): bias added to the sigmoid score, not to the logit; no
renormalisation of the top-k weights; ties go to the lower expert id; ids
ascending inside a token; NaN scores rank below every number; the clamp
acts on the fp32 pre-activations; bf16 rounding happens only at h, at the
ScMoE pre-norm output and at the final output; bf16(v) of a float64 value
is round-to-nearest-even of its fp32 rounding; eps is the fp32 value the
caller passes, widened.

W4A16 routed experts (optional, the next step after the bf16 path): the
pages name a grouped W4A16 expert GEMM ("Module glm5next_mlp", Modules
forward_prefill_gemm and Constants MOE_GROUPED_MODULE / W4A16_GEMV_MODULE)
and call the routed MoE NVFP4 (module doc), but give no layout.  The
reading taken here keeps NVFP4's two levels of scaling -- a one-byte
OCP E4M3 scale per block and one fp32 scale per weight tensor -- over
4-bit integer codes: signed 4-bit integers in offset-binary nibbles
(u - 8), packed along K in 4-byte words of 8 columns, byte j of a word
holding its columns j (low nibble) and j + 4 (high nibble) -- the
interleaved order lets a kernel split a word into its low and high
nibbles with one mask each; one E4M3 scale per output row and group of
128 columns, stored group-major ([K/128, rows]); one fp32 scale per
expert and projection.  The weight is exactly
(u - 8) * e4m3(scale) * tensor_scale and the expert FFN then runs as
above on those values.  The shared expert stays bf16.

Precision: all sums in float64 (BLAS matmul as a step), single roundings
at the points named above.  bf16 tensors are uint16 bit patterns.
"""
from __future__ import annotations

import numpy as np

KERNEL_MAX_TOP_K = 16


# ---------------------------------------------------------------- bf16 ----

def bf16_to_f64(u: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float64 (exact)."""
    u32 = np.asarray(u, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u32.view(np.float32).astype(np.float64)


def bf16_of_f32(f: np.ndarray) -> np.ndarray:
    """fp32 values -> bf16 bit patterns, round to nearest, ties to even."""
    f = np.ascontiguousarray(f, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint16)
    nan = np.isnan(f)
    if nan.any():                         # keep sign and payload, force quiet
        top = (f.view(np.uint32)[nan] >> np.uint32(16)).astype(np.uint16)
        r[nan] = top | np.uint16(0x0040)
    return r


def bf16_round(v: np.ndarray) -> np.ndarray:
    """float64 -> bf16 bit patterns via the fp32 value (the activation
    precision of the layer), round to nearest even."""
    with np.errstate(over="ignore", invalid="ignore"):
        return bf16_of_f32(np.asarray(v, dtype=np.float64).astype(np.float32))


# -------------------------------------------------------------- S0 norm ---

def rmsnorm_bf16(x_bits: np.ndarray, gamma: np.ndarray | None, eps: float) -> np.ndarray:
    """S0: xr = bf16(x * r * gamma), r = 1/sqrt(sum(x^2)/H + eps), fp64.

    `eps` is the fp32 value of the norm's epsilon, used widened to fp64.
    The product is formed as (x * r) * gamma in fp64, rounded to fp32,
    then to bf16 -- one fixed order so that an implementation doing the
    same IEEE operations reproduces every bit.
    """
    x = bf16_to_f64(x_bits)
    H = x.shape[-1]
    ms = np.sum(x * x, axis=-1) / H
    r = 1.0 / np.sqrt(ms + float(np.float32(eps)))
    v = x * r[..., None]
    if gamma is not None:
        v = v * np.asarray(gamma, dtype=np.float32).astype(np.float64)
    return bf16_round(v)


def rmsnorm_f64(z: np.ndarray, gamma: np.ndarray | None, eps: float) -> np.ndarray:
    """RMSNorm of a float64 matrix (the ScMoE post-norm before rounding)."""
    ms = np.mean(z * z, axis=-1)
    r = 1.0 / np.sqrt(ms + float(np.float32(eps)))
    v = z * r[..., None]
    if gamma is not None:
        v = v * np.asarray(gamma, dtype=np.float32).astype(np.float64)
    return v


# ------------------------------------------------------------ S1 router ---

def router_logits(x_bits: np.ndarray, w_router: np.ndarray) -> np.ndarray:
    """S1: l = fp32(x @ W_r^T), x widened exactly from bf16, fp64 sums."""
    x = bf16_to_f64(x_bits)
    wr = np.asarray(w_router, dtype=np.float32).astype(np.float64)
    return (x @ wr.T).astype(np.float32)


def sigmoid_f32(l: np.ndarray) -> np.ndarray:
    """S2: s = fp32(1 / (1 + exp(-l))) evaluated in fp64, rounded once."""
    l64 = np.asarray(l, dtype=np.float32).astype(np.float64)
    with np.errstate(over="ignore"):
        s = 1.0 / (1.0 + np.exp(-l64))
    return s.astype(np.float32)


def selection_order(s_biased: np.ndarray) -> np.ndarray:
    """Experts of each token ranked by (s' descending, id ascending); NaN
    scores rank after every number (NaNs among themselves by id)."""
    T, E = s_biased.shape
    ids = np.broadcast_to(np.arange(E), (T, E))
    neg = -s_biased.astype(np.float64)
    # lexsort: last key is primary; NaN sorts to the end of an ascending key.
    return np.lexsort((ids, neg), axis=-1)


def topk_route(logits: np.ndarray, corr_bias: np.ndarray | None, k: int,
               rsf: float) -> dict:
    """S2: scores, biased selection, ascending ids, unbiased weights.

    Returns dict(ids int32 [T,k], w fp32 [T,k], s fp32 [T,E], s_biased fp32
    [T,E], gap float64 [T]) where gap is the k-th minus the (k+1)-th biased
    score (inf when k == E) -- the tie margin of each token's selection.
    """
    T, E = logits.shape
    if not (1 <= k <= min(E, KERNEL_MAX_TOP_K)):
        raise ValueError(f"k={k} outside 1..min(E={E}, {KERNEL_MAX_TOP_K})")
    s = sigmoid_f32(logits)
    b = np.zeros(E, np.float32) if corr_bias is None else np.asarray(corr_bias, np.float32)
    sb = (s + b[None, :]).astype(np.float32)          # fp32 add
    order = selection_order(sb)
    ids = np.sort(order[:, :k], axis=1).astype(np.int32)
    w = (np.float32(rsf) * np.take_along_axis(s, ids, axis=1)).astype(np.float32)
    ranked = np.take_along_axis(sb, order, axis=1).astype(np.float64)
    if k < E:
        gap = ranked[:, k - 1] - ranked[:, k]
    else:
        gap = np.full(T, np.inf)
    return dict(ids=ids, w=w, s=s, s_biased=sb, gap=gap)


# ----------------------------------------------------------- S3 permute ---

def permute(ids: np.ndarray, E: int) -> dict:
    """S3: stable counting sort of the flattened (t, j) pairs by expert id."""
    T, k = ids.shape
    flat = ids.reshape(-1).astype(np.int64)
    counts = np.bincount(flat, minlength=E)
    offsets = np.zeros(E + 1, dtype=np.int64)
    np.cumsum(counts, out=offsets[1:])
    order = np.argsort(flat, kind="stable")
    inv_pos = np.empty(T * k, dtype=np.int64)
    inv_pos[order] = np.arange(T * k)
    return dict(offsets=offsets.astype(np.int32),
                sorted_token=(order // k).astype(np.int32),
                inv_pos=inv_pos.astype(np.int32),
                counts=counts.astype(np.int64))


# ------------------------------------------- W4A16 expert weights ----

W4_GROUP = 128


def e4m3_to_f64(codes: np.ndarray) -> np.ndarray:
    """OCP FP8 E4M3 bytes -> float64 (exact).

    Bit 7 is the sign, bits 6..3 the exponent field (bias 7), bits 2..0 the
    mantissa.  Exponent field 0 holds the subnormals m/8 * 2^-6 (and the
    two zeros); the others (1 + m/8) * 2^(field - 7); the one pattern per
    sign with every exponent and mantissa bit set is NaN -- the format has
    no infinities, so its largest value is 1.75 * 2^8 = 448.
    """
    b = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    field = (b >> 3) & 0xF
    m = (b & 7).astype(np.float64)
    mag = np.where(field == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(field - 7.0))
    v = np.where(b & 0x80, -mag, mag)
    return np.where((field == 15) & ((b & 7) == 7), np.nan, v)


def dequant_w4(q: np.ndarray, scale_codes: np.ndarray, tensor_scale: float = 1.0) -> np.ndarray:
    """W4A16 weights -> float64 values (exact).

    q             uint8 [R, K/2]: per 4-byte word w (columns 8w .. 8w+7), byte
                  4w + j holds column 8w + j (low nibble) and column 8w + j + 4
                  (high nibble); a nibble u stands for the integer u - 8
    scale_codes   uint8 [ceil(K/128), R]: one E4M3 scale per row and group of
                  128 columns
    tensor_scale  the fp32 scale of the whole matrix
    Returns w [R, K] with w[r, c] = (u[r, c] - 8) * e4m3(scale[c // 128, r])
    * tensor_scale.
    """
    q = np.asarray(q, dtype=np.uint8)
    R, half = q.shape
    K = 2 * half
    words = q.reshape(R, K // 8, 4).astype(np.int64)
    u = np.concatenate([words & 0x0F, words >> 4], axis=2).reshape(R, K)
    s = e4m3_to_f64(scale_codes)                                # [groups, R]
    per_col = np.repeat(s.T, W4_GROUP, axis=1)[:, :K]
    ts = float(np.float32(tensor_scale))
    return (u - 8).astype(np.float64) * per_col * ts


def _weights_f64(w: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) or already-widened float64 weights."""
    w = np.asarray(w)
    return bf16_to_f64(w) if w.dtype == np.uint16 else w.astype(np.float64)


def expert_weights(inp: dict, e: int) -> tuple[np.ndarray, np.ndarray]:
    """Routed expert e's (gate_up [2I, H], down [H, I]) weights: bf16 bits,
    or float64 values dequantised from the W4A16 arrays when `inp` holds
    w_gate_up_q / w_gate_up_scale / w_down_q / w_down_scale (and the
    per-expert tensor scales w_gate_up_tscale / w_down_tscale [E] fp32;
    absent = 1)."""
    if "w_gate_up_q" in inp:
        def ts(name):
            t = inp.get(name + "_tscale")
            return 1.0 if t is None else float(t[e])
        return (dequant_w4(inp["w_gate_up_q"][e], inp["w_gate_up_scale"][e], ts("w_gate_up")),
                dequant_w4(inp["w_down_q"][e], inp["w_down_scale"][e], ts("w_down")))
    return inp["w_gate_up"][e], inp["w_down"][e]


# ---------------------------------------------------------- S4-S6 FFN ----

def swiglu_pre(a: np.ndarray, w_gate_up: np.ndarray, limit: float,
               cols: np.ndarray | None = None) -> dict:
    """The SwiGLU of S4 (S6) before its bf16 rounding, fp64, for the output
    columns `cols` (all when None): g = a Wg^T and u = a Wu^T, the clamped
    h = silu(min(g, L)) * clamp(u, -L, L), and sum_i |a_i| |w_i| of the gate
    and up dot products (the scale of their rounding errors in any fp32
    evaluation).

    a          float64 [n, H];  w_gate_up bf16 [2I, H] (or float64 values)
    Returns dict(g, u, h, gabs, uabs), each [n, len(cols)] (or [n, I]).
    """
    I = w_gate_up.shape[0] // 2
    wg = _weights_f64(w_gate_up[:I] if cols is None else w_gate_up[:I][cols])
    wu = _weights_f64(w_gate_up[I:] if cols is None else w_gate_up[I:][cols])
    g = a @ wg.T
    u = a @ wu.T
    L = float(np.float32(limit))
    gc = np.minimum(g, L)                 # gate: bounded above only
    uc = np.clip(u, -L, L)                # up: bounded on both sides
    with np.errstate(over="ignore", invalid="ignore"):
        h = gc / (1.0 + np.exp(-gc)) * uc
    aa = np.abs(a)
    return dict(g=g, u=u, h=h, gabs=aa @ np.abs(wg).T, uabs=aa @ np.abs(wu).T)


def swiglu_ffn(a: np.ndarray, w_gate_up: np.ndarray, w_down: np.ndarray,
               limit: float, round_h: bool = True,
               h_given: np.ndarray | None = None) -> tuple[np.ndarray, np.ndarray]:
    """S4+S5 for one expert (or S6 for the shared one), fp64.

    a          float64 [n, H] (the rows routed to this expert)
    w_gate_up  bf16 [2I, H]: gate rows [0, I), up rows [I, 2I) (or float64
               weight values, e.g. dequantised W4A16 weights)
    w_down     bf16 [H, I] (or float64)
    h_given    float64 [n, I] or None: bf16 values of h to use instead of
               this function's own rounding (a valid rounding chosen by
               another evaluation: the layer is then re-derived from it)
    Returns (h float64 [n, I] -- the bf16 value when round_h, y float64
    [n, H], unrounded).
    """
    if h_given is not None:
        h = np.asarray(h_given, dtype=np.float64)
    else:
        I = w_gate_up.shape[0] // 2
        wg = _weights_f64(w_gate_up[:I])
        wu = _weights_f64(w_gate_up[I:])
        g = a @ wg.T
        u = a @ wu.T
        L = float(np.float32(limit))
        gc = np.minimum(g, L)                 # gate: bounded above only
        uc = np.clip(u, -L, L)                # up: bounded on both sides
        with np.errstate(over="ignore", invalid="ignore"):
            h = gc / (1.0 + np.exp(-gc)) * uc
        if round_h:
            h = bf16_to_f64(bf16_round(h))
    y = h @ _weights_f64(w_down).T
    return h, y


def routed_experts(xr_bits: np.ndarray, perm: dict, inp: dict, limit: float,
                   round_h: bool = True,
                   expert_range: tuple[int, int] | None = None,
                   h_given: np.ndarray | None = None) -> tuple[np.ndarray, np.ndarray]:
    """S4+S5 over all experts: rows of segment e of the permutation go
    through expert e (weights from expert_weights(inp, e)).  Returns
    (h_perm [T*k, I], y_perm [T*k, H]) float64 in permuted-row order; rows
    of experts outside `expert_range` stay 0.  h_given [T*k, I] (permuted
    rows) replaces the rounded h, as in swiglu_ffn."""
    offsets = perm["offsets"]
    st = perm["sorted_token"]
    E = offsets.shape[0] - 1
    H = xr_bits.shape[1]
    if "w_gate_up_q" in inp:
        I = inp["w_gate_up_q"].shape[1] // 2
    else:
        I = inp["w_gate_up"].shape[1] // 2
    M = st.shape[0]
    h_perm = np.zeros((M, I))
    y_perm = np.zeros((M, H))
    lo, hi = (0, E) if expert_range is None else expert_range
    for e in range(lo, hi):
        a0, a1 = int(offsets[e]), int(offsets[e + 1])
        if a1 == a0:
            continue
        a = bf16_to_f64(xr_bits[st[a0:a1]])
        wgu, wd = expert_weights(inp, e)
        hg = None if h_given is None else h_given[a0:a1]
        h, y = swiglu_ffn(a, wgu, wd, limit, round_h, hg)
        h_perm[a0:a1] = h
        y_perm[a0:a1] = y
    return h_perm, y_perm


# ----------------------------------------------------------- S7 combine ---

def combine(y_perm: np.ndarray, w: np.ndarray, inv_pos: np.ndarray,
            ys: np.ndarray | None) -> np.ndarray:
    """S7 (before rounding): z[t] = sum_j w[t,j] y[inv_pos[t*k+j]] + ys[t]."""
    T, k = w.shape
    H = y_perm.shape[1]
    z = np.zeros((T, H)) if ys is None else np.array(ys, dtype=np.float64)
    rows = inv_pos.reshape(T, k)
    for j in range(k):
        z += w[:, j].astype(np.float64)[:, None] * y_perm[rows[:, j]]
    return z


# ------------------------------------------------ S8 finish (optional) ---

def finish(out_bits: np.ndarray, residual_bits: np.ndarray, out_scale: float = 1.0,
           residual_scale: float = 1.0) -> np.ndarray:
    """S8: the residual add after the layer output, bf16 bits in and out.

    The pages' scaled_residual_add is output * coefs[0] + residual *
    coefs[1] in the residual's dtype: bf16 tensor arithmetic, where each
    product and the sum are computed in fp32 and rounded to bf16.  The
    layer has no output bias and dropout is the identity at inference, so
    the bias-dropout-add of the plain (ScMoE) finish is the case
    c0 = c1 = 1: bf16(o + res).  c0 and c1 are the caller's (the pages give
    only that their squares sum to one for Beam's depth-scaled add).
    """
    o = bf16_to_f64(out_bits).astype(np.float32)
    r = bf16_to_f64(residual_bits).astype(np.float32)
    with np.errstate(over="ignore", invalid="ignore"):
        a = bf16_of_f32(o * np.float32(out_scale))
        b = bf16_of_f32(r * np.float32(residual_scale))
        return bf16_of_f32(bf16_to_f64(a).astype(np.float32) + bf16_to_f64(b).astype(np.float32))


# ----------------------------------------- router backward (optional) ---

def router_backward(grad_logits: np.ndarray, x_bits: np.ndarray, w_router: np.ndarray) -> dict:
    """Gradients of l = x @ W_r^T (+ b) for the upstream gradient dL [T, E]
    (fp32; any strides, e.g. a broadcast view).  The GEMMs run in the
    router dtype (fp32), so their exact values are rounded once to fp32;
    grad_x is returned in the input's dtype (bf16), as autograd gives a
    gradient in its input's dtype.

    Returns dict(grad_x bf16 bits [T, H], grad_x_f64 (exact), grad_w fp32
    [E, H], grad_w_f64, grad_b fp32 [E], grad_b_f64).
    """
    dl = np.asarray(grad_logits, dtype=np.float64)
    x = bf16_to_f64(x_bits)
    w = np.asarray(w_router, dtype=np.float64)
    gx = dl @ w
    gw = dl.T @ x
    gb = dl.sum(axis=0)
    return dict(grad_x=bf16_round(gx), grad_x_f64=gx,
                grad_w=gw.astype(np.float32), grad_w_f64=gw,
                grad_b=gb.astype(np.float32), grad_b_f64=gb)


# ------------------------------------------------------------ the layer ---

def forward(inp: dict, *, k: int, rsf: float, limit: float, scmoe: bool = False,
            eps: float = 1e-6, ids: np.ndarray | None = None,
            round_h: bool = True, expert_range: tuple[int, int] | None = None,
            include_shared: bool = True, post_norm: bool = False,
            residual: np.ndarray | None = None, out_scale: float = 1.0,
            residual_scale: float = 1.0, h_given: np.ndarray | None = None,
            hs_given: np.ndarray | None = None) -> dict:
    """The whole layer (S0-S7) on one batch.

    `inp` holds the arrays named in moe_inputs.generate (x, x_cur,
    w_router, corr_bias, w_gate_up, w_down -- or their W4A16 forms
    w_gate_up_q, w_gate_up_scale, w_down_q, w_down_scale --, ws_gate_up,
    ws_down, gamma_pre, gamma_post).  When `ids` is given, routing uses those
    expert ids instead of the oracle's own top-k (the weights are still the
    oracle's unbiased scores for those ids); this re-derives the layer for
    tokens whose selection is a near-tie.  `expert_range` keeps only the
    routed slots of experts in [lo, hi) (one expert-parallel rank's share);
    `include_shared` drops the shared expert.  `post_norm` applies the
    post-norm (gamma_post) to a plain layer too; `residual` (bf16 bits
    [T, H]) adds the finish S8 with the two scales.  `h_given` (routed h,
    [T*k, I] in the permuted-row order of the routing used) and `hs_given`
    (shared h, [T, I_s]) replace the oracle's own bf16 rounding of h: an h
    within one bf16 step of the exact value is a valid result wherever the
    exact value lies within the rounding error of fp32 arithmetic of a
    rounding midpoint, and the rest of the layer is then re-derived from the
    rounding another evaluation chose, as for near-tie ids.

    Returns a dict with every intermediate: xr, logits, s, s_biased, gap,
    ids, w, offsets, sorted_token, inv_pos, h_perm, y_perm, hs, ys, z,
    out_layer (bf16 bits of the layer output), out (the same, or after the
    finish when a residual is given) and out_f64 (the value before the
    layer output's rounding).
    """
    x = inp["x"]
    T, H = x.shape
    wr = inp["w_router"]
    E = wr.shape[0]
    res: dict = {}
    if scmoe:
        xr = rmsnorm_bf16(x, inp.get("gamma_pre"), eps)
        x_sh = inp["x_cur"]
    else:
        xr = np.asarray(x, dtype=np.uint16)
        x_sh = x
    res["xr"] = xr
    logits = router_logits(xr, wr)
    r = topk_route(logits, inp.get("corr_bias"), k, rsf)
    res.update(logits=logits, s=r["s"], s_biased=r["s_biased"], gap=r["gap"])
    if ids is None:
        ids, w = r["ids"], r["w"]
    else:
        ids = np.asarray(ids, dtype=np.int32)
        w = (np.float32(rsf) * np.take_along_axis(r["s"], ids.astype(np.int64), axis=1)).astype(np.float32)
    res["ids"], res["w"] = ids, w
    p = permute(ids, E)
    res.update(offsets=p["offsets"], sorted_token=p["sorted_token"],
               inv_pos=p["inv_pos"], counts=p["counts"])
    h_perm, y_perm = routed_experts(xr, p, inp, limit, round_h, expert_range, h_given)
    res["h_perm"], res["y_perm"] = h_perm, y_perm
    ys = None
    if include_shared and inp.get("ws_gate_up") is not None and inp["ws_gate_up"].shape[0] > 0:
        hs, ys = swiglu_ffn(bf16_to_f64(x_sh), inp["ws_gate_up"], inp["ws_down"],
                            limit, round_h, hs_given)
        res["hs"] = hs
    res["ys"] = ys
    z = combine(y_perm, w, p["inv_pos"], ys)
    res["z"] = z
    if scmoe or post_norm:
        v = rmsnorm_f64(z, inp.get("gamma_post"), eps)
    else:
        v = z
    res["out_f64"] = v
    res["out_layer"] = bf16_round(v)
    res["out"] = res["out_layer"]
    if residual is not None:
        res["out"] = finish(res["out_layer"], residual, out_scale, residual_scale)
    return res


def take_rows(inp: dict, rows: np.ndarray) -> dict:
    """The same inputs restricted to a subset of tokens.  Every step of the
    layer is row-independent (the router ranks each token on its own), so
    forward(take_rows(inp, rows)) gives exactly those rows of the full
    forward's ids, weights and outputs."""
    out = dict(inp)
    out["x"] = inp["x"][rows]
    if "x_cur" in inp:
        out["x_cur"] = inp["x_cur"][rows]
    return out
