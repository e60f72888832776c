"""Seeded synthetic inputs for the MoE layer: weights, activations, router,
selection bias from a Zipf popularity trace, and partition masks.

Every array is a pure function of (workload id, kind, indices), drawn from
``np.random.SeedSequence(ENTROPY, spawn_key=...)`` so that any single expert
of any layer can be regenerated on its own.  This module is the only code the
oracle side and the GPU side both consume; it holds no arithmetic of the MoE
forward (no routing, no FFN, no decoding).  The packers below *encode* fp32
draws into the stored weight formats; reading those bytes back is done
separately by the oracle and by the kernels.

Packed expert record (one contiguous byte string per expert, stride rounded up
to 4 KiB): the gate matrix [I, H], the up matrix [I, H] and the down matrix
[H, I], each row-major with the reduction dimension contiguous.
  f32 / bf16 : the three matrices' elements back to back.
  mxfp4      : E2M1 codes of gate, up, down (two per byte, low nibble = even
               element), then the E8M0 scales of gate, up, down ([rows, K/32]).
  nvfp4      : E2M1 codes as above, then E4M3 block scales ([rows, K/16]) of
               gate, up, down, then three little-endian fp32 tensor scales.
"""
import numpy as np

from .configs import F32, BF16, MXFP4, NVFP4, MoEConfig

ENTROPY = 20260817
KIND_EXPERT, KIND_ROUTER, KIND_ACT, KIND_TRACE, KIND_MASK, KIND_PERM, KIND_DRIFT = 0, 1, 2, 3, 4, 5, 6
RECORD_ALIGN = 4096


def rng(*key) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(ENTROPY, spawn_key=tuple(int(k) for k in key))))


# ---------------------------------------------------------------- encoders ---
def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest, ties to even); returns uint16 bit patterns."""
    b = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    rounding = ((b >> 16) & 1) + np.uint32(0x7FFF)
    return ((b + rounding) >> 16).astype(np.uint16)


def _e2m1_encode_mag(m: np.ndarray) -> np.ndarray:
    """Magnitude (already divided by the block scale) -> 3-bit E2M1 magnitude code,
    nearest with ties to the even code, saturating at 6.  The midpoints between
    neighbouring values are 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5; a value exactly
    on a midpoint goes to the even code, hence the alternating > / >=."""
    m = np.asarray(m, dtype=np.float32)
    code = (m > 0.25).astype(np.uint8)
    code += m >= 0.75
    code += m > 1.25
    code += m >= 1.75
    code += m > 2.5
    code += m >= 3.5
    code += m > 5.0
    return code


def e2m1_encode(v: np.ndarray) -> np.ndarray:
    sign = (np.signbit(v)).astype(np.uint8) << 3
    return sign | _e2m1_encode_mag(np.abs(v))


def e4m3_encode(v: np.ndarray) -> np.ndarray:
    """fp64/fp32 -> OCP E4M3 (bias 7, max 448, no inf), nearest-even, saturating."""
    v = np.asarray(v, dtype=np.float64)
    sign = np.signbit(v).astype(np.uint8) << 7
    a = np.minimum(np.abs(v), 448.0)
    # candidate exponent: normals cover [2^-6, 448]; below that subnormal step 2^-9
    _, e = np.frexp(np.where(a > 0, a, 1.0))     # a = f*2^e, f in [0.5,1)
    ex = np.clip(e - 1, -6, 8)                    # unbiased exponent of the binade
    step = np.ldexp(1.0, ex - 3)                  # spacing of 3 mantissa bits
    q = np.rint(a / step) * step                  # rint = ties to even on the step grid
    q = np.minimum(q, 448.0)
    # re-derive fields from the rounded value (rounding may carry into next binade)
    _, e2 = np.frexp(np.where(q > 0, q, 1.0))
    ex2 = e2 - 1
    normal = q >= 2.0 ** -6
    exp_field = np.where(normal, ex2 + 7, 0)
    mant = np.where(normal, np.rint((q / np.ldexp(1.0, ex2) - 1.0) * 8), np.rint(q / 2.0 ** -9))
    return (sign | (exp_field.astype(np.uint8) << 3) | mant.astype(np.uint8)).astype(np.uint8)


def _pack_nibbles(codes: np.ndarray) -> np.ndarray:
    c = codes.reshape(codes.shape[:-1] + (codes.shape[-1] // 2, 2))
    return (c[..., 0] | (c[..., 1] << 4)).astype(np.uint8)


def mxfp4_encode_matrix(w: np.ndarray):
    """[rows, K] fp32 -> (codes [rows, K/2] u8, scales [rows, K/32] u8 E8M0),
    shared exponent floor(log2(amax)) - 2 per 32-element block along K."""
    rows, K = w.shape
    blk = np.asarray(w, dtype=np.float32).reshape(rows, K // 32, 32)
    amax = np.abs(blk).max(axis=2).astype(np.float64)
    _, e = np.frexp(np.where(amax > 0, amax, 1.0))
    X = np.where(amax > 0, (e - 1) - 2, -127)
    X = np.clip(X, -127, 127)
    q = blk * np.ldexp(1.0, -X).astype(np.float32)[..., None]   # exact: power-of-two scaling
    codes = e2m1_encode(q).reshape(rows, K)
    return _pack_nibbles(codes), (X + 127).astype(np.uint8)


def nvfp4_encode_matrix(w: np.ndarray):
    """[rows, K] fp32 -> (codes [rows, K/2], E4M3 block scales [rows, K/16], fp32 tensor scale)."""
    rows, K = w.shape
    w32 = np.asarray(w, dtype=np.float32)
    amax_t = float(np.abs(w32).max())
    ts = np.float32(amax_t / (6.0 * 448.0)) if amax_t > 0 else np.float32(1.0)
    blk = w32.reshape(rows, K // 16, 16)
    amax_b = np.abs(blk).max(axis=2).astype(np.float64)
    sc = e4m3_encode(amax_b / 6.0 / float(ts))
    # decoded block-scale values are needed to place elements; E4M3 decoding here is
    # part of encoding (choosing codes), not of reading the record back
    sc_val = (_e4m3_value_for_encoding(sc) * float(ts)).astype(np.float32)
    inv = np.where(sc_val > 0, 1.0 / np.where(sc_val > 0, sc_val, 1.0), 0.0).astype(np.float32)
    q = blk * inv[..., None]
    codes = e2m1_encode(q).reshape(rows, K)
    return _pack_nibbles(codes), sc, ts


def _e4m3_value_for_encoding(c: np.ndarray) -> np.ndarray:
    c = c.astype(np.int64)
    e = (c >> 3) & 15
    m = c & 7
    mag = np.where(e == 0, m * 2.0 ** -9, (1 + m / 8.0) * np.ldexp(1.0, e - 7))
    return np.where(c & 0x80, -mag, mag)


# ------------------------------------------------------------ record layout ---
def record_bytes(H: int, I: int, w_dtype: int) -> int:
    n = 3 * H * I
    if w_dtype == F32:
        raw = 4 * n
    elif w_dtype == BF16:
        raw = 2 * n
    elif w_dtype == MXFP4:
        raw = n // 2 + n // 32
    elif w_dtype == NVFP4:
        raw = n // 2 + n // 16 + 12
    else:
        raise ValueError(w_dtype)
    return raw


def record_stride(H: int, I: int, w_dtype: int) -> int:
    r = record_bytes(H, I, w_dtype)
    return (r + RECORD_ALIGN - 1) // RECORD_ALIGN * RECORD_ALIGN


def expert_fp32(cfg: MoEConfig, layer: int, expert: int):
    """The fp32 draws (before format encoding) of one expert: gate [I,H], up [I,H], down [H,I]."""
    H, I, s = cfg.hidden, cfg.inter, cfg.weight_std
    out = []
    for tensor, shape in enumerate(((I, H), (I, H), (H, I))):
        g = rng(cfg.cid, KIND_EXPERT, layer, expert, tensor)
        out.append((g.standard_normal(shape, dtype=np.float32) * np.float32(s)).astype(np.float32))
    return out


def pack_record(mats, w_dtype: int, stride: int) -> np.ndarray:
    """Encode (gate, up, down) fp32 matrices into one packed record of `stride` bytes."""
    rec = np.zeros(stride, dtype=np.uint8)
    parts = []
    if w_dtype == F32:
        parts = [np.ascontiguousarray(m, dtype=np.float32).view(np.uint8).ravel() for m in mats]
    elif w_dtype == BF16:
        parts = [f32_to_bf16_bits(m).view(np.uint8).ravel() for m in mats]
    elif w_dtype == MXFP4:
        enc = [mxfp4_encode_matrix(m) for m in mats]
        parts = [c.ravel() for c, _ in enc] + [s.ravel() for _, s in enc]
    elif w_dtype == NVFP4:
        enc = [nvfp4_encode_matrix(m) for m in mats]
        parts = [c.ravel() for c, _, _ in enc] + [s.ravel() for _, s, _ in enc]
        parts.append(np.array([t for _, _, t in enc], dtype="<f4").view(np.uint8))
    else:
        raise ValueError(w_dtype)
    flat = np.concatenate(parts)
    assert flat.size <= stride
    rec[: flat.size] = flat
    return rec


def expert_record(cfg: MoEConfig, layer: int, expert: int) -> np.ndarray:
    return pack_record(expert_fp32(cfg, layer, expert), cfg.w_dtype,
                       record_stride(cfg.hidden, cfg.inter, cfg.w_dtype))


def layer_records(cfg: MoEConfig, layer: int) -> np.ndarray:
    """All E packed records of one layer, [E, stride] uint8."""
    stride = record_stride(cfg.hidden, cfg.inter, cfg.w_dtype)
    out = np.empty((cfg.n_experts, stride), dtype=np.uint8)
    for e in range(cfg.n_experts):
        out[e] = expert_record(cfg, layer, e)
    return out


# ------------------------------------------------------ activations, router ---
def _as_dtype(a32: np.ndarray, dtype: int) -> np.ndarray:
    """fp32 draws -> stored element type: float32 array, or uint16 bf16 bits."""
    if dtype == F32:
        return a32.astype(np.float32)
    if dtype == BF16:
        return f32_to_bf16_bits(a32)
    raise ValueError(dtype)


def router_weights(cfg: MoEConfig, layer: int) -> np.ndarray:
    g = rng(cfg.cid, KIND_ROUTER, layer)
    w = g.standard_normal((cfg.n_experts, cfg.hidden), dtype=np.float32) * np.float32(cfg.weight_std)
    return _as_dtype(w, cfg.router_dtype)


def activations(cfg: MoEConfig, step: int, layer: int, n_tokens: int) -> np.ndarray:
    g = rng(cfg.cid, KIND_ACT, step, layer, n_tokens)
    x = g.standard_normal((n_tokens, cfg.hidden), dtype=np.float32)
    return _as_dtype(x, cfg.act_dtype)


def layer_correlated_activations(cfg: MoEConfig, step: int, n_tokens: int, alpha: float) -> np.ndarray:
    """[layers, n_tokens, hidden] router inputs that drift from layer to layer
    like a residual stream: x_0 ~ N(0, 1), x_{l+1} = alpha x_l + sqrt(1 -
    alpha^2) z_l with fresh z_l ~ N(0, 1) (so every layer's input stays
    N(0, 1), and consecutive layers' inputs have correlation alpha), each
    stored in the activation dtype.  alpha = 0 gives independent layers."""
    L, H = cfg.n_layers, cfg.hidden
    out = []
    x = rng(cfg.cid, KIND_DRIFT, step, 0, n_tokens).standard_normal((n_tokens, H))
    for l in range(L):
        out.append(_as_dtype(x.astype(np.float32), cfg.act_dtype))
        z = rng(cfg.cid, KIND_DRIFT, step, l + 1, n_tokens).standard_normal((n_tokens, H))
        x = alpha * x + np.sqrt(1.0 - alpha * alpha) * z
    return np.stack(out)


# ------------------------------------------------------- trace and masks ----
def zipf_trace(cfg: MoEConfig, n_steps: int = None, n_tokens: int = 4) -> np.ndarray:
    """[steps, layers, n_tokens, k] int32 expert ids.  Per layer a seeded permutation
    maps popularity rank r (P proportional to r^-s) to an expert id; each token draws
    k distinct experts one after another without replacement (done with the
    Gumbel-top-k construction, which samples the same distribution)."""
    n_steps = cfg.trace_steps if n_steps is None else n_steps
    E, k, L = cfg.n_experts, cfg.top_k, cfg.n_layers
    ranks = np.arange(1, E + 1, dtype=np.float64)
    logp = -cfg.zipf_s * np.log(ranks)
    out = np.empty((n_steps, L, n_tokens, k), dtype=np.int32)
    for layer in range(L):
        perm = rng(cfg.cid, KIND_PERM, layer).permutation(E)
        g = rng(cfg.cid, KIND_TRACE, layer)
        gum = g.gumbel(size=(n_steps, n_tokens, E))
        order = np.argsort(-(logp[None, None, :] + gum), axis=-1, kind="stable")[..., :k]
        out[:, layer] = perm[order]
    return out


def sticky_trace(cfg: MoEConfig, n_steps: int, n_tokens: int, p_keep: float) -> np.ndarray:
    """[steps, layers, n_tokens, k] like zipf_trace, but with temporal
    locality: from one step to the next each of a token's k experts stays
    with probability p_keep, and the others are redrawn from the same
    popularity law (distinct from the kept ones)."""
    E, k, L = cfg.n_experts, cfg.top_k, cfg.n_layers
    ranks = np.arange(1, E + 1, dtype=np.float64)
    logp = -cfg.zipf_s * np.log(ranks)
    out = np.empty((n_steps, L, n_tokens, k), dtype=np.int32)
    for layer in range(L):
        perm = rng(cfg.cid, KIND_PERM, layer).permutation(E)
        g = rng(cfg.cid, KIND_TRACE, layer, 1)
        cur = None
        for st in range(n_steps):
            gum = logp[None, :] + g.gumbel(size=(n_tokens, E))
            if cur is None:
                cur = np.argsort(-gum, axis=-1, kind="stable")[:, :k]
            else:
                keep = g.random((n_tokens, k)) < p_keep
                nxt = np.empty_like(cur)
                for t in range(n_tokens):
                    kept = [r for r, kp in zip(cur[t], keep[t]) if kp]
                    sc = gum[t].copy()
                    sc[kept] = -np.inf
                    fresh = np.argsort(-sc, kind="stable")[:k - len(kept)]
                    nxt[t] = np.concatenate([np.array(kept, dtype=np.int64), fresh])
                cur = nxt
            out[st, layer] = perm[cur]
    return out


def trace_bias(ids_tk: np.ndarray, n_experts: int, value: float = 30.0) -> np.ndarray:
    """Selection-only bias [T, E] fp32 that puts the trace's experts on top."""
    T = ids_tk.shape[0]
    b = np.zeros((T, n_experts), dtype=np.float32)
    b[np.arange(T)[:, None], ids_tk] = np.float32(value)
    return b


def partition_masks(cfg: MoEConfig, layer: int, n: int = None) -> np.ndarray:
    """[n, ceil(E/32)] uint32 bitsets, each expert in with probability 1/2."""
    n = cfg.n_masks if n is None else n
    g = rng(cfg.cid, KIND_MASK, layer)
    bits = g.integers(0, 2, size=(n, cfg.n_experts), dtype=np.uint8)
    return bits_to_mask(bits)


def bits_to_mask(bits: np.ndarray) -> np.ndarray:
    bits = np.atleast_2d(bits)
    n, E = bits.shape
    W = (E + 31) // 32
    out = np.zeros((n, W), dtype=np.uint32)
    for e in range(E):
        out[:, e // 32] |= (bits[:, e].astype(np.uint32) << np.uint32(e % 32))
    return out


# ------------------------------------------------- device-side generation ---
# The benchmark pools (tens of GB) are generated on the device with torch's
# seeded generator: the same distribution and the same encoding rules as the
# host generator above, different random streams.  Parity tests use the host
# generator.
def _torch_e2m1_codes(torch, m):
    code = (m > 0.25).to(torch.uint8)
    code += (m >= 0.75).to(torch.uint8)
    code += (m > 1.25).to(torch.uint8)
    code += (m >= 1.75).to(torch.uint8)
    code += (m > 2.5).to(torch.uint8)
    code += (m >= 3.5).to(torch.uint8)
    code += (m > 5.0).to(torch.uint8)
    return code


def _torch_pack(torch, q):
    codes = _torch_e2m1_codes(torch, q.abs()) | (torch.signbit(q).to(torch.uint8) << 3)
    codes = codes.reshape(codes.shape[0], -1, 2)
    return (codes[..., 0] | (codes[..., 1] << 4)).reshape(codes.shape[0], -1)


def device_record_fp4(torch, gen, H: int, I: int, std: float, w_dtype: int, stride: int):
    """One packed MXFP4 / NVFP4-like record generated on the current device."""
    rec = torch.zeros(stride, dtype=torch.uint8, device="cuda")
    codes, scales, tscales = [], [], []
    for rows, K in ((I, H), (I, H), (H, I)):
        w = torch.randn((rows, K), generator=gen, device="cuda", dtype=torch.float32) * std
        if w_dtype == MXFP4:
            blk = w.view(rows, K // 32, 32)
            amax = blk.abs().amax(-1)
            _, e = torch.frexp(torch.where(amax > 0, amax, torch.ones_like(amax)))
            X = torch.where(amax > 0, e - 1 - 2, torch.full_like(e, -127)).clamp(-127, 127)
            q = blk * torch.ldexp(torch.ones_like(amax), -X)[..., None]
            codes.append(_torch_pack(torch, q.view(rows, K)).flatten())
            scales.append((X + 127).to(torch.uint8).flatten())
        else:
            amax_t = float(w.abs().max())
            ts = amax_t / (6.0 * 448.0) if amax_t > 0 else 1.0
            ts = float(np.float32(ts))
            blk = w.view(rows, K // 16, 16)
            sc = (blk.abs().amax(-1) / 6.0 / ts).to(torch.float8_e4m3fn)
            sv = sc.to(torch.float32) * ts
            q = blk / torch.where(sv > 0, sv, torch.ones_like(sv))[..., None]
            q = torch.where(sv[..., None] > 0, q, torch.zeros_like(q))
            codes.append(_torch_pack(torch, q.view(rows, K)).flatten())
            scales.append(sc.view(torch.uint8).flatten())
            tscales.append(ts)
    parts = codes + scales
    if w_dtype == NVFP4:
        parts.append(torch.from_numpy(np.array(tscales, dtype="<f4").view(np.uint8)).cuda())
    flat = torch.cat(parts)
    rec[: flat.numel()] = flat
    return rec


def device_layer_pool(torch, cfg: MoEConfig, layer: int, stride: int):
    """[E, stride] u8 device pool holding every expert record of one layer,
    generated on the device from a generator seeded by (workload, layer).
    bf16 layers: bf16 values (torch's nearest-even conversion) of N(0, std)
    draws, gate, up and down back to back; fp4 layers: device_record_fp4."""
    g = torch.Generator(device="cuda")
    g.manual_seed(ENTROPY * 1000 + cfg.cid * 100 + layer)
    if cfg.w_dtype == BF16:
        n = 3 * cfg.hidden * cfg.inter
        if stride < 2 * n:
            raise ValueError("stride below the bf16 record size")
        pool = torch.zeros((cfg.n_experts, stride), dtype=torch.uint8, device="cuda")
        for e in range(cfg.n_experts):
            w = torch.randn(n, generator=g, device="cuda", dtype=torch.float32).mul_(cfg.weight_std)
            pool[e, : 2 * n].copy_(w.to(torch.bfloat16).view(torch.uint8))
        return pool
    pool = torch.empty((cfg.n_experts, stride), dtype=torch.uint8, device="cuda")
    for e in range(cfg.n_experts):
        pool[e].copy_(device_record_fp4(torch, g, cfg.hidden, cfg.inter, cfg.weight_std, cfg.w_dtype, stride))
    return pool
