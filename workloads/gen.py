"""Seeded input generation (numpy PCG64), no arithmetic of the method.

Recipe: ``Generator(PCG64(seed))``, ``standard_normal(float32)`` times the
config's std, then encoded round-to-nearest-even as bf16 bit patterns
(uint16) for bf16 configs or kept as float32 for the fp32 config.
Draw order per block: q, k_cur, v_cur, k_ctx, v_ctx; after all blocks the
shared text k, v; then the latents x and the noise prediction eps (N(0,1)).
"""
import numpy as np

from .configs import Config


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Encode float32 values as bf16 bit patterns, round to nearest even.

    NaN inputs are kept quiet NaN.  This is an input encoding only.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    out = rounded.astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = 0x7FC0
    return out


def draw(rng: np.random.Generator, shape, std: float, dtype: str) -> np.ndarray:
    """One normally distributed tensor: float32 for "f32", bf16 bits for "bf16"."""
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    if dtype == "f32":
        return x
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    raise ValueError(dtype)


def make_attention_inputs(cfg: Config, rng: np.random.Generator = None) -> dict:
    """All attention inputs of a config, in the token-major layout
    ``[tokens][heads][head_dim]`` that a QKV projection emits."""
    if rng is None:
        rng = np.random.Generator(np.random.PCG64(cfg.seed))
    H, D = cfg.heads, cfg.head_dim
    out = {"q": [], "k_cur": [], "v_cur": [], "k_ctx": [], "v_ctx": []}
    for _ in range(cfg.n_blocks):
        out["q"].append(draw(rng, (cfg.q_len, H, D), cfg.std, cfg.dtype))
        out["k_cur"].append(draw(rng, (cfg.cur_len, H, D), cfg.std, cfg.dtype))
        out["v_cur"].append(draw(rng, (cfg.cur_len, H, D), cfg.std, cfg.dtype))
        if cfg.ctx_len:
            out["k_ctx"].append(draw(rng, (cfg.ctx_len, H, D), cfg.std, cfg.dtype))
            out["v_ctx"].append(draw(rng, (cfg.ctx_len, H, D), cfg.std, cfg.dtype))
    res = {k: np.stack(v) for k, v in out.items() if v}
    res["k_text"] = draw(rng, (cfg.text_len, H, D), cfg.std, cfg.dtype)
    res["v_text"] = draw(rng, (cfg.text_len, H, D), cfg.std, cfg.dtype)
    res["_rng"] = rng
    return res


def make_update_inputs(cfg: Config, rng: np.random.Generator) -> dict:
    """Latents x and noise prediction eps, ``[n_blocks][elems]`` bf16 bits."""
    E = cfg.update_elems
    x = draw(rng, (cfg.n_blocks, E), 1.0, "bf16")
    eps = draw(rng, (cfg.n_blocks, E), 1.0, "bf16")
    return {"x": x, "eps": eps, "t": np.array(cfg.timesteps, dtype=np.int32)}
