"""Seeded random configurations of the supported space, shared by the GPU test that runs them
and the CPU test that checks what they cover.  No library call: the supported space is
restated here (element type bf16 or fp32, head dim 64 or 128, blocks of 4 to 128 slots; MFMA or
VALU tiles for bf16 at head dim 128 with up to 16 query heads per KV head, the vector kernel
for blocks of at most 32 slots and up to 8 query heads per KV head), and the GPU test checks
that the library selects the same path."""
import numpy as np

N_CASES = 80
MAX_WORKSPACE = 256 << 20


def expected_path(dt: str, D: int, B: int, g: int) -> str | None:
    if D not in (64, 128) or B not in (4, 8, 16, 32, 64, 128):
        return None
    if dt == "bf16" and D == 128 and g <= 16:
        return "valu" if g == 1 else "mfma"
    return "vector" if B <= 32 and g <= 8 else None


def draw(case: int) -> dict:
    """One supported configuration from seed `case` (deterministic)."""
    rng = np.random.default_rng(20_000 + case)
    while True:
        dt = "f32" if rng.random() < 0.2 else "bf16"
        D = 128 if dt == "bf16" and rng.random() < 0.8 else 64
        B = int(rng.choice([4, 8, 16, 32, 64, 128]))
        g = int(rng.choice([1, 2, 3, 4, 5, 6, 7, 8, 12, 16]))
        Hkv = int(rng.choice([1, 2, 4, 8]))
        path = expected_path(dt, D, B, g)
        if path is None:
            continue
        S = int(rng.integers(1, 25))
        maxlen = int(rng.choice([40, 300, 1500, 5000]))
        P = 0 if rng.random() < 0.3 else B * int(rng.choice([1, 2, 3, 4, 8, 16, 32, 64]))
        if P > 2 * maxlen:
            P = 0
        ctx = rng.integers(1, maxlen + 1, size=S)
        edges = [1, B, B + 1, maxlen] + ([P, P + 1] if P else [])
        for i in range(S):
            if rng.random() < 0.3:
                ctx[i] = min(maxlen, int(rng.choice(edges)))
        np_ = -(-int(ctx.max()) // P) if P else 1
        if np_ > 1 and S * g * Hkv * np_ * (D + 32) * 4 > MAX_WORKSPACE:
            continue
        tile = path in ("mfma", "valu") and B >= 16
        width = str(rng.choice(["", "1", "2", "4"])) if tile else ""
        fused = bool(rng.random() < 0.4)
        return {"dt": dt, "D": D, "B": B, "Hq": g * Hkv, "Hkv": Hkv, "S": S, "ctx": ctx.astype(np.int64), "P": P,
                "parts": np_, "width": width, "fused": fused, "path": path}


def case_id(case: int) -> str:
    c = draw(case)
    return (f"{case}-{c['dt']}-D{c['D']}-B{c['B']}-g{c['Hq'] // c['Hkv']}-kv{c['Hkv']}-S{c['S']}-P{c['P']}"
            f"{'-w' + c['width'] if c['width'] else ''}{'-fused' if c['fused'] else ''}")
