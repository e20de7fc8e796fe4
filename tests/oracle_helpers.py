"""Tiny hand-shaped problems for pinning the oracle (no generator, no HIP)."""
import numpy as np
import torch


def tiny_problem(T=64, Hq=4, Hkv=2, D=16, P=16, S=4, seed=0, sel=None, q_scale=1.0):
    N = T // P
    rng = np.random.default_rng(seed)
    gen = torch.Generator().manual_seed(seed)
    q = (torch.randn((T, Hq, D), generator=gen) * q_scale).to(torch.bfloat16)
    k = torch.randn((N, Hkv, P, D), generator=gen).to(torch.float8_e4m3fn)
    v = torch.randn((N, Hkv, P, D), generator=gen).to(torch.float8_e4m3fn)
    # dequantised values stay on the workloads' scale (|K|, |V| <~ 4.5): the bf16
    # output's own rounding (2^-8 relative) then stays inside the 2e-2 bound
    scales = rng.uniform(0.05, 1.0, size=(2, N, Hkv)).astype(np.float32)
    if sel is None:
        sel = np.full((Hkv, T, S), -1, dtype=np.int32)
        for h in range(Hkv):
            for t in range(T):
                p = t // P
                cand = rng.permutation(p + 1)[: min(S, p + 1)]
                sel[h, t, : cand.size] = np.sort(cand)
    return {
        "q_bits": q.view(torch.int16).numpy().view(np.uint16),
        "k_codes": k.view(torch.uint8).numpy(),
        "v_codes": v.view(torch.uint8).numpy(),
        "scales": scales,
        "sel_pages": sel,
    }


def torch_dense_reference(inp, allowed):
    """fp64 masked attention through torch SDPA; allowed: bool [H_kv][T][T]."""
    qb, kc, vc, sc = inp["q_bits"], inp["k_codes"], inp["v_codes"], inp["scales"]
    T, Hq, D = qb.shape
    N, Hkv, P, _ = kc.shape
    G = Hq // Hkv
    q = torch.from_numpy(qb.view(np.int16)).view(torch.bfloat16).double()
    k = torch.from_numpy(kc).view(torch.float8_e4m3fn).double() * torch.from_numpy(sc[0]).double()[:, :, None, None]
    v = torch.from_numpy(vc).view(torch.float8_e4m3fn).double() * torch.from_numpy(sc[1]).double()[:, :, None, None]
    k = k.permute(1, 0, 2, 3).reshape(Hkv, N * P, D)     # token j = u*P + c
    v = v.permute(1, 0, 2, 3).reshape(Hkv, N * P, D)
    kq = k.repeat_interleave(G, dim=0)                   # Q head hq -> KV head hq // G
    vq = v.repeat_interleave(G, dim=0)
    mask = torch.from_numpy(allowed).repeat_interleave(G, dim=0)
    out = torch.nn.functional.scaled_dot_product_attention(
        q.transpose(0, 1), kq, vq, attn_mask=mask)
    return out.transpose(0, 1).numpy()                    # [T][H_q][D]
