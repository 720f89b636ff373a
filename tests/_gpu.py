"""Helpers for the GPU parity tests: upload, error metric, routing comparison."""
import numpy as np
import torch

import oracle
import quantized_sparse_moe_amd as qm

# Max relative error of the fp32 output per token, max_j |y - y_ref| / max_j |y_ref|,
# against the float64 oracle (fp32 accumulation, bf16 activations).
TOL = 2e-3


def xdev(x_bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x_bits).view(np.int16)).cuda()


def rel_err(y, ref) -> np.ndarray:
    y = np.asarray(y, dtype=np.float64).reshape(ref.shape)
    den = np.abs(ref).max(axis=-1)
    den = np.where(den > 0, den, 1.0)
    return np.abs(y - ref).max(axis=-1) / den


def near_tie_ok(gpu_ids_t, key_t, k, tau_rel=1e-5):
    """A routing difference is accepted only where the float64 keys of the
    experts involved lie within tau of the k-th key (a certified near-tie):
    fp32 and float64 keys can order such experts differently."""
    order = sorted(range(len(key_t)), key=lambda e: (-key_t[e], e))
    kth = key_t[order[k - 1]]
    tau = tau_rel * (1.0 + abs(kth))
    ref_set, gpu_set = set(order[:k]), set(int(e) for e in gpu_ids_t)
    if len(gpu_set) != k:
        return False
    for e in ref_set ^ gpu_set:
        if abs(key_t[e] - kth) > tau:
            return False
    # order within the selection: adjacent keys must be non-increasing up to tau
    kg = [key_t[int(e)] for e in gpu_ids_t]
    return all(kg[i] >= kg[i + 1] - tau_rel * (1 + abs(kg[i])) for i in range(k - 1))


def check_topk_ids(gpu_ids: np.ndarray, ref_ids: np.ndarray, key: np.ndarray, k: int, max_ties: int = 2) -> int:
    """GPU ids equal the oracle's except at certified near-ties; returns their count."""
    ties = 0
    for t in range(gpu_ids.shape[0]):
        if not np.array_equal(gpu_ids[t], ref_ids[t]):
            assert near_tie_ok(gpu_ids[t], key[t], k), f"token {t}: gpu {gpu_ids[t]} oracle {ref_ids[t]}"
            ties += 1
    assert ties <= max_ties, f"{ties} near-tie tokens"
    return ties


def stable_sort_perm(ids: np.ndarray, E: int):
    flat = ids.reshape(-1)
    perm = np.argsort(flat, kind="stable").astype(np.int32)
    off = np.zeros(E + 1, np.int64)
    off[1:] = np.cumsum(np.bincount(flat, minlength=E))
    return off, perm


def run_staged(dl, x_bits, token_ids=None):
    xd = xdev(x_bits)
    tok = None if token_ids is None else torch.from_numpy(np.ascontiguousarray(token_ids)).cuda()
    ws = dl.workspace(x_bits.shape[0])
    st = qm.forward_staged(dl, xd, tok, out_dtype="f32", ws=ws)
    out_f32 = qm.forward(dl, xd, tok, out_dtype="f32", ws=ws)
    out_bf16 = qm.forward(dl, xd, tok, out_dtype="bf16", ws=ws)
    torch.cuda.synchronize()
    assert qm.device_error(ws) == 0
    return st, out_f32, out_bf16, ws
