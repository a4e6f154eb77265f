"""Helpers for GPU parity tests: moving seeded numpy inputs to the device and
running stages through the Python binding of the C ABI."""
import numpy as np
import pytest
import torch

import indexer_top_kv_amd as ech

TOL_BF16 = 1e-3   # logits tolerance for bf16 keys (relative)
TOL_FP8 = 2e-2    # logits tolerance for fp8 keys (relative)


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip('no GPU visible')
    torch.cuda.set_device(0)


def dev(x: np.ndarray) -> torch.Tensor:
    x = np.ascontiguousarray(x)
    if x.dtype == np.uint16:
        x = x.view(np.int16)
    return torch.from_numpy(x).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()


def rel_err(gpu: np.ndarray, ref: np.ndarray) -> np.ndarray:
    """Elementwise |g - o| / max(|o|, 1e-2 * max_t |o_t|) for one row."""
    ref = np.asarray(ref, np.float64)
    if ref.size == 0:
        return np.zeros(0)
    floor = 1e-2 * np.abs(ref).max()
    den = np.maximum(np.abs(ref), floor if floor > 0 else 1.0)
    return np.abs(np.asarray(gpu, np.float64) - ref) / den


def run_logits(q_bits, w, key_bits, scale, tok0, lens, ld=None, fill=np.nan):
    R = q_bits.shape[0]
    max_len = int(max(lens)) if len(lens) else 0
    ld = ld or max(4, ((max_len + 3) // 4) * 4)
    out = torch.full((R, ld), float(fill), dtype=torch.float32, device='cuda')
    ech.ech_index_logits(dev(q_bits), dev(w), dev(key_bits), None if scale is None else dev(scale),
                         dev(np.asarray(tok0, np.int64)), dev(np.asarray(lens, np.int32)), max_len, out)
    torch.cuda.synchronize()
    return host(out)


def run_topk(logits: np.ndarray, lens, k: int, theta=None):
    R = logits.shape[0]
    ld = logits.shape[1]
    assert ld % 4 == 0
    max_len = int(max(lens)) if len(lens) else 0
    L = dev(logits.astype(np.float32))
    ws = torch.empty(ech.ech_topk_ws_bytes(R, max_len, k), dtype=torch.uint8, device='cuda')
    ws.fill_(0x5a)   # the workspace carries no state between calls: any contents will do
    idx = torch.full((R, k), -7, dtype=torch.int32, device='cuda')
    kth = torch.full((R,), 123.0, dtype=torch.float32, device='cuda')
    th_in = None if theta is None else dev(np.asarray(theta, np.float32))
    th_out = torch.full((R,), -5.0, dtype=torch.float32, device='cuda')
    ech.ech_topk(L, dev(np.asarray(lens, np.int32)), max_len, k, th_in, th_out, idx, kth, ws)
    torch.cuda.synchronize()
    return host(idx), host(kth), host(th_out)
