"""Host <-> device transfers through a pinned staging buffer.

Large copies from pageable (numpy-owned) host memory make the HIP runtime pin
the caller's pages in place, which not every system permits.  These helpers
copy through a buffer allocated as pinned memory up front, in fixed-size
chunks, so no existing host memory ever needs registering.  Plumbing only:
no arithmetic of the method happens here.
"""

from __future__ import annotations

import numpy as np

CHUNK_BYTES = 32 << 20

_staging = None


def _stage(nbytes):
    import torch
    global _staging
    if _staging is None or _staging.numel() < nbytes:
        _staging = torch.empty(max(nbytes, CHUNK_BYTES), dtype=torch.uint8, pin_memory=True)
    return _staging


def _bytes_view(t):
    import torch
    return t.view(-1).view(torch.uint8)


def upload_bytes(arr, shape, dtype, device="cuda"):
    """Copy the raw bytes of a contiguous numpy array into a new device
    tensor of ``shape`` and torch ``dtype`` (same total size)."""
    import torch
    arr = np.ascontiguousarray(arr)
    dst = torch.empty(shape, dtype=dtype, device=device)
    n = arr.nbytes
    if n == 0:
        return dst
    assert dst.numel() * dst.element_size() == n, "size mismatch"
    src = torch.from_numpy(arr.reshape(-1).view(np.uint8))
    flat = _bytes_view(dst)
    buf = _stage(min(n, CHUNK_BYTES))
    for off in range(0, n, CHUNK_BYTES):
        m = min(CHUNK_BYTES, n - off)
        buf[:m].copy_(src[off:off + m])
        flat[off:off + m].copy_(buf[:m])
    torch.cuda.current_stream(dst.device).synchronize()
    return dst


def download_bytes(t):
    """Raw bytes of a contiguous device tensor as a numpy uint8 array."""
    import torch
    t = t.contiguous()
    n = t.numel() * t.element_size()
    out = np.empty(n, dtype=np.uint8)
    if n == 0:
        return out
    flat = _bytes_view(t)
    dst = torch.from_numpy(out)
    buf = _stage(min(n, CHUNK_BYTES))
    for off in range(0, n, CHUNK_BYTES):
        m = min(CHUNK_BYTES, n - off)
        buf[:m].copy_(flat[off:off + m])
        torch.cuda.current_stream(t.device).synchronize()
        dst[off:off + m].copy_(buf[:m])
    return out


def upload_bf16_bits(bits, device="cuda"):
    """uint16 bfloat16 bit patterns -> device bfloat16 tensor."""
    import torch
    return upload_bytes(bits, bits.shape, torch.bfloat16, device)


def upload_f32(arr, device="cuda"):
    import torch
    arr = np.ascontiguousarray(arr, dtype=np.float32)
    return upload_bytes(arr, arr.shape, torch.float32, device)


def download_f64(t):
    """Device bf16/fp32 tensor -> float64 numpy array (exact)."""
    import torch
    raw = download_bytes(t)
    if t.dtype == torch.bfloat16:
        vals = (raw.view(np.uint16).astype(np.uint32) << 16).view(np.float32)
    elif t.dtype == torch.float32:
        vals = raw.view(np.float32)
    else:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return vals.astype(np.float64).reshape(tuple(t.shape))
