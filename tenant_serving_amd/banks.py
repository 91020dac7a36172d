"""Host-side layout of packed deltas for loading ([P5] "Key Contributions" 4: the
packed delta of a module moves in one transfer; [P1] "How BitDelta Works": the base
weights stay resident, per-user deltas are swapped in).

One user's deltas of one module (a layer's linear matrices) sit back to back in one
byte buffer: per matrix its packed signs (d_out * d_in / 8 bytes, the bd_compress
layout) and then its scales, each at a 256-byte boundary, so that the views handed to
bd_apply are aligned.  The same layout serves a pinned host buffer and its device
copy; moving a module is then one copy."""
from typing import List, Sequence, Tuple

import torch

ALIGN = 256


def module_layout(shapes: Sequence[Tuple[int, int]], scale_counts: Sequence[int],
                  scale_bytes: int = 4) -> Tuple[List[Tuple[int, int]], int]:
    """(signs offset, scales offset) of each matrix and the module's total bytes."""
    off, out = 0, []
    for (d_out, d_in), n_sc in zip(shapes, scale_counts):
        s_off = off
        off += (d_out * d_in // 8 + ALIGN - 1) // ALIGN * ALIGN
        c_off = off
        off += (scale_bytes * n_sc + ALIGN - 1) // ALIGN * ALIGN
        out.append((s_off, c_off))
    return out, off


def module_views(buf: torch.Tensor, shapes, scale_counts, scale_dtype=torch.float32):
    """(signs int64[d_out][d_in/64], scales[n]) views of each matrix inside a byte buffer."""
    offs, _ = module_layout(shapes, scale_counts, torch.tensor([], dtype=scale_dtype).element_size())
    views = []
    for (s_off, c_off), (d_out, d_in), n_sc in zip(offs, shapes, scale_counts):
        signs = buf[s_off:s_off + d_out * d_in // 8].view(torch.int64).view(d_out, d_in // 64)
        esz = torch.tensor([], dtype=scale_dtype).element_size()
        scales = buf[c_off:c_off + esz * n_sc].view(scale_dtype)
        views.append((signs, scales))
    return views


def pack_module(buf: torch.Tensor, shapes, signs_list, scales_list) -> None:
    """Copies each matrix's signs and scales into its place in `buf` (any device)."""
    views = module_views(buf, shapes, [s.numel() for s in scales_list], scales_list[0].dtype)
    for (sv, cv), s, c in zip(views, signs_list, scales_list):
        sv.copy_(s.reshape(sv.shape))
        cv.copy_(c.reshape(-1))
