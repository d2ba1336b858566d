"""An independent numpy rendering of the documented device blob layout (format
only: it moves bytes and nibbles, computes nothing of the method), shared by
the CPU and GPU layout tests."""
import numpy as np

import oracle as O


def numpy_prepack(canon, H, I, g, fmt=O.FMT_SYM):
    """Independent rendering of the documented device layout (format only)."""
    sec = O.blob_sections(canon, H, I, g, fmt)
    gq, uq, dq, gs, us, ds = sec[:6]
    out = np.zeros_like(canon)

    def relayout(chunk):   # 16 canonical bytes -> 16 device bytes
        w = chunk.view(np.uint32)
        o = np.zeros(4, np.uint32)
        for i in range(4):
            o |= ((w >> (8 * i)) & 0xF) << (4 * i)
            o |= ((w >> (8 * i + 4)) & 0xF) << (16 + 4 * i)
        return o[[0, 2, 1, 3]].view(np.uint8)   # elements 0-7, 16-23, 8-15, 24-31

    o = 0
    for b in range(I // 32):
        for c in range(H // 32):
            for r in range(64):
                src = (gq if r < 32 else uq)[32 * b + (r & 31), 16 * c:16 * c + 16]
                out[o:o + 16] = relayout(src)
                o += 16
    o = -(-o // 256) * 256
    for b in range(H // 64):
        for c in range(I // 32):
            for r in range(64):
                out[o:o + 16] = relayout(dq[64 * b + r, 16 * c:16 * c + 16])
                o += 16
    o = -(-o // 256) * 256
    v = out[o:].view(np.uint16)
    j = 0
    for b in range(I // 32):
        for G in range(H // g):
            for r in range(64):
                v[j] = (gs if r < 32 else us)[32 * b + (r & 31), G]
                j += 1
    o2 = -(-(o + 2 * j) // 256) * 256
    v = out[o2:].view(np.uint16)
    j = 0
    for b in range(H // 64):
        for G in range(I // g):
            for r in range(64):
                v[j] = ds[64 * b + r, G]
                j += 1
    if fmt == O.FMT_ZP:
        # zero points in the scales' order, one byte each
        gz, uz, dz = sec[6:]
        o3 = -(-(o2 + 2 * j) // 256) * 256
        j = 0
        for b in range(I // 32):
            for G in range(H // g):
                for r in range(64):
                    out[o3 + j] = (gz if r < 32 else uz)[32 * b + (r & 31), G]
                    j += 1
        o4 = -(-(o3 + j) // 256) * 256
        j = 0
        for b in range(H // 64):
            for G in range(I // g):
                for r in range(64):
                    out[o4 + j] = dz[64 * b + r, G]
                    j += 1
    return out
