"""Poisoned outputs and a self-classifying report for the pack -> unpack round trip.

Every output buffer is filled with an all-ones bit pattern (NaN for bf16 and fp32, an
out-of-range candidate for hard indices) on the launch stream before the library writes it, so
an element the kernels leave unwritten cannot pass for a correct value.  When the dense output
of an unpack disagrees with the selection of the weights by the hard mask, `classify` says what
the wrong elements hold:

  poison          the unpack never wrote the element (the poison is still there);
  zero_for_kept   +0.0 where the hard mask keeps the weight (a field read as another position);
  weight_dropped  the element's own weight where the mask drops it (same cause);
  other_weight    another weight of the same group of M (a kept value put at the wrong place);
  foreign         none of these: a value from outside the group, i.e. the packed values read
                  were not the ones written, or the buffer was written again afterwards;

and where they are: flat element span, the 16-byte store slots and 256-thread blocks of the
flat unpack grid that own them, the 4 KB pages of the buffer, and the data pointers of every
buffer with the pointers of the previous matrix's buffers (reuse of freed blocks by the caching
allocator).  The report is printed and, when NM_DIAG_DIR is set, written there as JSON.
"""
import json
import os
import time

import numpy as np
import torch

POISON16 = -1  # 0xFFFF as int16
POISON32 = -1  # 0xFFFFFFFF as int32


def bits(t):
    """Integer view of a bf16 / fp32 tensor (integer tensors as they are)."""
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16)
    if t.dtype == torch.float32:
        return t.view(torch.int32)
    return t


def poisoned(shape, dtype, device):
    """A tensor of `shape` whose every byte is 0xFF (filled on the current stream)."""
    t = torch.empty(shape, dtype=dtype, device=device)
    t.view(torch.uint8).fill_(0xFF)
    return t


def pack_outputs(w, n, m, wpr, with_hard=True):
    rows, cols = w.shape
    values = poisoned((rows, cols // m * n), w.dtype, w.device)
    indices = poisoned((rows, wpr), torch.int32, w.device)
    hard = poisoned((rows, cols // m), torch.uint8, w.device) if with_hard else None
    return values, indices, hard


def classify(w, dense, want, m):
    """numpy classification of the wrong elements of `dense` (bit patterns) against `want`."""
    got = bits(dense).cpu().numpy().reshape(-1)
    ref = bits(want).cpu().numpy().reshape(-1)
    wb = bits(w).cpu().numpy().reshape(-1)
    bad = np.flatnonzero(got != ref)
    out = {"wrong": int(bad.size)}
    if bad.size == 0:
        return out
    g = got[bad]
    group = (bad // m) * m
    in_group = np.zeros(bad.size, bool)
    for j in range(m):
        in_group |= g == wb[group + j]
    poison = g == (POISON16 if dense.dtype == torch.bfloat16 else POISON32)
    zero_for_kept = (g == 0) & (ref[bad] != 0)
    weight_dropped = (g == wb[bad]) & (ref[bad] == 0)
    other = in_group & ~weight_dropped & ~zero_for_kept & ~poison
    foreign = ~(poison | zero_for_kept | weight_dropped | other)
    out.update({k: int(v.sum()) for k, v in (("poison", poison), ("zero_for_kept", zero_for_kept),
                                             ("weight_dropped", weight_dropped), ("other_weight", other),
                                             ("foreign", foreign))})
    esz = dense.element_size()
    cols = dense.shape[1]
    slots = bad * esz // 16
    blocks = slots // 256
    lines = (dense.data_ptr() + bad * esz) // 128  # absolute 128-byte lines
    ul, per_line = np.unique(lines, return_counts=True)
    out.update({
        "lines_128B": int(ul.size), "lines_fully_wrong": int((per_line == 128 // esz).sum()),
        "first_byte_mod_4096": int((dense.data_ptr() + bad[0] * esz) % 4096),
        "end_byte_mod_4096": int((dense.data_ptr() + (bad[-1] + 1) * esz) % 4096),
        "runs": _runs(bad)[:32],
        "high_byte_hist": np.bincount(((g.astype(np.int64) & 0xFFFF) >> 8), minlength=256).nonzero()[0].tolist()[:64],
    })
    out.update({
        "first": [int(bad[0] // cols), int(bad[0] % cols)], "last": [int(bad[-1] // cols), int(bad[-1] % cols)],
        "span_elements": int(bad[-1] - bad[0] + 1),
        "store_slots_16B": [int(slots.min()), int(slots.max()), int(np.unique(slots).size)],
        "blocks_256": [int(blocks.min()), int(blocks.max()), int(np.unique(blocks).size)],
        "block_mod_8_counts": np.bincount(np.unique(blocks) % 8, minlength=8).tolist(),
        "buffer_pages_4K": sorted({int(x) for x in (bad * esz // 4096)})[:64],
        "abs_pages_4K": sorted({int(x) for x in ((dense.data_ptr() + bad * esz) // 4096)})[:64],
        "first_values": [[int(i), int(got[i]) & 0xFFFFFFFF, int(ref[i]) & 0xFFFFFFFF] for i in bad[:16]],
    })
    return out


def group_dump(w, dense, want, values, indices, m, n, limit=4096):
    """Per wrong group (up to `limit`): the observed and expected dense group, the group's kept
    values and index fields as written by the pack, and where each observed value occurs among
    the packed values of the same row (the value the unpack must have read, and from where)."""
    if m != 4 or n != 2 or dense.dtype != torch.bfloat16:
        return []
    got = bits(dense).cpu().numpy().view(np.uint16)
    ref = bits(want).cpu().numpy().view(np.uint16)
    rows, cols = got.shape
    gpr = cols // m
    g_got = got.reshape(rows, gpr, m)
    g_ref = ref.reshape(rows, gpr, m)
    bad = np.argwhere((g_got != g_ref).any(-1))[:limit]
    vals = bits(values).cpu().numpy().view(np.uint16).reshape(rows, gpr, n)
    idx_bytes = indices.cpu().numpy().view(np.uint8).reshape(rows, -1)
    out = []
    for r, q in bad:
        r, q = int(r), int(q)
        byte = int(idx_bytes[r, q // 2])
        fields = [(byte >> (2 * (2 * (q % 2) + t))) & 3 for t in range(n)]
        row_vals = vals[r].reshape(-1)
        where = []
        for v in g_got[r, q]:
            hits = np.flatnonzero(row_vals == v)[:3] if v != 0 else []
            where.append([int(h) for h in hits])
        out.append({"row": r, "group": q, "got": [int(x) for x in g_got[r, q]], "want": [int(x) for x in g_ref[r, q]],
                    "values": [int(x) for x in vals[r, q]], "index_byte": byte, "fields": fields,
                    "got_found_in_row_values_at": where})
    return out


def _runs(idx):
    """[start, length] of the maximal runs of consecutive indices."""
    if idx.size == 0:
        return []
    cut = np.flatnonzero(np.diff(idx) != 1) + 1
    starts = np.concatenate([[0], cut])
    ends = np.concatenate([cut, [idx.size]])
    return [[int(idx[a]), int(b - a)] for a, b in zip(starts, ends)]


def report(tag, w, values, indices, hard, dense, want, m, rechecks, pointers_prev=None, n=2):
    """Print (and write when NM_DIAG_DIR is set) the classification of a failed round trip."""
    doc = {"tag": tag, "time": time.time(), "shape": list(w.shape), "dtype": str(w.dtype),
           "pointers": {k: int(t.data_ptr()) for k, t in (("w", w), ("values", values), ("indices", indices),
                                                           ("dense", dense)) if t is not None},
           "pointers_prev": pointers_prev or {},
           "classification": classify(w, dense, want, m)}
    try:
        st = torch.cuda.memory_stats(dense.device)
        doc["allocator"] = {k: st.get(k) for k in ("num_alloc_retries", "num_device_alloc", "num_device_free",
                                                   "segment.all.current", "reserved_bytes.all.current",
                                                   "num_sync_all_streams")}
    except Exception as e:
        doc["allocator_error"] = repr(e)
    try:
        doc["groups"] = group_dump(w, dense, want, values, indices, m, n)
    except Exception as e:  # the dump must never hide the classification
        doc["groups_error"] = repr(e)
    doc["reused_from_prev"] = sorted(k for k, p in doc["pointers"].items()
                                     if p in set((pointers_prev or {}).values()))
    doc.update(rechecks)
    line = json.dumps(doc)
    short = {k: v for k, v in doc.items() if k != "groups"}
    short["groups_first"] = doc.get("groups", [])[:6]
    print("ROUND TRIP DIAGNOSIS", json.dumps(short), flush=True)
    d = os.environ.get("NM_DIAG_DIR")
    if d:
        os.makedirs(d, exist_ok=True)
        with open(os.path.join(d, f"roundtrip_{int(doc['time'] * 1000)}.json"), "w") as f:
            f.write(line + "\n")
    return doc
