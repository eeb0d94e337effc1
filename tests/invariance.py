"""I-relation runner: a kernel against itself under batch-shape transforms.

The invariance relation compares the kernel with itself while only the
surrounding batch shape moves, bit for bit (atol = rtol = 0): page "[RFC]
Batch-Invariant RL Kernel Suite for Train-Inference Consistency", the
maintainer reply's relation table (I / A / P); page "docs(ws1):
batch-invariance contract RFC", the PR summary (six transform classes T1-T6).

Fixture rules followed here (page "docs(ws1): ...", section
"InvarianceFixture", requirements 1-4):

1. baseline and variant come from the same tensors; nothing is regenerated
   per case (fresh neighbour or padding rows are drawn once, from a recorded
   seed, and are never compared);
2. the row under test is extracted by integer indexing only;
3. masked rows are excluded by the runner, never by the caller;
4. each case is replayable from its manifest (workload, seed, transform and
   its parameters), whose hash is the fixture id.

Comparison is on raw 32-bit patterns, which is stricter than an all-close with
zero tolerances: -0.0 differs from +0.0 and NaN payloads must match.

Drift records name the logical token of a mismatch as (sample_id,
token_position), whatever packing, padding or chunking the variant used: the
drift report of page "[RFC] Batch-Invariant RL Kernel Suite for
Train-Inference Consistency" (its list of proposed deliverables) carries the
sequence id and token position, and page "[WS1 Test] #154 dtype pin + ...",
section "Workstream 3 - #153", compares outputs by logical-workload identity.

A batch here is a dict of row-aligned tensors -- ``x`` (logits or hidden
rows), ``targets``, ``mask`` and optionally ``grad`` -- all with the same first
dimension.  ``run(batch) -> dict`` returns row-aligned outputs (``logp``,
``lse``, ``dlogits`` ...).
"""

import hashlib
import json

import torch

TRANSFORM_NAMES = {
    "T1": "batch_population",
    "T2": "batch_position",
    "T3": "neighbour_content",
    "T4": "padding_layout",
    "T5": "execution_schedule",
    "T6": "selection_packing",
}


def fixture_id(manifest):
    blob = json.dumps(manifest, sort_keys=True, default=str).encode()
    return f"{manifest.get('operator', 'op')}-{hashlib.sha256(blob).hexdigest()[:12]}"


def take(batch, idx):
    idx = torch.as_tensor(idx, dtype=torch.int64)
    return {k: v.index_select(0, idx.to(v.device)) for k, v in batch.items()}


def cat(batches):
    keys = batches[0].keys()
    return {k: torch.cat([b[k] for b in batches], dim=0) for k in keys}


def nrows(batch):
    return next(iter(batch.values())).shape[0]


# ---------------------------------------------------------------------------
# transforms: each returns (list_of_variant_calls, row_map) where row_map[k]
# is the base row that variant row k (rows of all calls, concatenated) holds,
# or -1 for an inserted row.


def t1_population(base, size, start=0):
    n = nrows(base)
    sel = [(start + k) % n for k in range(size)]
    return [take(base, sel)], torch.tensor(sel)


def t2_position(base, seed):
    g = torch.Generator().manual_seed(seed)
    perm = torch.randperm(nrows(base), generator=g)
    return [take(base, perm)], perm


def t3_neighbours(base, keep, filler, seed):
    """Keep rows ``keep`` of the base at their positions; every other row
    gets fresh content from ``filler(n, seed)``."""
    n = nrows(base)
    fresh = filler(n, seed)
    keep = torch.as_tensor(keep, dtype=torch.int64)
    var = {k: v.clone() for k, v in fresh.items()}
    for k in var:
        var[k][keep.to(var[k].device)] = base[k][keep.to(base[k].device)]
    row_map = torch.full((n,), -1, dtype=torch.int64)
    row_map[keep] = keep
    return [var], row_map


def t4_padding(base, filler, seed, left=0, right=0, every=0):
    """Insert masked padding rows with random content and invalid targets:
    ``left`` rows before, ``right`` after, and one after every ``every``
    base rows (0 = none)."""
    n = nrows(base)
    pieces = []
    row_map = []
    k = 0
    if left:
        pieces.append(_pad_rows(filler, left, seed))
        row_map += [-1] * left
        k += 1
    step = every if every else n
    for r0 in range(0, n, step):
        r1 = min(n, r0 + step)
        pieces.append(take(base, list(range(r0, r1))))
        row_map += list(range(r0, r1))
        if every and r1 < n:
            pieces.append(_pad_rows(filler, 1, seed + 7919 * (r0 + 1)))
            row_map += [-1]
    if right:
        pieces.append(_pad_rows(filler, right, seed + 1))
        row_map += [-1] * right
    return [cat(pieces)], torch.tensor(row_map)


def _pad_rows(filler, n, seed):
    rows = filler(n, seed)
    rows["mask"] = torch.zeros_like(rows["mask"])
    rows["targets"] = torch.full_like(rows["targets"], -100)
    return rows


def t5_schedule(base, chunk):
    """Split the same rows across several launches of ``chunk`` rows."""
    n = nrows(base)
    calls = [take(base, list(range(r0, min(n, r0 + chunk)))) for r0 in range(0, n, chunk)]
    return calls, torch.arange(n)


def t6_padded_layout(base, seq_lens, s_max, filler, seed, side="right"):
    """Packed varlen rows -> a padded [B, S_max] layout flattened to rows."""
    pieces = []
    row_map = []
    off = 0
    for b, L in enumerate(seq_lens):
        pad = s_max - L
        seq = take(base, list(range(off, off + L)))
        padr = _pad_rows(filler, pad, seed + b) if pad else None
        if side == "left" and pad:
            pieces.append(padr)
            row_map += [-1] * pad
        pieces.append(seq)
        row_map += list(range(off, off + L))
        if side == "right" and pad:
            pieces.append(padr)
            row_map += [-1] * pad
        off += L
    return [cat(pieces)], torch.tensor(row_map)


def t6_compacted(base):
    """Only the active rows, passed without a mask (indexed selection) vs the
    full batch with the mask (dense with mask)."""
    act = torch.nonzero(base["mask"].to("cpu") != 0).flatten()
    var = take(base, act)
    var["mask"] = None
    return [var], act


def canonical_positions(n, seq_lens=None):
    """(sample_id, token_position) of each of ``n`` base rows, int64 [n, 2].

    With ``seq_lens`` the rows are sequences of those lengths packed back to
    back (rows past them are padding: (-1, -1)); without, every row is a
    sample of its own (position 0)."""
    pos = torch.full((n, 2), -1, dtype=torch.int64)
    if seq_lens is None:
        pos[:, 0] = torch.arange(n)
        pos[:, 1] = 0
        return pos
    off = 0
    for s, L in enumerate(seq_lens):
        L = int(L)
        hi = min(n, off + L)
        if hi > off:
            pos[off:hi, 0] = s
            pos[off:hi, 1] = torch.arange(hi - off)
        off += L
    return pos


# ---------------------------------------------------------------------------
# running and comparing


def run_calls(run, calls):
    outs = [run(c) for c in calls]
    keys = outs[0].keys()
    return {k: torch.cat([o[k] for o in outs], dim=0) for k in keys}


def _bits(t):
    t = t.detach().to("cpu").contiguous()
    if t.dtype == torch.float32:
        return t.view(torch.int32)
    if t.dtype == torch.float64:
        return t.view(torch.int64)
    return t


def compare(base_out, var_out, row_map, base_mask, manifest, positions=None):
    """Bitwise comparison of every output on the active base rows the
    variant holds.  Returns a list of drift records (empty when invariant).
    ``positions``: (sample_id, token_position) of each base row (see
    canonical_positions; default: every row its own sample)."""
    if positions is None:
        positions = canonical_positions(nrows(base_out))
    row_map = torch.as_tensor(row_map, dtype=torch.int64)
    bm = base_mask.to("cpu") != 0
    held = torch.nonzero(row_map >= 0).flatten()
    base_rows = row_map[held]
    keep = bm[base_rows]
    var_rows = held[keep]
    base_rows = base_rows[keep]
    # canonical (logical) order: ascending base row
    order = torch.argsort(base_rows)
    var_rows, base_rows = var_rows[order], base_rows[order]
    records = []
    for name in base_out:
        b = _bits(base_out[name]).index_select(0, base_rows)
        v = _bits(var_out[name]).index_select(0, var_rows)
        neq = b != v
        if not bool(neq.any()):
            continue
        bf = base_out[name].detach().to("cpu").index_select(0, base_rows).double()
        vf = var_out[name].detach().to("cpu").index_select(0, var_rows).double()
        diff = (bf - vf).abs()
        finite = torch.isfinite(diff)
        nz = torch.nonzero(neq.reshape(neq.shape[0], -1))
        r, c = int(nz[0, 0]), int(nz[0, 1])
        bad_rows = torch.unique(nz[:, 0])
        logical = positions.index_select(0, base_rows.index_select(0, bad_rows))
        records.append({
            "relation": "invariance",
            "status": "fail",
            "fixture_id": fixture_id(manifest),
            "operator": manifest.get("operator"),
            "op_class": "logprob",
            "chain_index": manifest.get("chain_index"),
            "transform": manifest.get("transform"),
            "backend": "hip",
            "arch_key": "gfx950",
            "device": manifest.get("device"),
            "dtype": "bfloat16",
            "direction": manifest.get("direction", "forward"),
            "output": name,
            "threshold": {"atol": 0.0, "rtol": 0.0},
            "max_abs_error": float(diff[finite].max()) if bool(finite.any()) else float("nan"),
            "mean_abs_error": float(diff[finite].mean()) if bool(finite.any()) else float("nan"),
            "n_mismatched": int(neq.sum()),
            "n_compared": int(neq.numel()),
            "units": "output elements",
            "first_mismatch": {"sample_id": int(positions[base_rows[r], 0]),
                               "token_position": int(positions[base_rows[r], 1]),
                               "logical_row": int(base_rows[r]), "variant_row": int(var_rows[r]),
                               "column": c},
            "n_tokens_mismatched": int(bad_rows.numel()),
            "mismatched_tokens": [[int(a), int(b)] for a, b in logical[:16].tolist()],
            "launch": manifest.get("launch"),
            "seed": manifest.get("seed"),
        })
    return records


def check(run, base, calls, row_map, manifest, base_out=None, positions=None):
    """Run baseline and variant, compare, return (records, base_out)."""
    if base_out is None:
        base_out = run(base)
    var_out = run_calls(run, calls)
    return compare(base_out, var_out, row_map, base["mask"], manifest, positions), base_out
