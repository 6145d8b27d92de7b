"""Data-tree views over one flat fp32 root (oracle; test infrastructure only).

[SS-HSDP §3.2, "Data Tree"]: every tensor or tensor list is a node; a child is a
view at an offset inside its parent, its size given by its own shape; only the
root owns storage and a child reaches it through the offset accumulated along
its chain.  [SS-HSDP Appendix A, "Packing and compatibility" and Table 4]: the
planner rejects incompatible metadata, invalid geometry and storage overlap,
and every field describes the same units.

A node is a mapping with keys
  parent      -1 for a view of the root allocation, else the index of an
              EARLIER node
  offset      elements from the parent's first element
  rows, cols  view shape; ``cols`` is the contiguous (K) dimension, 1-D = 1 row
  row_stride  elements between consecutive rows (== cols when contiguous)
  is_unit     True for an update parameter (leaf of the optimisation)
  optimizer   'muon' or 'adamw' for units, None otherwise
  quantize    G mode of a region [SS-HSDP §2.1: G casts or quantises the main
              weight]: True (or 'mxfp8') = requantised to MXFP8, 'bf16' = cast
              to bfloat16, False/None = no G.  Resolved entries carry
              ``quantize`` (MXFP8) and ``cast`` (bf16) as booleans.

Reading taken where the pages are silent: the planner's error classes and their
precedence (one rule list, first failing node in index order, overlap last) are
this implementation's own; the conditions themselves are those of Table 4:
geometry, bounds, storage overlap, a Muon unit being a matrix, and MXFP8
regions covering whole 1x32 blocks along their contiguous dimension (the block
the scale belongs to, OCP-MX) in the chosen scale layout.  Restrictions that
come from one implementation's memory access (vector widths, alignment of a
strided view) are not rules of the method and are not checked here.
"""

import numpy as np


class ViewError(ValueError):
    """Raised with ``.code`` in {'ARG','TREE','BOUNDS','OVERLAP','SCHEMA'}."""

    def __init__(self, code, msg):
        super().__init__(f"{code}: {msg}")
        self.code = code


def _extent(rows, cols, row_stride):
    # number of root elements from a view's first to one past its last element
    return (rows - 1) * row_stride + cols


def resolve_views(nodes, root_numel, scale_layout="rowmajor", check_overlap=True):
    """Resolve accumulated offsets and validate the tree.

    Returns a list of dicts: the input keys plus ``abs`` (absolute element
    offset in the root) and ``extent``.  Raises ViewError on the first
    violated rule; the storage-overlap rule, checked last, is skipped when
    ``check_overlap`` is false.
    """
    if len(nodes) == 0 or root_numel <= 0:
        raise ViewError("ARG", "empty node table or root")
    out = []
    for i, nd in enumerate(nodes):
        p = int(nd["parent"])
        if p < -1 or p >= i:
            raise ViewError("TREE", f"node {i}: parent {p} is not an earlier node")
        rows, cols, off = int(nd["rows"]), int(nd["cols"]), int(nd["offset"])
        rs = int(nd["row_stride"]) if rows > 1 else cols
        if rows < 1 or cols < 1 or off < 0 or rs < cols:
            raise ViewError("SCHEMA", f"node {i}: invalid geometry")
        base = 0 if p < 0 else out[p]["abs"]
        pext = root_numel if p < 0 else out[p]["extent"]
        ext = _extent(rows, cols, rs)
        a = base + off
        if off + ext > pext or a + ext > root_numel:
            raise ViewError("BOUNDS", f"node {i}: view leaves its parent")
        is_unit = bool(nd["is_unit"])
        opt = nd.get("optimizer")
        qv = nd.get("quantize", False)
        if qv not in (None, False, True, "mxfp8", "bf16", 0, 1, 2):
            raise ViewError("SCHEMA", f"node {i}: unknown G mode {qv!r}")
        q = qv in (True, "mxfp8", 1)
        cast = qv in ("bf16", 2)
        if is_unit and opt not in ("muon", "adamw"):
            raise ViewError("SCHEMA", f"node {i}: unit without a known optimizer")
        if is_unit and opt == "muon":
            if rows < 2 or cols < 2:
                raise ViewError("SCHEMA", f"node {i}: Muon unit must be a matrix")
        if q:
            if rs != cols or cols % 32 or a % 32:
                raise ViewError("SCHEMA", f"node {i}: quantised region not block aligned")
            if scale_layout == "tile32x4" and (rows % 32 or cols % 128):
                raise ViewError("SCHEMA", f"node {i}: tile32x4 needs rows%32==0, cols%128==0")
            if scale_layout == "block32x32" and (rows % 32 or a % 1024):
                raise ViewError("SCHEMA", f"node {i}: block32x32 needs rows%32==0 and a 1024-aligned start")
        r = dict(nd)
        r.update(abs=a, extent=ext, row_stride=rs, rows=rows, cols=cols,
                 is_unit=is_unit, optimizer=opt if is_unit else None, quantize=q, cast=cast)
        out.append(r)
    if not check_overlap:
        return out
    # storage overlap, by brute force marking [SS-HSDP Appendix A, Table 4]
    for key, what in (("is_unit", "units"), ("quantize", "G regions")):
        marks = np.zeros(root_numel, dtype=np.uint8)
        for r in out:
            if not (r["quantize"] or r["cast"]) if key == "quantize" else not r[key]:
                continue
            if r["row_stride"] == r["cols"]:
                segs = [(r["abs"], r["rows"] * r["cols"])]
            else:
                segs = [(r["abs"] + i0 * r["row_stride"], r["cols"]) for i0 in range(r["rows"])]
            for s, n in segs:
                seg = marks[s:s + n]
                if seg.any():
                    raise ViewError("OVERLAP", f"two {what} share storage")
                seg[:] = 1
    return out


def unit_indices(r):
    """Flat root indices of a resolved view, shape (rows, cols), row-major."""
    i = np.arange(r["rows"], dtype=np.int64)[:, None] * r["row_stride"]
    j = np.arange(r["cols"], dtype=np.int64)[None, :]
    return r["abs"] + i + j
