"""The library's own admission rules, beside the method's.

The oracle (oracle/views.py) checks what the method fixes: tree, geometry,
bounds, overlap, a Muon unit being a matrix, MXFP8 regions made of whole 1x32
blocks in the chosen scale layout.  libsshdp.so additionally refuses views its
kernels cannot address with their vector accesses (the SCHEMA rules of
include/sshdp.h that the pages do not give):

* a Muon unit's first element, row stride and column count are multiples of 4
  (16-byte loads and stores of fp32 rows), and both edges are at most
  4194176 (a 256-row bf16 operand panel must span < 2^31 bytes);
* a BF16-cast region is contiguous, with its first element and column count
  multiples of 8 (16-byte stores of bf16);
* a G region (either kind) has at most 2^30 columns, an MXFP8 region fewer
  than 2^31 rows (32-bit work-item fields).

``expected_code`` combines both lists in the planner's order: nodes are
checked in index order; within a node the tree, geometry and bounds rules come
first and every later rule (the method's or the library's) answers SCHEMA;
storage overlap is checked last, over the whole table.
"""

from oracle.views import ViewError, resolve_views

MAX_EDGE = 4194176


def library_rule_violated(r):
    """True when a resolved node breaks one of the library-only rules."""
    if r["is_unit"] and r["optimizer"] == "muon":
        if r["abs"] % 4 or r["row_stride"] % 4 or r["cols"] % 4:
            return True
        if r["rows"] > MAX_EDGE or r["cols"] > MAX_EDGE:
            return True
    if r["cast"] and (r["row_stride"] != r["cols"] or r["cols"] % 8 or r["abs"] % 8):
        return True
    if (r["cast"] or r["quantize"]) and r["cols"] > (1 << 30):
        return True
    if r["quantize"] and r["rows"] > 0x7FFFFFFF:
        return True
    return False


def expected_code(nodes, root_numel, layout="rowmajor"):
    """Error class the planner must return for this table (None = accepted)."""
    for k in range(len(nodes)):
        try:
            res = resolve_views(nodes[:k + 1], root_numel, layout, check_overlap=False)
        except ViewError as e:
            return e.code
        if library_rule_violated(res[k]):
            return "SCHEMA"
    try:
        resolve_views(nodes, root_numel, layout)
    except ViewError as e:
        return e.code
    return None
