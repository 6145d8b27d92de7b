"""ctypes binding of libsshdp.so (argument marshalling only).

Every call forwards to the C ABI declared in include/sshdp.h; no step of the
update phase runs in Python.  Device buffers are passed as integer addresses
(or any object with ``data_ptr()``, e.g. a torch tensor); streams as the
integer hipStream_t handle (``torch.cuda.current_stream().cuda_stream``) or
None for the default stream.  Loading fails loudly if the library has not been
built: there is no fallback implementation.
"""

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsshdp.so")

OK, ERR_ARG, ERR_TREE, ERR_BOUNDS, ERR_OVERLAP, ERR_SCHEMA, ERR_ALIGN, ERR_WORKSPACE, ERR_HIP, ERR_STATE, \
    ERR_SCRATCH = 0, -1, -2, -3, -4, -5, -6, -7, -8, -9, -10
ERROR_NAMES = {ERR_ARG: "ARG", ERR_TREE: "TREE", ERR_BOUNDS: "BOUNDS", ERR_OVERLAP: "OVERLAP",
               ERR_SCHEMA: "SCHEMA", ERR_ALIGN: "ALIGN", ERR_WORKSPACE: "WORKSPACE", ERR_HIP: "HIP",
               ERR_STATE: "STATE", ERR_SCRATCH: "SCRATCH"}
NOALLOC_SCRATCH_BYTES = 64 << 20    # SSHDP_NOALLOC_SCRATCH_BYTES
OPT = {None: 0, "muon": 1, "adamw": 2}
LAYOUT = {"rowmajor": 0, "tile32x4": 1, "block32x32": 2}
PLAN_HOST_ONLY = 1
# Newton-Schulz tile policy: planner default, all 128 x 128, or 256 x 256 over every 256-aligned block
NS_TILES = {"auto": 0, "small": 2, "large": 4}
# Gram operand: planner default (128-tile Grams read X^T), or X row-major for every Gram
NS_GRAM = {"auto": 0, "nt": 8}
NS_STREAMS = {"auto": 0, "one": 16}
ABI_VERSION = 6                     # SSHDP_ABI_VERSION of the header this binding follows
PROF_CLASSES = ["momentum", "norm", "ns_gram", "ns_poly", "ns_update", "adamw", "adamw_requant", "requant",
                "ns_phase", "cast_bf16", "lane0_gram", "lane0_poly", "lane0_update", "lane0_update_last"]
# node["quantize"]: False/None (no G), True or "mxfp8" (MXFP8 codes + scales), "bf16" (bfloat16 cast)
GMODE = {None: 0, False: 0, True: 1, "mxfp8": 1, "bf16": 2}


class SshdpError(RuntimeError):
    def __init__(self, code, what):
        self.code = code
        self.name = ERROR_NAMES.get(code, str(code))
        super().__init__(f"{what}: {self.name} ({_status_string(code)})")


class Node(ctypes.Structure):
    _fields_ = [("parent", ctypes.c_int32), ("is_unit", ctypes.c_int32), ("offset", ctypes.c_int64),
                ("rows", ctypes.c_int64), ("cols", ctypes.c_int64), ("row_stride", ctypes.c_int64),
                ("optimizer", ctypes.c_int32), ("quantize", ctypes.c_int32)]


class PlanOpts(ctypes.Structure):
    _fields_ = [("ns_steps", ctypes.c_int32), ("ns_a", ctypes.c_float), ("ns_b", ctypes.c_float),
                ("ns_c", ctypes.c_float), ("ns_eps", ctypes.c_float), ("scale_layout", ctypes.c_int32),
                ("nesterov", ctypes.c_int32), ("muon_scale_mode", ctypes.c_int32), ("flags", ctypes.c_uint32)]


class MuonHP(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_float), ("momentum", ctypes.c_float), ("weight_decay", ctypes.c_float)]


class AdamWHP(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_float), ("beta1", ctypes.c_float), ("beta2", ctypes.c_float),
                ("eps", ctypes.c_float), ("weight_decay", ctypes.c_float)]


class Buffers(ctypes.Structure):
    _fields_ = [("w_main", ctypes.c_void_p), ("grad", ctypes.c_void_p), ("mom", ctypes.c_void_p),
                ("adam_v", ctypes.c_void_p), ("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("w_bf16", ctypes.c_void_p)]


class PlanStats(ctypes.Structure):
    _fields_ = [("root_numel", ctypes.c_int64), ("scale_bytes", ctypes.c_int64),
                ("workspace_bytes", ctypes.c_int64), ("n_nodes", ctypes.c_int32), ("n_units", ctypes.c_int32),
                ("n_muon_units", ctypes.c_int32), ("n_adamw_units", ctypes.c_int32),
                ("n_quant_regions", ctypes.c_int32), ("n_groups", ctypes.c_int32),
                ("muon_elems", ctypes.c_int64), ("adamw_elems", ctypes.c_int64), ("quant_elems", ctypes.c_int64),
                ("fused_quant_elems", ctypes.c_int64), ("ns_flops", ctypes.c_double),
                ("ns_tile_flops", ctypes.c_double), ("cast_elems", ctypes.c_int64), ("n_cast_regions", ctypes.c_int32),
                ("pad_", ctypes.c_int32)]


class GroupInfo(ctypes.Structure):
    _fields_ = [("r", ctypes.c_int32), ("c", ctypes.c_int32), ("r_pad", ctypes.c_int32),
                ("c_pad", ctypes.c_int32), ("n_units", ctypes.c_int32), ("tile", ctypes.c_int32),
                ("tile_gram", ctypes.c_int32), ("gram256", ctypes.c_int32), ("upd256_rows", ctypes.c_int32),
                ("upd256_cols", ctypes.c_int32), ("gram_kmajor", ctypes.c_int32),
                ("split_b", ctypes.c_int32), ("lane", ctypes.c_int32)]


# every symbol include/sshdp.h declares, with its argument and return types
_P = ctypes.c_void_p
SIGNATURES = {
    "sshdp_abi_version": ([], ctypes.c_int),
    "sshdp_status_string": ([ctypes.c_int], ctypes.c_char_p),
    "sshdp_default_opts": ([ctypes.POINTER(PlanOpts)], ctypes.c_int),
    "sshdp_plan_views": ([ctypes.POINTER(Node), ctypes.c_int32, ctypes.c_int64, ctypes.POINTER(PlanOpts),
                          ctypes.POINTER(_P)], ctypes.c_int),
    "sshdp_plan_info": ([_P, ctypes.POINTER(PlanStats)], ctypes.c_int),
    "sshdp_plan_group": ([_P, ctypes.c_int32, ctypes.POINTER(GroupInfo)], ctypes.c_int),
    "sshdp_plan_node": ([_P, ctypes.c_int32, ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_int32)],
                        ctypes.c_int),
    "sshdp_plan_destroy": ([_P], None),
    "sshdp_update_muon": ([_P, ctypes.POINTER(Buffers), ctypes.POINTER(MuonHP), _P, ctypes.c_size_t, _P],
                          ctypes.c_int),
    "sshdp_update_adamw": ([_P, ctypes.POINTER(Buffers), ctypes.POINTER(AdamWHP), ctypes.c_int64, _P],
                           ctypes.c_int),
    "sshdp_requant_mxfp8": ([_P, _P, _P, _P, _P], ctypes.c_int),
    "sshdp_cast_bf16": ([_P, _P, _P, _P], ctypes.c_int),
    "sshdp_rs_reduce": ([_P, ctypes.c_int32, ctypes.c_int32, _P, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64,
                         ctypes.c_uint64, ctypes.c_int64, _P], ctypes.c_int),
    "sshdp_rs_accumulate": ([_P, ctypes.c_int32, ctypes.c_int32, _P, ctypes.c_int64, ctypes.c_int32, _P],
                            ctypes.c_int),
    "sshdp_update_step": ([_P, ctypes.POINTER(Buffers), ctypes.POINTER(MuonHP), ctypes.POINTER(AdamWHP),
                           ctypes.c_int64, _P, ctypes.c_size_t, _P], ctypes.c_int),
    "sshdp_update_step_noalloc": ([_P, ctypes.POINTER(Buffers), ctypes.POINTER(MuonHP), ctypes.POINTER(AdamWHP),
                                   ctypes.c_int64, _P], ctypes.c_int),
    "sshdp_gemm_bf16_nt": ([_P, _P, _P, _P, _P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                            ctypes.c_float, ctypes.c_float, ctypes.c_int32, _P], ctypes.c_int),
    "sshdp_ns_executed": ([_P, _P, ctypes.c_size_t, ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_double),
                           _P], ctypes.c_int),
    "sshdp_profile_enable": ([_P, ctypes.c_int32], ctypes.c_int),
    "sshdp_profile_read": ([_P, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64)], ctypes.c_int),
}

_lib = None


def lib():
    """The loaded libsshdp.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with `python -m mxfp8_weight_repack_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in SIGNATURES.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = res
        if L.sshdp_abi_version() != ABI_VERSION:
            raise ImportError(f"{LIB_PATH} has ABI {L.sshdp_abi_version()}, the binding expects {ABI_VERSION}: rebuild it")
        _lib = L
    return _lib


def _status_string(code):
    try:
        return lib().sshdp_status_string(code).decode()
    except Exception:  # pragma: no cover - only while reporting another error
        return "?"


def _check(code, what):
    if code != OK:
        raise SshdpError(code, what)


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(s):
    if s is None:
        return None
    if isinstance(s, int):
        return s
    return s.cuda_stream


def default_opts():
    o = PlanOpts()
    _check(lib().sshdp_default_opts(ctypes.byref(o)), "sshdp_default_opts")
    return o


def _gmode(q):
    try:
        return GMODE[q]
    except (KeyError, TypeError):
        return int(q) if isinstance(q, int) else 99


def node_array(nodes):
    arr = (Node * len(nodes))()
    for i, n in enumerate(nodes):
        arr[i] = Node(int(n["parent"]), int(bool(n["is_unit"])), int(n["offset"]), int(n["rows"]),
                      int(n["cols"]), int(n["row_stride"]), OPT.get(n.get("optimizer"), 99),
                      _gmode(n.get("quantize")))
    return arr


class Plan:
    """A resolved data tree (sshdp_plan_views) and its tables."""

    def __init__(self, nodes, root_numel, layout="rowmajor", ns_steps=5, ns_a=3.4445, ns_b=-4.7750, ns_c=2.0315,
                 ns_eps=1e-7, nesterov=False, scale_mode=0, host_only=False, ns_tiles="auto", ns_gram="auto",
                 ns_streams="auto"):
        o = default_opts()
        o.ns_steps, o.ns_a, o.ns_b, o.ns_c, o.ns_eps = ns_steps, ns_a, ns_b, ns_c, ns_eps
        o.scale_layout = LAYOUT[layout]
        o.nesterov = int(bool(nesterov))
        o.muon_scale_mode = scale_mode
        # an unknown policy sets both tile flags, which the library rejects (ARG)
        # (an unknown gram or stream value sets a flag bit the library does not define: ARG as well)
        o.flags = (PLAN_HOST_ONLY if host_only else 0) | NS_TILES.get(ns_tiles, 6) | NS_GRAM.get(ns_gram, 1 << 30) \
            | NS_STREAMS.get(ns_streams, 1 << 30)
        self._nodes = node_array(nodes)
        self._h = ctypes.c_void_p()
        self.layout = layout
        _check(lib().sshdp_plan_views(self._nodes, len(nodes), int(root_numel), ctypes.byref(o),
                                      ctypes.byref(self._h)), "sshdp_plan_views")

    @property
    def handle(self):
        if not self._h:
            raise ValueError("plan destroyed")
        return self._h

    def stats(self):
        s = PlanStats()
        _check(lib().sshdp_plan_info(self.handle, ctypes.byref(s)), "sshdp_plan_info")
        return {k: getattr(s, k) for k, _ in PlanStats._fields_}

    def group(self, g):
        gi = GroupInfo()
        _check(lib().sshdp_plan_group(self.handle, g, ctypes.byref(gi)), "sshdp_plan_group")
        return {k: getattr(gi, k) for k, _ in GroupInfo._fields_}

    def groups(self):
        return [self.group(g) for g in range(self.stats()["n_groups"])]

    def node(self, i):
        a = ctypes.c_int64()
        g = ctypes.c_int32()
        _check(lib().sshdp_plan_node(self.handle, i, ctypes.byref(a), ctypes.byref(g)), "sshdp_plan_node")
        return a.value, g.value

    def ns_executed(self, workspace, workspace_bytes, stream=None):
        """(units per group, MFMA flops) the Newton-Schulz tiles executed in the
        last Muon call that used this workspace (units with all-zero momentum
        count 0); synchronises."""
        ng = self.stats()["n_groups"]
        units = (ctypes.c_int32 * max(ng, 1))()
        f = ctypes.c_double()
        _check(lib().sshdp_ns_executed(self.handle, _ptr(workspace), int(workspace_bytes), units, ctypes.byref(f),
                                       _stream(stream)), "sshdp_ns_executed")
        return [units[i] for i in range(ng)], f.value

    def profile(self, enable=True):
        _check(lib().sshdp_profile_enable(self.handle, int(enable)), "sshdp_profile_enable")

    def profile_read(self):
        ms = (ctypes.c_double * len(PROF_CLASSES))()
        n = (ctypes.c_int64 * len(PROF_CLASSES))()
        _check(lib().sshdp_profile_read(self.handle, ms, n), "sshdp_profile_read")
        return {c: (ms[i], n[i]) for i, c in enumerate(PROF_CLASSES)}

    def destroy(self):
        if self._h:
            lib().sshdp_plan_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.destroy()
        except Exception:
            pass


def buffers(w_main=None, grad=None, mom=None, adam_v=None, codes=None, scales=None, w_bf16=None):
    return Buffers(_ptr(w_main), _ptr(grad), _ptr(mom), _ptr(adam_v), _ptr(codes), _ptr(scales), _ptr(w_bf16))


def muon_hp(lr=0.02, momentum=0.95, weight_decay=0.0):
    return MuonHP(lr, momentum, weight_decay)


def adamw_hp(lr=1e-3, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1):
    return AdamWHP(lr, beta1, beta2, eps, weight_decay)


def update_muon(plan, bufs, hp, workspace, workspace_bytes, stream=None):
    _check(lib().sshdp_update_muon(plan.handle, ctypes.byref(bufs), ctypes.byref(hp), _ptr(workspace),
                                   int(workspace_bytes), _stream(stream)), "sshdp_update_muon")


def update_adamw(plan, bufs, hp, step, stream=None):
    _check(lib().sshdp_update_adamw(plan.handle, ctypes.byref(bufs), ctypes.byref(hp), int(step),
                                    _stream(stream)), "sshdp_update_adamw")


def requant_mxfp8(plan, w_main, codes, scales, stream=None):
    _check(lib().sshdp_requant_mxfp8(plan.handle, _ptr(w_main), _ptr(codes), _ptr(scales), _stream(stream)),
           "sshdp_requant_mxfp8")


def cast_bf16(plan, w_main, w_bf16, stream=None):
    _check(lib().sshdp_cast_bf16(plan.handle, _ptr(w_main), _ptr(w_bf16), _stream(stream)), "sshdp_cast_bf16")


RS_DTYPE = {"fp32": 0, "bf16": 1}
RS_OUT = {"fp32": 0, "bf16_sr": 1}


def _ptr_array(inputs):
    arr = (ctypes.c_void_p * len(inputs))()
    for k, t in enumerate(inputs):
        arr[k] = _ptr(t)
    return arr


def rs_reduce(inputs, in_dtype, out, out_mode, n, seed=0, ctr=0, g0=0, stream=None):
    _check(lib().sshdp_rs_reduce(_ptr_array(inputs), len(inputs), RS_DTYPE[in_dtype], _ptr(out), RS_OUT[out_mode],
                                 int(n), int(seed), int(ctr), int(g0), _stream(stream)), "sshdp_rs_reduce")


def rs_accumulate(inputs, in_dtype, g, n, first, stream=None):
    _check(lib().sshdp_rs_accumulate(_ptr_array(inputs), len(inputs), RS_DTYPE[in_dtype], _ptr(g), int(n),
                                     int(bool(first)), _stream(stream)), "sshdp_rs_accumulate")


def _ref(x):
    """Pointer to a ctypes structure, or NULL for None."""
    return None if x is None else ctypes.byref(x)


def update_step(plan, bufs, mhp, ahp, step, workspace, workspace_bytes, stream=None):
    """mhp (ahp) may be None for a plan without Muon (AdamW) units."""
    _check(lib().sshdp_update_step(plan.handle, ctypes.byref(bufs), _ref(mhp), _ref(ahp),
                                   int(step), _ptr(workspace), int(workspace_bytes), _stream(stream)),
           "sshdp_update_step")


def update_step_noalloc(plan, bufs, mhp, ahp, step, stream=None):
    """sshdp_update_step with the library's built-in scratch as workspace."""
    _check(lib().sshdp_update_step_noalloc(plan.handle, ctypes.byref(bufs), _ref(mhp), _ref(ahp), int(step),
                                           _stream(stream)), "sshdp_update_step_noalloc")


def gemm_bf16_nt(P, Q, D, O, OT, M, N, K, batch, alpha, beta, tile, stream=None):
    _check(lib().sshdp_gemm_bf16_nt(_ptr(P), _ptr(Q), _ptr(D), _ptr(O), _ptr(OT), M, N, K, batch, alpha, beta,
                                    tile, _stream(stream)), "sshdp_gemm_bf16_nt")
