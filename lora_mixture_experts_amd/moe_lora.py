"""ctypes binding of libmoelora.so (the C ABI declared in include/moe_lora.h).

Argument marshalling only: every step of the layer runs in the library's HIP
kernels. PyTorch is used for device memory and the current stream. There is
no fallback: if the library is missing, loading fails with an error.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoelora.so")

OK, EINVAL, EWORKSPACE, EHIP, ESCRATCH = 0, -1, -2, -3, -4
SCRATCH_BYTES = 64 << 20
FLAG_OUT_BF16 = 1
FLAG_SHRINK_LAUNCH = 2
FLAG_FUSED_COMBINE = 4
FLAG_NO_SHRINK_WAIT = 8
FLAG_ROUTE_LAUNCH = 16
NKERNELS = 7


class MoeLoraError(RuntimeError):
    def __init__(self, code: int, what: str):
        super().__init__(f"{what}: {strerror(code)} ({code})")
        self.code = code


class Desc(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("T", "H", "I", "E", "top_k", "L", "r", "block_m_base", "block_m_lora", "flags",
                 "down_ksplit", "shrink_ksplit", "waves_gate_up", "waves_down", "frags_gate_up")]


class PlanInfo(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("block_m_base", "block_m_lora", "down_ksplit", "shrink_ksplit", "waves_gate_up",
                 "waves_down", "shrinks_in_projections", "combine_in_down", "routing_in_gate_up",
                 "frags_gate_up")]

    def as_dict(self):
        return {n: getattr(self, n) for n, _ in self._fields_}


class Weights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("w_gate_up", "w_down", "a_gate_up", "b_gate_up", "a_down", "b_down",
                 "w_gate_up_packed", "w_down_packed")]


_lib = None


def lib():
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it first "
                               "(python -m lora_mixture_experts_amd.build)")
        L = ctypes.CDLL(LIB_PATH)
        P, I32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        pD, pW = ctypes.POINTER(Desc), ctypes.POINTER(Weights)
        pI32, pSZ = ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_size_t)
        sig = {
            "moe_lora_strerror": ([ctypes.c_int], ctypes.c_char_p),
            "moe_lora_validate": ([pD, pW, SZ], ctypes.c_int),
            "moe_lora_block_sizes": ([pD, pI32, pI32], ctypes.c_int),
            "moe_lora_plan": ([pD, ctypes.POINTER(PlanInfo)], ctypes.c_int),
            "moe_lora_workspace_bytes": ([pD, pSZ], ctypes.c_int),
            "moe_lora_align_capacity": ([pD, pI32, pI32], ctypes.c_int),
            "moe_lora_route": ([pD, P, P, P, P], ctypes.c_int),
            "moe_lora_align": ([pD] + [P] * 9 + [P, SZ, P], ctypes.c_int),
            "moe_lora_pack_weights": ([pD, P, P, P, P, P], ctypes.c_int),
            "moe_lora_forward": ([pD, pW, P, P, P, P, P, SZ, P], ctypes.c_int),
            "moe_lora_forward_noalloc": ([pD, pW, P, P, P, P, P], ctypes.c_int),
            "moe_lora_read_stages": ([pD, P, SZ, P, P, P, P, P, P, P], ctypes.c_int),
            "moe_lora_read_alignment": ([pD, P, SZ, P, P, P, P, P, P, P, P], ctypes.c_int),
            "moe_lora_read_status": ([pD, P, SZ, P, P], ctypes.c_int),
            "moe_lora_timing_enable": ([I32], ctypes.c_int),
            "moe_lora_timing_read": ([ctypes.POINTER(ctypes.c_float), pI32], ctypes.c_int),
            "moe_lora_kernel_name": ([I32], ctypes.c_char_p),
        }
        for name, (args, res) in sig.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = res
        _lib = L
    return _lib


EXPORTED = ("moe_lora_strerror", "moe_lora_validate", "moe_lora_block_sizes", "moe_lora_plan",
            "moe_lora_workspace_bytes", "moe_lora_align_capacity", "moe_lora_route",
            "moe_lora_align", "moe_lora_pack_weights", "moe_lora_forward", "moe_lora_forward_noalloc",
            "moe_lora_read_stages",
            "moe_lora_read_alignment",
            "moe_lora_read_status",
            "moe_lora_timing_enable", "moe_lora_timing_read", "moe_lora_kernel_name")


def strerror(code: int) -> str:
    return lib().moe_lora_strerror(code).decode()


def _check(rc: int, what: str):
    if rc != OK:
        raise MoeLoraError(rc, what)


# launch tuning fields of the descriptor (0 = the library's choice)
TUNING_FIELDS = ("down_ksplit", "shrink_ksplit", "waves_gate_up", "waves_down", "frags_gate_up")


def make_desc(T, H, I, E, top_k, L, r, block_m_base=0, block_m_lora=0, flags=0, down_ksplit=0,
              shrink_ksplit=0, waves_gate_up=0, waves_down=0, frags_gate_up=0) -> Desc:
    return Desc(T, H, I, E, top_k, L, r, block_m_base, block_m_lora, flags, down_ksplit, shrink_ksplit,
                waves_gate_up, waves_down, frags_gate_up)


def plan(desc: Desc) -> dict:
    """The launch choices the library makes for a descriptor (host only)."""
    info = PlanInfo()
    _check(lib().moe_lora_plan(ctypes.byref(desc), ctypes.byref(info)), "plan")
    return info.as_dict()


def validate(desc: Desc, weights: Weights | None = None, ws_bytes: int = -1) -> int:
    """Host-only check; returns the library's code (0 = valid)."""
    wp = ctypes.byref(weights) if weights is not None else None
    sz = ctypes.c_size_t(ws_bytes if ws_bytes >= 0 else (1 << 64) - 1)
    return lib().moe_lora_validate(ctypes.byref(desc), wp, sz)


def block_sizes(desc: Desc):
    a, b = ctypes.c_int32(), ctypes.c_int32()
    _check(lib().moe_lora_block_sizes(ctypes.byref(desc), ctypes.byref(a), ctypes.byref(b)), "block_sizes")
    return a.value, b.value


def workspace_bytes(desc: Desc) -> int:
    n = ctypes.c_size_t()
    _check(lib().moe_lora_workspace_bytes(ctypes.byref(desc), ctypes.byref(n)), "workspace_bytes")
    return n.value


def align_capacity(desc: Desc):
    a, b = ctypes.c_int32(), ctypes.c_int32()
    _check(lib().moe_lora_align_capacity(ctypes.byref(desc), ctypes.byref(a), ctypes.byref(b)),
           "align_capacity")
    return a.value, b.value


# ------------------------------------------------------------------ tensor calls

def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is not None:
        return ctypes.c_void_p(stream)
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def route(desc, logits, topk_ids, topk_w, stream=None):
    _check(lib().moe_lora_route(ctypes.byref(desc), _ptr(logits), _ptr(topk_ids), _ptr(topk_w),
                                _stream(stream)), "route")


def align(desc, topk_ids, adapter_ids, sorted_b, blk_e_b, n_b, sorted_l, blk_e_l, blk_a_l, n_l,
          workspace=None, stream=None):
    """workspace: a uint8 device tensor of >= workspace_bytes(desc) bytes, or
    None (accepted up to E*(L+1) = 9712 keys)."""
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().moe_lora_align(ctypes.byref(desc), _ptr(topk_ids), _ptr(adapter_ids),
                                _ptr(sorted_b), _ptr(blk_e_b), _ptr(n_b), _ptr(sorted_l),
                                _ptr(blk_e_l), _ptr(blk_a_l), _ptr(n_l), _ptr(workspace),
                                ctypes.c_size_t(ws_bytes), _stream(stream)), "align")


def weights_struct(w_gate_up, w_down, a_gate_up=None, b_gate_up=None, a_down=None, b_down=None,
                   w_gate_up_packed=None, w_down_packed=None):
    return Weights(*(None if t is None or t.numel() == 0 else t.data_ptr()
                     for t in (w_gate_up, w_down, a_gate_up, b_gate_up, a_down, b_down,
                               w_gate_up_packed, w_down_packed)))


def pack_weights(desc, w_gate_up, w_down, w_gate_up_packed, w_down_packed, stream=None):
    """Write the 16-row kernels' packed copies of the base weights (either
    pair may be None)."""
    _check(lib().moe_lora_pack_weights(ctypes.byref(desc), _ptr(w_gate_up), _ptr(w_down), _ptr(w_gate_up_packed),
                                       _ptr(w_down_packed), _stream(stream)), "pack_weights")


def forward(desc, weights: Weights, x, logits, adapter_ids, out, workspace, stream=None):
    _check(lib().moe_lora_forward(ctypes.byref(desc), ctypes.byref(weights), _ptr(x), _ptr(logits),
                                  _ptr(adapter_ids), _ptr(out), _ptr(workspace),
                                  ctypes.c_size_t(workspace.numel() * workspace.element_size()),
                                  _stream(stream)), "forward")


def forward_noalloc(desc, weights: Weights, x, logits, adapter_ids, out, stream=None):
    """The layer with the library's static scratch instead of a workspace
    (include/moe_lora.h, moe_lora_forward_noalloc)."""
    _check(lib().moe_lora_forward_noalloc(ctypes.byref(desc), ctypes.byref(weights), _ptr(x), _ptr(logits),
                                          _ptr(adapter_ids), _ptr(out), _stream(stream)), "forward_noalloc")


def read_stages(desc, workspace, topk_ids=None, topk_w=None, s1=None, h=None, s2=None, dn=None,
                stream=None):
    _check(lib().moe_lora_read_stages(ctypes.byref(desc), _ptr(workspace),
                                      ctypes.c_size_t(workspace.numel() * workspace.element_size()),
                                      _ptr(topk_ids), _ptr(topk_w), _ptr(s1), _ptr(h), _ptr(s2),
                                      _ptr(dn), _stream(stream)), "read_stages")


STATUS_SHRINK_FALLBACK = 1


def read_status(desc, workspace, status, stream=None):
    """Enqueue a copy of the last forward call's status word into `status`
    (a device int32 tensor of one element)."""
    _check(lib().moe_lora_read_status(ctypes.byref(desc), _ptr(workspace),
                                      ctypes.c_size_t(workspace.numel() * workspace.element_size()),
                                      _ptr(status), _stream(stream)), "read_status")


def read_alignment(desc, workspace, sorted_b=None, blk_e_b=None, n_b=None, sorted_l=None,
                   blk_e_l=None, blk_a_l=None, n_l=None, stream=None):
    _check(lib().moe_lora_read_alignment(ctypes.byref(desc), _ptr(workspace),
                                         ctypes.c_size_t(workspace.numel() * workspace.element_size()),
                                         _ptr(sorted_b), _ptr(blk_e_b), _ptr(n_b), _ptr(sorted_l),
                                         _ptr(blk_e_l), _ptr(blk_a_l), _ptr(n_l), _stream(stream)),
           "read_alignment")


def timing_enable(max_calls: int):
    _check(lib().moe_lora_timing_enable(max_calls), "timing_enable")


def timing_read():
    ms = (ctypes.c_float * NKERNELS)()
    n = ctypes.c_int32()
    _check(lib().moe_lora_timing_read(ms, ctypes.byref(n)), "timing_read")
    return list(ms), n.value


def kernel_names():
    return [lib().moe_lora_kernel_name(i).decode() for i in range(NKERNELS)]


# ------------------------------------------------------------------ convenience

class Layer:
    """Device-resident weights + descriptor + workspace for repeated calls."""

    def __init__(self, T, H, I, E, top_k, L, r, w_gate_up, w_down, a_gate_up=None, b_gate_up=None,
                 a_down=None, b_down=None, block_m_base=0, block_m_lora=0, out_bf16=False,
                 shrink_launch=False, tuning=None, fused_combine=False, no_shrink_wait=False,
                 packed_weights=False, route_launch=False, **launch):
        """tuning: a tuning.Table; when it holds a choice for this shape and
        token count it sets the block sizes, the shrink placement and the
        launch tuning fields (only if none of them is given explicitly).
        packed_weights: where the plan uses 16-row base blocks, also hold
        packed copies of the base weights, which those kernels then read
        (twice the base weight memory; self.packed says whether it did).
        route_launch: keep the routing and alignment launches where the
        library would route a decode-sized batch inside the gate_up launch.
        launch: any of TUNING_FIELDS (0 = the library's choice)."""
        import torch
        bad = set(launch) - set(TUNING_FIELDS)
        if bad:
            raise TypeError(f"unknown launch options {sorted(bad)}")
        self.tuned = None
        if (tuning is not None and block_m_base == 0 and block_m_lora == 0 and not shrink_launch
                and not any(launch.values())):
            self.tuned = tuning.lookup(T, H, I, E, top_k, L, r)
            if self.tuned is not None:
                block_m_base = self.tuned.block_m_base
                block_m_lora = self.tuned.block_m_lora
                shrink_launch = self.tuned.shrink_launch
                launch = {f: getattr(self.tuned, f) for f in TUNING_FIELDS}
        self.desc = make_desc(T, H, I, E, top_k, L, r, block_m_base, block_m_lora,
                              (FLAG_OUT_BF16 if out_bf16 else 0) |
                              (FLAG_SHRINK_LAUNCH if shrink_launch else 0) |
                              (FLAG_FUSED_COMBINE if fused_combine else 0) |
                              (FLAG_NO_SHRINK_WAIT if no_shrink_wait else 0) |
                              (FLAG_ROUTE_LAUNCH if route_launch else 0), **launch)
        # the down projection's rows are kept (and readable) only when a
        # separate launch does the weighted combine
        self.keeps_down_rows = not fused_combine
        self.out_dtype = torch.bfloat16 if out_bf16 else torch.float32
        # packed copies only where the plan runs the 16-row kernels, which
        # are the ones that read them
        packed = (None, None)
        self.packed = bool(packed_weights) and plan(self.desc)["block_m_base"] == 16
        if self.packed:
            packed = (torch.empty_like(w_gate_up), torch.empty_like(w_down))
            pack_weights(self.desc, w_gate_up, w_down, *packed)
        self.tensors = (w_gate_up, w_down, a_gate_up, b_gate_up, a_down, b_down) + packed
        self.weights = weights_struct(*self.tensors)
        _check(validate(self.desc, self.weights), "validate")
        self.workspace = torch.empty(workspace_bytes(self.desc), dtype=torch.uint8, device=w_gate_up.device)
        self.device = w_gate_up.device

    def __call__(self, x, logits, adapter_ids, out=None, stream=None):
        import torch
        if out is None:
            out = torch.empty((self.desc.T, self.desc.H), dtype=self.out_dtype, device=self.device)
        forward(self.desc, self.weights, x, logits, adapter_ids, out, self.workspace, stream)
        return out

    def status(self, stream=None) -> int:
        """Status word of the last call (0 = every projection wave found the
        shrink of its launch done; STATUS_SHRINK_FALLBACK = some wave computed
        its own, output still valid); synchronises."""
        import torch
        st = torch.full((1,), -1, dtype=torch.int32, device=self.device)
        read_status(self.desc, self.workspace, st, stream)
        torch.cuda.synchronize(self.device)
        return int(st.item())

    def stages(self, stream=None):
        import torch
        d, dev = self.desc, self.device
        P = d.T * d.top_k
        r = d.r if d.L > 0 else 8
        st = dict(topk_ids=torch.empty(P, dtype=torch.int32, device=dev),
                  topk_w=torch.empty(P, dtype=torch.float32, device=dev),
                  s1=torch.empty((P, r), dtype=torch.float32, device=dev),
                  h=torch.empty((P, d.I), dtype=torch.bfloat16, device=dev),
                  s2=torch.empty((P, r), dtype=torch.float32, device=dev),
                  dn=(torch.empty((P, d.H), dtype=torch.float32, device=dev) if self.keeps_down_rows
                      else None))
        read_stages(d, self.workspace, stream=stream, **st)
        return {k: v for k, v in st.items() if v is not None}

    def alignment(self, stream=None):
        import torch
        d, dev = self.desc, self.device
        C_b, C_l = align_capacity(d)
        bm_b, bm_l = block_sizes(d)
        z = lambda n: torch.empty(n, dtype=torch.int32, device=dev)
        out = dict(sorted_b=z(C_b), blk_e_b=z(C_b // bm_b), n_b=z(1), sorted_l=z(C_l),
                   blk_e_l=z(C_l // bm_l), blk_a_l=z(C_l // bm_l), n_l=z(1))
        read_alignment(d, self.workspace, stream=stream, **out)
        return out
