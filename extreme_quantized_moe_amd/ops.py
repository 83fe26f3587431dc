"""Thin torch-facing binding of libmilo (same call names as include/milo.h
without the `milo_` prefix).  torch supplies device memory and the current
stream; every computation runs in the library's HIP kernels.  There is no
fallback: if libmilo.so is missing, importing the binding raises."""
import ctypes as C

import torch

from . import _lib as L
from ._lib import check

_DEV_CHECKED = set()


def _stream():
    return torch.cuda.current_stream().cuda_stream


def _p(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _cuda(*ts):
    for t in ts:
        if t is not None and (not t.is_cuda or not t.is_contiguous()):
            raise ValueError("libmilo needs contiguous CUDA (HIP) tensors")


def packed_words(rows, K):
    return int(L.lib().milo_packed_words(rows, K))


def sz_words(rows, K):
    return int(L.lib().milo_sz_words(rows, K))


def quantize_rtn_int3(W, group=64):
    """fp32 [rows][K] -> (codes u8 [rows][K], scale fp16 [rows][K/group], zero fp16)."""
    W = W.contiguous()
    _cuda(W)
    rows, K = W.shape
    codes = torch.empty((rows, K), dtype=torch.uint8, device=W.device)
    scale = torch.empty((rows, K // group), dtype=torch.float16, device=W.device)
    zero = torch.empty_like(scale)
    if group == 64:
        check("milo_quantize_rtn_int3", L.lib().milo_quantize_rtn_int3(
            _p(W), rows, K, _p(codes), _p(scale), _p(zero), _stream()))
    else:
        check("milo_quantize_rtn_int3_grouped", L.lib().milo_quantize_rtn_int3_grouped(
            _p(W), rows, K, group, _p(codes), _p(scale), _p(zero), _stream()))
    return codes, scale, zero


def quantize_hqq_int3(W, iters=20, p_norm=0.7, beta=10.0, kappa=1.01):
    """HQQ-style zero-point optimization on top of the RTN scale (see
    include/milo.h).  fp32 [rows][K] -> (codes, scale fp16, zero fp16)."""
    W = W.contiguous()
    _cuda(W)
    rows, K = W.shape
    codes = torch.empty((rows, K), dtype=torch.uint8, device=W.device)
    scale = torch.empty((rows, K // 64), dtype=torch.float16, device=W.device)
    zero = torch.empty_like(scale)
    check("milo_quantize_hqq_int3", L.lib().milo_quantize_hqq_int3(
        _p(W), rows, K, iters, p_norm, beta, kappa, _p(codes), _p(scale), _p(zero), _stream()))
    return codes, scale, zero


def lr_words(N, K, max_rank):
    """Per-expert uint32 word counts of the int3 compensator layouts:
    (V codes, V scale/zero, U codes, U scale/zero)."""
    lib = L.lib()
    return (int(lib.milo_lr_v_words(max_rank, K)), int(lib.milo_lr_v_sz_words(max_rank, K)),
            int(lib.milo_lr_u_words(N, max_rank)), int(lib.milo_lr_u_sz_words(N)))


def pack_lr_int3(v, u, N, K, rank, max_rank, out=None):
    """Pack one expert's quantized factors: v = (codes [rank][K], scale, zero
    [rank][K/64]), u = (codes [N][rank], scale, zero [N]) (None when rank == 0).
    out: optional (vq, vsz, uq, usz) int32 views to write into."""
    dev = torch.device("cuda", torch.cuda.current_device())
    if out is None:
        out = tuple(torch.empty(n, dtype=torch.int32, device=dev) for n in lr_words(N, K, max_rank))
    vq, vsz, uq, usz = out
    vc, vs, vz = v if v is not None else (None, None, None)
    uc, us, uz = u if u is not None else (None, None, None)
    _cuda(vc, vs, vz, uc, us, uz, vq, vsz, uq, usz)
    check("milo_pack_lr_int3", L.lib().milo_pack_lr_int3(
        _p(vc), _p(vs), _p(vz), _p(uc), _p(us), _p(uz), N, K, rank, max_rank,
        _p(vq), _p(vsz), _p(uq), _p(usz), _stream()))
    return out


def pack_int3(codes, scale, zero):
    """codes u8 [rows][K], scale/zero fp16 [rows][K/64] -> (packed int32 words,
    tiled scale/zero int32 words) in layout v1 (bit patterns in int32)."""
    _cuda(codes, scale, zero)
    rows, K = codes.shape
    packed = torch.empty(packed_words(rows, K), dtype=torch.int32, device=codes.device)
    sz = torch.empty(sz_words(rows, K), dtype=torch.int32, device=codes.device)
    check("milo_pack_int3", L.lib().milo_pack_int3(
        _p(codes), _p(scale), _p(zero), rows, K, _p(packed), _p(sz), _stream()))
    return packed, sz


def lowrank_svd(R, rank, omega, power_iters=2):
    """Rank-r approximation R ~ U V (randomized subspace iteration, see
    include/milo.h).  R fp32 [N][K]; omega fp32 [rank + oversample][K].
    Returns (U [N][rank], V [rank][K], sigma [rank])."""
    R = R.contiguous()
    omega = omega.contiguous()
    _cuda(R, omega)
    N, K = R.shape
    p = omega.shape[0] - rank
    dev = R.device
    U = torch.empty((N, rank), dtype=torch.float32, device=dev)
    V = torch.empty((rank, K), dtype=torch.float32, device=dev)
    sigma = torch.empty(rank, dtype=torch.float32, device=dev)
    nbytes = int(L.lib().milo_lowrank_svd_workspace_bytes(N, K, rank, p))
    ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=dev)
    check("milo_lowrank_svd", L.lib().milo_lowrank_svd(
        _p(R), N, K, rank, p, power_iters, _p(omega), _p(U), _p(V), _p(sigma), _p(ws), ws.numel(), _stream()))
    return U, V, sigma


def build_compensator(W, rank, iters, omega, power_iters=2, quantizer="rtn"):
    """Quantize-and-compensate refinement of one weight matrix (see
    include/milo.h).  W fp32 [N][K]; omega fp32 [iters][rank + oversample][K]
    (ignored when rank == 0); quantizer "rtn" or "hqq".  Returns (codes,
    scale, zero, U, V, sigma)."""
    qid = {"rtn": L.QUANT_RTN, "hqq": L.QUANT_HQQ}[quantizer]
    W = W.contiguous()
    _cuda(W)
    N, K = W.shape
    dev = W.device
    if rank > 0:
        omega = omega.contiguous()
        _cuda(omega)
        p = omega.shape[1] - rank
    else:
        p = 0
    codes = torch.empty((N, K), dtype=torch.uint8, device=dev)
    scale = torch.empty((N, K // 64), dtype=torch.float16, device=dev)
    zero = torch.empty_like(scale)
    U = torch.empty((N, rank), dtype=torch.float32, device=dev)
    V = torch.empty((rank, K), dtype=torch.float32, device=dev)
    sigma = torch.empty(rank, dtype=torch.float32, device=dev)
    nbytes = int(L.lib().milo_build_compensator_workspace_bytes(N, K, rank, p))
    ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=dev)
    check("milo_build_compensator", L.lib().milo_build_compensator(
        _p(W), N, K, rank, iters, p, power_iters, qid, _p(omega) if rank > 0 else None, _p(codes), _p(scale),
        _p(zero), _p(U) if rank else None, _p(V) if rank else None, _p(sigma) if rank else None,
        _p(ws), ws.numel(), _stream()))
    return codes, scale, zero, U, V, sigma


def weight_kurtosis(W, count=None):
    """W: fp32, `count` matrices stored back to back (default: the leading
    dimension of a 3-D tensor, else one matrix).  Returns (kurtosis, mean) as
    float64 device tensors [count]."""
    W = W.contiguous()
    _cuda(W)
    if count is None:
        count = W.shape[0] if W.dim() > 2 else 1
    elems = W.numel() // count
    kurt = torch.empty(count, dtype=torch.float64, device=W.device)
    mean = torch.empty(count, dtype=torch.float64, device=W.device)
    nbytes = int(L.lib().milo_weight_kurtosis_workspace_bytes(count))
    ws = torch.empty(max(nbytes, 8), dtype=torch.uint8, device=W.device)
    check("milo_weight_kurtosis", L.lib().milo_weight_kurtosis(
        _p(W), count, elems, _p(kurt), _p(mean), _p(ws), ws.numel(), _stream()))
    return kurt, mean


def expert_counts(offsets, counts):
    """counts (int64 device [E]) += pairs per expert of one routing call."""
    _cuda(offsets, counts)
    check("milo_expert_counts", L.lib().milo_expert_counts(
        _p(offsets), counts.numel(), _p(counts), _stream()))
    return counts


def rank_policy(kurtosis, frequency, dense, total_rank, r_min=0, r_max=64, step=8):
    """Host rank apportionment (see include/milo.h); sequences of floats /
    bools in, list of ints out."""
    n = len(kurtosis)
    k = (C.c_double * n)(*[float(v) for v in kurtosis])
    f = (C.c_double * n)(*[float(v) for v in frequency])
    d = (C.c_int32 * n)(*[1 if v else 0 for v in dense])
    out = (C.c_int32 * n)()
    check("milo_rank_policy", L.lib().milo_rank_policy(
        C.cast(k, C.c_void_p), C.cast(f, C.c_void_p), C.cast(d, C.c_void_p), n, total_rank, r_min, r_max,
        step, C.cast(out, C.c_void_p)))
    return list(out)


_route_ws = {}


def route_sort(logits, k, S=0, renormalize=True):
    """Softmax top-k routing + expert sort.  Returns dict of device tensors:
    ids [T][k], w [T][k], slot_w [T*(k+S)], sorted_pairs, pair_pos [T*(k+S)],
    offsets [E+S+1]."""
    logits = logits.contiguous()
    _cuda(logits)
    T, E = logits.shape
    slots = k + S
    dev = logits.device
    out = {
        "ids": torch.empty((T, k), dtype=torch.int32, device=dev),
        "w": torch.empty((T, k), dtype=torch.float32, device=dev),
        "slot_w": torch.empty(T * slots, dtype=torch.float32, device=dev),
        "sorted_pairs": torch.empty(T * slots, dtype=torch.int32, device=dev),
        "pair_pos": torch.empty(T * slots, dtype=torch.int32, device=dev),
        "offsets": torch.empty(E + S + 1, dtype=torch.int32, device=dev),
    }
    nbytes = int(L.lib().milo_route_workspace_bytes(T, E, k, S))
    ws = None
    if nbytes:
        key = (dev.index, nbytes)
        ws = _route_ws.get(key)
        if ws is None:
            ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
            _route_ws[key] = ws
    check("milo_route_sort", L.lib().milo_route_sort(
        _p(logits), T, E, k, S, 1 if renormalize else 0, _p(out["ids"]), _p(out["w"]),
        _p(out["slot_w"]), _p(out["sorted_pairs"]), _p(out["pair_pos"]), _p(out["offsets"]),
        _p(ws), nbytes, _stream()))
    return out


class Family:
    """One projection family (e.g. every expert's W1) in the library's format:
    packed int3 codes (layout v1), tiled scale/zero, compensator factors and
    the device rank array.  Factors are fp16 U [E][N][max_rank] and
    V [E][max_rank][K] (zero beyond each expert's rank), or with
    lr_format "int3" the int3 compensator layouts Uq, Usz, Vq, Vsz."""

    def __init__(self, packed, sz, U, V, rank, num_experts, N, K, max_rank,
                 lr_format="fp16", lrq=None):
        self.packed, self.sz, self.U, self.V, self.rank = packed, sz, U, V, rank
        self.num_experts, self.N, self.K, self.max_rank = num_experts, N, K, max_rank
        self.lr_format = lr_format
        self.lrq = lrq            # (Vq, Vsz, Uq, Usz) for int3 factors

    @staticmethod
    def from_dense(Ws, As, Bs, max_rank=None, device="cuda", lr_format="fp16", quantizer="rtn"):
        """Ws: list of fp32 [N][K]; As: list of fp16 [K][r_e]; Bs: fp16 [r_e][N]
        (the compensator as X A B, i.e. V = A^T, U = B^T).  Quantizes each W on
        the GPU (int3, group 64; quantizer "rtn" or "hqq") and packs all
        experts in one call.  With
        lr_format "int3" the factors are quantized on the GPU as well (V rows
        in groups of 64 along K, U rows in one group of r_e) and packed per
        expert."""
        E = len(Ws)
        N, K = Ws[0].shape
        ranks = [int(a.shape[1]) for a in As]
        R = max(ranks) if max_rank is None else max_rank
        codes = torch.empty((E * N, K), dtype=torch.uint8, device=device)
        scale = torch.empty((E * N, K // 64), dtype=torch.float16, device=device)
        zero = torch.empty_like(scale)
        for e, W in enumerate(Ws):
            Wd = W.to(device=device, dtype=torch.float32)
            c, s, z = quantize_hqq_int3(Wd) if quantizer == "hqq" else quantize_rtn_int3(Wd)
            codes[e * N:(e + 1) * N] = c
            scale[e * N:(e + 1) * N] = s
            zero[e * N:(e + 1) * N] = z
        packed, sz = pack_int3(codes, scale, zero)
        del codes, scale, zero
        rank = torch.tensor(ranks, dtype=torch.int32, device=device)
        if lr_format == "int3":
            lrq = Family._pack_int3_factors(As, Bs, ranks, N, K, R, device)
            return Family(packed, sz, None, None, rank, E, N, K, R, "int3", lrq)
        if lr_format != "fp16":
            raise ValueError(f"unknown compensator format {lr_format!r}")
        U = torch.zeros((E, N, max(R, 1)), dtype=torch.float16, device=device)
        V = torch.zeros((E, max(R, 1), K), dtype=torch.float16, device=device)
        for e in range(E):
            r = ranks[e]
            if r:
                U[e, :, :r] = Bs[e].to(device).t()
                V[e, :r, :] = As[e].to(device).t()
        return Family(packed, sz, U, V, rank, E, N, K, R)

    @staticmethod
    def _pack_int3_factors(As, Bs, ranks, N, K, R, device):
        E = len(As)
        if R == 0:
            return None
        nv, nvs, nu, nus = lr_words(N, K, R)
        Vq = torch.empty(E * nv, dtype=torch.int32, device=device)
        Vsz = torch.empty(E * nvs, dtype=torch.int32, device=device)
        Uq = torch.empty(E * nu, dtype=torch.int32, device=device)
        Usz = torch.empty(E * nus, dtype=torch.int32, device=device)
        for e in range(E):
            r = ranks[e]
            out = (Vq[e * nv:(e + 1) * nv], Vsz[e * nvs:(e + 1) * nvs],
                   Uq[e * nu:(e + 1) * nu], Usz[e * nus:(e + 1) * nus])
            v = u = None
            if r:
                Vt = As[e].to(device=device, dtype=torch.float32).t().contiguous()   # [r][K]
                Ut = Bs[e].to(device=device, dtype=torch.float32).t().contiguous()   # [N][r]
                v = quantize_rtn_int3(Vt, 64)
                uc, us, uz = quantize_rtn_int3(Ut, r)
                u = (uc, us.reshape(N).contiguous(), uz.reshape(N).contiguous())
            pack_lr_int3(v, u, N, K, r, R, out)
        return (Vq, Vsz, Uq, Usz)

    def weights_struct(self):
        w = L.MiloWeights()
        w.packed = self.packed.data_ptr()
        w.sz = self.sz.data_ptr()
        w.rank = self.rank.data_ptr()
        if self.lr_format == "int3":
            w.lr_format = L.LR_INT3
            if self.lrq is not None:
                w.Vq, w.Vsz, w.Uq, w.Usz = (t.data_ptr() for t in self.lrq)
        else:
            w.lr_format = L.LR_FP16
            w.U = self.U.data_ptr()
            w.V = self.V.data_ptr()
        return w

    def nbytes(self):
        out = {"packed": self.packed.numel() * 4, "sz": self.sz.numel() * 4}
        if self.lr_format == "int3":
            for n, t in zip(("Vq", "Vsz", "Uq", "Usz"), self.lrq or ()):
                out[n] = t.numel() * 4
        else:
            out.update({"U": self.U.numel() * 2, "V": self.V.numel() * 2})
        return out


_gemm_ws = {}


def _workspace(dev, nbytes):
    """A scratch workspace per (device, stream), grown on demand.  Calls on
    one stream run in order, so they can share it; calls on different streams
    may overlap in time and get different workspaces."""
    key = (dev.index, torch.cuda.current_stream(dev).cuda_stream)
    ws = _gemm_ws.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=dev)
        _gemm_ws[key] = ws
    return ws


def make_gemm_desc(families, x, offsets, num_pairs, epilogue, y, sorted_pairs=None,
                   gather_div=0, slot_w=None, y_rows=0, max_rows_per_expert=0,
                   path=L.PATH_AUTO):
    f0 = families[0]
    d = L.MiloGemmDesc()
    d.num_experts, d.N, d.K, d.max_rank = f0.num_experts, f0.N, f0.K, f0.max_rank
    d.n_w = len(families)
    for i, f in enumerate(families):
        d.w[i] = f.weights_struct()
    d.x = x.data_ptr()
    d.x_rows = x.shape[0]
    d.gather_div = gather_div
    d.sorted_pairs = None if sorted_pairs is None else sorted_pairs.data_ptr()
    d.offsets = offsets.data_ptr()
    d.num_pairs = num_pairs
    d.max_rows_per_expert = max_rows_per_expert
    d.slot_w = None if slot_w is None else slot_w.data_ptr()
    d.y_rows = y_rows
    d.epilogue = epilogue
    d.y = y.data_ptr()
    d.path = path
    return d


def moe_w3a16_lowrank_gemm(families, x, offsets, num_pairs, epilogue, y, sorted_pairs=None,
                           gather_div=0, slot_w=None, y_rows=0, max_rows_per_expert=0,
                           path=L.PATH_AUTO, workspace=None, flags=0):
    """Routed W3A16 + low-rank grouped GEMM (see include/milo.h).  Writes y."""
    _cuda(x, offsets, y, sorted_pairs, slot_w)
    d = make_gemm_desc(families, x, offsets, num_pairs, epilogue, y, sorted_pairs, gather_div,
                       slot_w, y_rows, max_rows_per_expert, path)
    d.flags = flags
    nbytes = int(L.lib().milo_moe_gemm_workspace_bytes(C.byref(d)))
    ws = workspace if workspace is not None else _workspace(x.device, nbytes)
    check("milo_moe_w3a16_lowrank_gemm", L.lib().milo_moe_w3a16_lowrank_gemm(
        C.byref(d), _p(ws) if nbytes else None, ws.numel() if nbytes else 0, _stream()))
    return y


def moe_lowrank_prepass(families, x, offsets, num_pairs, epilogue, y, sorted_pairs=None,
                        gather_div=0, slot_w=None, y_rows=0, max_rows_per_expert=0,
                        path=L.PATH_AUTO, workspace=None):
    """First stage of the GEMM on its own (see include/milo.h); follow with
    moe_w3a16_lowrank_gemm(..., flags=GEMM_PREPASS_DONE) on the same workspace."""
    _cuda(x, offsets, y, sorted_pairs, slot_w)
    d = make_gemm_desc(families, x, offsets, num_pairs, epilogue, y, sorted_pairs, gather_div,
                       slot_w, y_rows, max_rows_per_expert, path)
    nbytes = int(L.lib().milo_moe_gemm_workspace_bytes(C.byref(d)))
    ws = workspace if workspace is not None else _workspace(x.device, nbytes)
    check("milo_moe_lowrank_prepass", L.lib().milo_moe_lowrank_prepass(
        C.byref(d), _p(ws) if nbytes else None, ws.numel() if nbytes else 0, _stream()))


def moe_combine(y, T, slots, out=None):
    """fp32 [T*slots][H] -> fp16 [T][H]: sum of each token's slots in order."""
    _cuda(y)
    H = y.shape[1]
    if out is None:
        out = torch.empty((T, H), dtype=torch.float16, device=y.device)
    check("milo_moe_combine", L.lib().milo_moe_combine(_p(y), T, slots, H, _p(out), _stream()))
    return out


class MoELayer:
    """A routed SwiGLU MoE FFN with int3 + low-rank experts:
    route -> fused gate/up GEMM + SwiGLU -> fused down GEMM + route scale ->
    combine (four library calls)."""

    def __init__(self, w1, w3, w2, E, k, S=0, renormalize=True):
        self.w1, self.w3, self.w2 = w1, w3, w2
        self.E, self.k, self.S, self.renormalize = E, k, S, renormalize
        self.H, self.F = w2.N, w1.N

    def forward(self, x, logits, path=L.PATH_AUTO, return_all=False):
        T = x.shape[0]
        slots = self.k + self.S
        P = T * slots
        r = route_sort(logits, self.k, self.S, self.renormalize)
        G = torch.empty((P, self.F), dtype=torch.float16, device=x.device)
        moe_w3a16_lowrank_gemm((self.w1, self.w3), x, r["offsets"], P, L.EPI_SWIGLU, G,
                               sorted_pairs=r["sorted_pairs"], gather_div=slots,
                               max_rows_per_expert=T, path=path)
        Y = torch.empty((P, self.H), dtype=torch.float32, device=x.device)
        moe_w3a16_lowrank_gemm((self.w2,), G, r["offsets"], P, L.EPI_ROUTE_SCALE, Y,
                               sorted_pairs=r["sorted_pairs"], gather_div=0,
                               slot_w=r["slot_w"], y_rows=P, max_rows_per_expert=T, path=path)
        out = moe_combine(Y, T, slots)
        if return_all:
            return out, {"route": r, "G": G, "Y": Y}
        return out
