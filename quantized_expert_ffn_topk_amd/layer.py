"""One MoE layer resident on the GPU, driven through the C ABI.

Packs expert weights with moe_pack_expert_* on the host, uploads every blob to
its own device allocation, and keeps the router weights, the device table of
expert pointers and a moe_ctx.  torch supplies device memory and streams only.
"""
import numpy as np

from . import abi


def make_desc(H, F, E, k, n_shared, group=32, routed_scale=1.0, wfmt=abi.WFMT_INT4,
              out_dtype=abi.DT_F32):
    return abi.moe_layer_desc(H, F, E, k, n_shared, group, float(routed_scale), wfmt, out_dtype)


def pack_int4(desc, ex):
    blob = np.empty(abi.moe_blob_bytes(desc), np.uint8)
    arrs = [np.ascontiguousarray(ex[n]) for n in
            ("q_gate", "s_gate", "q_up", "s_up", "q_down", "s_down")]
    abi.moe_pack_expert_int4(desc, *arrs, blob)
    return blob


def pack_mxfp4(desc, ex):
    blob = np.empty(abi.moe_blob_bytes(desc), np.uint8)
    arrs = [np.ascontiguousarray(ex[n]) for n in
            ("c_gate", "e_gate", "c_up", "e_up", "c_down", "e_down")]
    abi.moe_pack_expert_mxfp4(desc, *arrs, blob)
    return blob


class Layer:
    """experts: list of distinct expert weight dicts; expert_map[e] picks the
    dict of routed expert e (default: e itself).  Every routed expert gets its
    own device blob even when several share a dict."""

    def __init__(self, desc, Wr, b, experts, shared=None, expert_map=None, max_tokens=1,
                 device=0, path=abi.PATH_AUTO):
        import torch
        self.torch = torch
        self.desc = desc
        self.dev = torch.device("cuda", device)
        E = desc.n_experts
        pack = pack_mxfp4 if desc.wfmt == abi.WFMT_MXFP4 else pack_int4
        emap = list(range(E)) if expert_map is None else list(expert_map)
        host = [pack(desc, ex) for ex in experts]
        staged = [torch.from_numpy(h).to(self.dev) for h in host]
        self.blobs = []
        for e in range(E):
            t = torch.empty(host[0].shape[0], dtype=torch.uint8, device=self.dev)
            t.copy_(staged[emap[e]])
            self.blobs.append(t)
        del staged
        self.shared_blob = None
        if shared is not None:
            self.shared_blob = torch.from_numpy(pack(desc, shared)).to(self.dev)
        self.ptrs = torch.tensor([t.data_ptr() for t in self.blobs], dtype=torch.int64,
                                 device=self.dev)
        self.Wr = torch.from_numpy(np.ascontiguousarray(Wr, np.float32)).to(self.dev)
        self.b = torch.from_numpy(np.ascontiguousarray(b, np.float32)).to(self.dev)
        self.weights = abi.moe_layer_weights(self.Wr.data_ptr(), self.b.data_ptr(),
                                             self.ptrs.data_ptr(),
                                             self.shared_blob.data_ptr() if shared is not None else None)
        self.max_tokens = max_tokens
        self.ctx = abi.moe_ctx_create(device, desc, max_tokens)
        if path != abi.PATH_AUTO:
            abi.moe_ctx_set_path(self.ctx, path)

    def set_bias(self, b):
        self.b.copy_(self.torch.from_numpy(np.ascontiguousarray(b, np.float32)))

    def set_path(self, path):
        abi.moe_ctx_set_path(self.ctx, path)

    def x_tensor(self, x_bf16_bits):
        return self.torch.from_numpy(np.ascontiguousarray(x_bf16_bits, np.uint16).view(np.int16)).to(self.dev)

    def _outs(self, T):
        t = self.torch
        k = self.desc.top_k
        idx = t.empty((T, k), dtype=t.int32, device=self.dev)
        w = t.empty((T, k), dtype=t.float32, device=self.dev)
        odt = t.bfloat16 if self.desc.out_dtype == abi.DT_BF16 else t.float32
        out = t.empty((T, self.desc.hidden), dtype=odt, device=self.dev)
        return idx, w, out

    def router(self, x, stream=None):
        T = x.shape[0]
        idx, w, _ = self._outs(T)
        abi.moe_router_topk(self.ctx, x, T, self.weights, idx, w, stream)
        return idx, w

    def ffn(self, x, idx, w, stream=None, out=None):
        T = x.shape[0]
        if out is None:
            out = self._outs(T)[2]
        abi.moe_expert_ffn(self.ctx, x, T, self.weights, idx, w, out, stream)
        return out

    def forward(self, x, stream=None, outs=None, cache=None, layer=0):
        T = x.shape[0]
        idx, w, out = outs if outs is not None else self._outs(T)
        abi.moe_layer_forward(self.ctx, x, T, self.weights, cache, layer, idx, w, out, stream)
        return idx, w, out

    def debug_read(self, which, shape, dtype):
        t = self.torch
        buf = t.empty(shape, dtype=dtype, device=self.dev)
        abi.moe_debug_read(self.ctx, which, buf, buf.numel() * buf.element_size())
        return buf

    def close(self):
        if getattr(self, "ctx", None):
            abi.moe_ctx_destroy(self.ctx)
            self.ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
