"""Device-memory plumbing around the C ABI: torch tensors for the workspace,
the slot pool and activations, the library's pinned allocator for the host
expert pool.  Every computation is a call into libmoe.so."""
from __future__ import annotations

import ctypes

import numpy as np
import torch

from . import binding as B


class HostPool:
    """Pinned host expert pool [L*E][S] allocated by the library."""

    def __init__(self, nbytes: int):
        p = ctypes.c_void_p()
        B.check(B.moe_host_alloc(nbytes, ctypes.byref(p)))
        self.ptr = p.value
        self.nbytes = nbytes

    def array(self) -> np.ndarray:
        """uint8 numpy view of the pool (no copy)."""
        return np.ctypeslib.as_array((ctypes.c_uint8 * self.nbytes).from_address(self.ptr))

    def free(self):
        if self.ptr:
            B.moe_host_free(self.ptr)
            self.ptr = None

    def __del__(self):
        try:
            self.free()
        except Exception:
            pass


class MoeRuntime:
    """One library context with its device buffers."""

    def __init__(self, L, E, k, H, I, wfmt, n_slots, max_tokens, host_pool: HostPool, host_threads=0,
                 device="cuda"):
        self.cfg = B.make_config(L, E, k, H, I, wfmt, n_slots, max_tokens, host_threads)
        self.S = B.moe_expert_bytes(ctypes.byref(self.cfg))
        wsb = B.moe_workspace_bytes(ctypes.byref(self.cfg))
        if wsb == 0:
            raise B.MoeError(B.MOE_E_INVAL, B.last_error())
        self.device = torch.device(device)
        self.ws = torch.empty(wsb, dtype=torch.uint8, device=self.device)
        self.slots = torch.empty(max(n_slots, 1) * self.S, dtype=torch.uint8, device=self.device)
        self.host = host_pool
        ctx = ctypes.c_void_p()
        torch.cuda.synchronize()
        B.check(B.moe_create(ctypes.byref(self.cfg), host_pool.ptr, host_pool.nbytes, self.slots.data_ptr(),
                             n_slots * self.S, self.ws.data_ptr(), wsb, ctypes.byref(ctx)))
        self.ctx = ctx.value

    # -- helpers -----------------------------------------------------------
    def _chk(self, rc):
        return B.check(rc, self.ctx)

    @staticmethod
    def stream_ptr(stream=None):
        s = torch.cuda.current_stream() if stream is None else stream
        return s.cuda_stream

    def slot_table(self) -> torch.Tensor:
        """The device residency table as an int32 tensor view [L*E] (shares memory)."""
        base = B.moe_slot_table(self.ctx)
        off = base - self.ws.data_ptr()
        n = self.cfg.L * self.cfg.E
        return self.ws[off:off + 4 * n].view(torch.int32)

    def close(self):
        if getattr(self, "ctx", None):
            torch.cuda.synchronize()
            B.moe_destroy(self.ctx)
            self.ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # -- calls -------------------------------------------------------------
    def set_policy(self, policy, B_P=1.0, B_H=1.0):
        self._chk(B.moe_set_policy(self.ctx, policy, B_P, B_H))

    def set_activations(self, act):
        """MOE_ACT_DEFAULT or MOE_ACT_MXFP6 (MXFP4 weights' large-batch path)."""
        self._chk(B.moe_set_activations(self.ctx, act))

    def calibrate(self):
        bp, bh = ctypes.c_double(), ctypes.c_double()
        self._chk(B.moe_calibrate(self.ctx, ctypes.byref(bp), ctypes.byref(bh)))
        return bp.value, bh.value

    def calibrate_ex(self, T=1):
        """Bandwidth calibration with its breakdown (dict of moe_calibration)."""
        m = B.moe_calibration()
        self._chk(B.moe_calibrate_ex(self.ctx, T, ctypes.byref(m)))
        return m.as_dict()

    def reset_cache(self, stream=None):
        self._chk(B.moe_reset_cache(self.ctx, self.stream_ptr(stream)))

    def route(self, hidden, router_w, bias, ids, w, stream=None):
        T = hidden.shape[0]
        self._chk(B.moe_route(self.ctx, hidden.data_ptr(), router_w.data_ptr(),
                              None if bias is None else bias.data_ptr(), T, ids.data_ptr(), w.data_ptr(),
                              self.stream_ptr(stream)))

    def route_from_logits(self, logits, ids, w, counts, offsets, perm_tok, pos, stream=None):
        T = logits.shape[0]
        self._chk(B.moe_route_from_logits(self.ctx, logits.data_ptr(), T, ids.data_ptr(), w.data_ptr(),
                                          counts.data_ptr(), offsets.data_ptr(), perm_tok.data_ptr(),
                                          pos.data_ptr(), self.stream_ptr(stream)))

    def plan(self, layer, ids, mask_out=None, stream=None):
        info = B.moe_plan_info()
        E = self.cfg.E
        fe = (ctypes.c_int32 * E)()
        fs = (ctypes.c_int32 * E)()
        T = ids.shape[0]
        self._chk(B.moe_plan(self.ctx, layer, ids.data_ptr(), T, None if mask_out is None else mask_out.data_ptr(),
                             ctypes.byref(info), fe, fs, self.stream_ptr(stream)))
        return info, list(fe[:info.q]), list(fs[:info.q])

    def fill(self, layer, experts, slots, copy_stream=None):
        n = len(experts)
        ea = (ctypes.c_int32 * max(n, 1))(*experts)
        sa = (ctypes.c_int32 * max(n, 1))(*slots)
        self._chk(B.slot_pool_fill(self.ctx, layer, ea, sa, n, self.stream_ptr(copy_stream)))

    def admit(self, layer, experts, copy_stream=None):
        n = len(experts)
        ea = (ctypes.c_int32 * max(n, 1))(*experts)
        self._chk(B.slot_pool_admit(self.ctx, layer, ea, n, self.stream_ptr(copy_stream)))

    def evict(self, layer, experts):
        n = len(experts)
        ea = (ctypes.c_int32 * max(n, 1))(*experts)
        self._chk(B.slot_pool_evict(self.ctx, layer, ea, n))

    def host_partial(self, layer, hidden_np, ids_np, w_np, mask_np):
        T = hidden_np.shape[0]
        out = np.zeros((T, self.cfg.H), dtype=np.float32)
        hidden_np = np.ascontiguousarray(hidden_np, dtype=np.uint16)
        ids_np = np.ascontiguousarray(ids_np, dtype=np.int32)
        w_np = np.ascontiguousarray(w_np, dtype=np.float32)
        mask_np = np.ascontiguousarray(mask_np, dtype=np.uint32)
        self._chk(B.moe_host_partial(self.ctx, layer, hidden_np.ctypes.data, ids_np.ctypes.data, w_np.ctypes.data,
                                     T, mask_np.ctypes.data, out.ctypes.data))
        return out

    def forward(self, layer, hidden, router_w, bias, slot_row, out, miss_mask=None, host_partial=None, stream=None):
        T = hidden.shape[0]
        self._chk(B.moe_layer_forward(self.ctx, layer, hidden.data_ptr(), router_w.data_ptr(),
                                      None if bias is None else bias.data_ptr(), T,
                                      None if slot_row is None else slot_row.data_ptr(),
                                      None if miss_mask is None else miss_mask.data_ptr(),
                                      None if host_partial is None else host_partial.data_ptr(),
                                      out.data_ptr(), self.stream_ptr(stream)))

    def decode_layer(self, layer, hidden, router_w, bias, out, stream=None, copy_stream=None):
        info = B.moe_plan_info()
        T = hidden.shape[0]
        self._chk(B.moe_decode_layer(self.ctx, layer, hidden.data_ptr(), router_w.data_ptr(),
                                     None if bias is None else bias.data_ptr(), T, out.data_ptr(),
                                     ctypes.byref(info), self.stream_ptr(stream),
                                     self.stream_ptr(copy_stream) if copy_stream is not None
                                     else self.stream_ptr(stream)))
        return info

    def decode_layer_async(self, layer, hidden, router_w, bias, out, stream=None, host_stream=None):
        """Enqueues the layer with no host read of the plan (capturable)."""
        T = hidden.shape[0]
        hs = host_stream if host_stream is not None else self._host_stream()
        self._chk(B.moe_decode_layer_async(self.ctx, layer, hidden.data_ptr(), router_w.data_ptr(),
                                           None if bias is None else bias.data_ptr(), T, out.data_ptr(),
                                           self.stream_ptr(stream), self.stream_ptr(hs)))

    def _host_stream(self):
        if getattr(self, "_hs", None) is None:
            self._hs = torch.cuda.Stream(device=self.device)
        return self._hs

    def resize(self, n_slots, in_place=False, stream=None):
        """Rebuilds the cache with n_slots slots (safe point).  in_place keeps
        the current allocation (n_slots must fit it); otherwise a new pool is
        allocated and the old one released after the call."""
        need = max(n_slots, 1) * self.S
        if in_place:
            if need > self.slots.numel():
                raise ValueError("in-place rebuild larger than the current slot pool")
            pool = self.slots
        else:
            pool = torch.empty(need, dtype=torch.uint8, device=self.device)
        self._chk(B.slot_pool_resize(self.ctx, pool.data_ptr(), pool.numel(), n_slots, self.stream_ptr(stream)))
        self.slots = pool
        self.cfg.n_slots = n_slots

    def plan_stats(self, reset=False):
        out = B.moe_plan_totals()
        self._chk(B.moe_plan_stats(self.ctx, ctypes.byref(out), 1 if reset else 0))
        return out.as_dict()

    def prefill_layer(self, layer, hidden, router_w, bias, out, stream=None, copy_stream=None, double_buffer=True):
        T = hidden.shape[0]
        return self._chk(B.prefill_stream_layer(self.ctx, layer, hidden.data_ptr(), router_w.data_ptr(),
                                                None if bias is None else bias.data_ptr(), T, out.data_ptr(),
                                                self.stream_ptr(stream),
                                                self.stream_ptr(copy_stream) if copy_stream is not None
                                                else self.stream_ptr(stream), 1 if double_buffer else 0))

    def profile_begin(self, max_launches=100000, stages=None):
        """Time launches of the named stages (all when None)."""
        mask = 0
        for i, name in enumerate(B.STAGES):
            if stages is None or name in stages:
                mask |= 1 << i
        self._chk(B.moe_profile_begin(self.ctx, max_launches, mask))

    def profile_end(self):
        p = B.moe_profile()
        self._chk(B.moe_profile_end(self.ctx, ctypes.byref(p)))
        d = p.as_dict()
        d["dropped"] = p.dropped
        return d

    def check_device_error(self):
        return B.moe_check_device_error(self.ctx)
