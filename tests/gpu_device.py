"""Device staging of a synthetic problem and calls through the library binding.

Used by the GPU tests and by bench.py; it does not touch the oracle."""
import numpy as np
import torch

import split_kv_asynchronous_amd as fd

def to_device(arr, kind):
    t = torch.from_numpy(np.ascontiguousarray(arr))
    if kind == "bf16":
        t = t.view(torch.int16).view(torch.bfloat16)
    elif kind == "e4m3fn":
        t = t.view(torch.float8_e4m3fn)
    return t.cuda()


class DeviceProblem:
    """A synthetic problem resident in GPU memory (inputs, workspace, outputs)."""

    def __init__(self, prob, out_dtype="f32", plan=0):
        self.prob = prob
        self.plan = plan
        self.q = to_device(prob.q, prob.q_dtype)
        self.k = to_device(prob.k_cache, prob.kv_dtype)
        self.v = to_device(prob.v_cache, prob.kv_dtype)
        self.seq_lens = torch.from_numpy(prob.seq_lens).cuda()
        self.block_table = None if prob.block_table is None else torch.from_numpy(
            prob.block_table).cuda()
        self.k_scale = None if prob.k_scale is None else torch.from_numpy(prob.k_scale).cuda()
        self.v_scale = None if prob.v_scale is None else torch.from_numpy(prob.v_scale).cuda()
        self.out_dtype = out_dtype
        B, Hq, D = prob.q.shape
        self.out = torch.empty((B, Hq, D), device="cuda",
                               dtype=torch.float32 if out_dtype == "f32" else torch.bfloat16)
        self.flags = torch.empty((B, Hq), device="cuda", dtype=torch.uint8)
        desc = self.desc()
        self.workspace = torch.empty(max(fd.fd_attn_workspace_size(desc), 256), device="cuda",
                                     dtype=torch.uint8)

    def desc(self):
        p = self.prob
        return fd.make_desc(batch=p.batch, num_q_heads=p.num_q_heads, num_kv_heads=p.num_kv_heads,
                            max_seq_len=p.max_seq_len, chunk_size=p.chunk_size,
                            page_size=p.page_size,
                            max_blocks_per_seq=0 if p.block_table is None else p.block_table.shape[1],
                            num_pages=p.k_cache.shape[0] if p.page_size else 0, scale=p.scale,
                            q_dtype=p.q_dtype, kv_dtype=p.kv_dtype, out_dtype=self.out_dtype,
                            plan=self.plan)

    def run(self, phi=None, a=None, b=None, stream=None, stage_events=None):
        # arguments are marshalled once per workspace (tests may swap it)
        call = getattr(self, "_call", None)
        if call is None or call.workspace is not self.workspace:
            p = self.prob
            call = self._call = fd.prepare_decode(
                self.q, self.k, self.v, self.seq_lens, self.block_table, p.phi, p.a, p.b,
                self.out, self.flags, chunk_size=p.chunk_size, max_seq_len=p.max_seq_len,
                num_kv_heads=p.num_kv_heads, page_size=p.page_size, scale=p.scale,
                k_scale=self.k_scale, v_scale=self.v_scale, workspace=self.workspace,
                q_dtype=p.q_dtype, kv_dtype=p.kv_dtype, out_dtype=self.out_dtype, plan=self.plan)
        return call(phi=phi, a=a, b=b, stream=stream, stage_events=stage_events)

    def results(self):
        torch.cuda.synchronize()
        out = self.out.float().cpu().numpy().reshape(-1, self.prob.head_dim).astype(np.float64)
        return out, self.flags.cpu().numpy().reshape(-1)

    def recomputed(self):
        torch.cuda.synchronize()
        return int(self.workspace[:4].cpu().view(torch.int32).item())




class DevicePrefill:
    """A synthetic prefill problem resident in GPU memory."""

    def __init__(self, prob, out_dtype="f32"):
        self.prob = prob
        self.q = to_device(prob.q, "bf16")
        self.k = to_device(prob.k, prob.cache_dtype)
        self.v = to_device(prob.v, prob.cache_dtype)
        self.kv_lens = torch.from_numpy(prob.kv_lens).cuda()
        self.block_table = None if prob.block_table is None else torch.from_numpy(prob.block_table).cuda()
        self.k_scale = None if prob.k_scale is None else torch.from_numpy(prob.k_scale).cuda()
        self.v_scale = None if prob.v_scale is None else torch.from_numpy(prob.v_scale).cuda()
        self.out_dtype = out_dtype
        self.out = torch.empty(prob.q.shape, device="cuda",
                               dtype=torch.float32 if out_dtype == "f32" else torch.bfloat16)
        self.flags = torch.empty(prob.q.shape[:3], device="cuda", dtype=torch.uint8)

    def run(self, phi=None, a=None, b=None, stream=None, stage_events=None):
        p = self.prob
        return fd.fd_attn_prefill(self.q, self.k, self.v, self.kv_lens,
                                  p.phi if phi is None else phi, p.a if a is None else a,
                                  p.b if b is None else b, self.out, self.flags,
                                  num_kv_heads=p.num_kv_heads, scale=p.scale,
                                  out_dtype=self.out_dtype, stream=stream,
                                  stage_events=stage_events, block_table=self.block_table,
                                  page_size=p.page_size,
                                  max_seq_len=p.max_seq_len if p.page_size else None,
                                  k_scale=self.k_scale, v_scale=self.v_scale)

    def results(self):
        torch.cuda.synchronize()
        out = self.out.float().cpu().numpy().reshape(-1, self.prob.head_dim).astype(np.float64)
        return out, self.flags.cpu().numpy().reshape(-1)
