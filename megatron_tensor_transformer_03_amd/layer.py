"""One rank's layer forward as a sequence of C-ABI calls (argument marshalling only).

The per-rank hot path of a Megatron-style layer ("Megatron-LM 深度学习与源码分析文档",
part 2 section 2): the QKV ColumnParallelLinear (with RoPE on its Q and K heads
where the model uses it), the attention out-projection
RowParallelLinear (its input, the attention context, is an input here: core
attention is not part of this path), and the MLP with fc1 column-parallel
(bias + GeLU or SwiGLU fused) and fc2 row-parallel.  For an MoE layer the
router and the expert MLPs ("ai阅读megatron", MoELayer forward).

``dims`` uses the keys of ``synth.configs``; ``inputs`` holds device tensors
named as there.  Outputs, and one zero-filled split-K workspace shared by the
step's GEMMs (they run in order on one stream), are allocated once by
``RankForward`` and reused by every ``step()``.
"""
from __future__ import annotations

import megatron_tensor_transformer_03_amd as mtp


class RankForward:
    """Buffers and launch sequence for one workload's per-rank forward on the current device."""

    def __init__(self, dims: dict, inputs: dict):
        import torch
        self.d, self.t = dims, inputs
        dev = next(iter(inputs.values())).device
        bf, f32 = torch.bfloat16, torch.float32
        self.out = {}
        self.ws = None
        if "E" in dims:  # MoE expert MLP (grouped GEMMs; the workspace lets fc2 split the experts' tail tiles)
            T, H, E, F, k = dims["T"], dims["H"], dims["E"], dims["F"], dims["k"]
            self.out.update(offsets=torch.empty(E + 1, dtype=torch.int32, device=dev),
                            token_idx=torch.empty(T * k, dtype=torch.int32, device=dev),
                            token_w=torch.empty(T * k, dtype=f32, device=dev),
                            token_rows=torch.empty(T * k, dtype=torch.int32, device=dev),
                            Z=torch.empty(T * k, F, dtype=bf, device=dev),
                            Y_rows=torch.empty(T * k, H, dtype=f32, device=dev),
                            Y=torch.empty(T, H, dtype=bf, device=dev))
            self.ws = mtp.gemm_workspace(mtp.mtp_moe_plan(T, H, E, F, k)[1], dev)
            return
        M, H, p = dims["M"], dims["H"], dims["p"]
        if "nq" in dims:
            nq_l, ng_l, d = dims["nq"] // p, dims["ng"] // p, dims["d"]
            self.out["qkv"] = torch.empty(M, (nq_l + 2 * ng_l) * d, dtype=bf, device=dev)
            if "rope" in dims:  # token positions of the rows (one sequence of M tokens)
                self.positions = torch.arange(M, dtype=torch.int32, device=dev)
        if "ctx" in inputs:
            if p == 1:
                self.out["attn_out"] = torch.empty(M, H, dtype=bf, device=dev)
            else:
                self.out["attn_partial"] = torch.empty(M, H, dtype=f32, device=dev)
        F_l = dims["F"] // p
        self.out["Z"] = torch.empty(M, F_l, dtype=bf, device=dev)
        # the step's GEMMs as (M, N, K, act) in mtp_gemm_plan's terms: one workspace fits them all
        shapes = [(M, H, F_l, mtp.ACT_NONE), (M, inputs["W1t"].shape[0] // (p if dims["ranks"] == "all" else 1), H,
                                              dims["act"])]
        if "nq" in dims:
            shapes.append((M, self.out["qkv"].shape[1], H, mtp.ACT_NONE))
        if "ctx" in inputs:
            shapes.append((M, H, inputs["ctx"].shape[1], mtp.ACT_NONE))
        self.ws = mtp.workspace_for(shapes, dev)
        if dims["ranks"] == "all":
            self.out["Y"] = torch.empty(M, H, dtype=bf, device=dev)
            if p > 1:  # fp32 sum over the shards
                self.out["Yacc"] = torch.empty(M, H, dtype=f32, device=dev)
        else:
            self.out["mlp_partial"] = torch.empty(M, H, dtype=f32, device=dev)

    def calls(self):
        """The forward's launches in order, as (label, thunk) pairs; each thunk enqueues one C-ABI call on the
        current stream (so a caller can also capture them into graphs)."""
        d, t, o = self.d, self.t, self.out
        if "E" in d:
            return [("route", lambda: mtp.mtp_moe_route(t["logits"], d["k"], o["offsets"], o["token_idx"],
                                                          o["token_w"], o["token_rows"])),
                    ("moe_mlp", lambda: mtp.mtp_moe_mlp_forward(t["X"], d["E"], d["F"], d["k"], o["offsets"],
                                                                o["token_idx"], o["token_w"], o["token_rows"],
                                                                t["W1t"], t["W2t"], o["Z"], o["Y_rows"], o["Y"],
                                                                workspace=self.ws))]
        p = d["p"]
        out = []
        if "nq" in d:
            out.append(("qkv", lambda: mtp.mtp_qkv_forward(t["X"], t["Wqkv_t"], t.get("bqkv"), d["nq"] // p,
                                                           d["ng"] // p, d["d"], o["qkv"], workspace=self.ws)))
        if "rope" in d:
            r = d["rope"]
            out.append(("rope", lambda: mtp.mtp_rope_qk(o["qkv"], self.positions, d["nq"] // p, d["ng"] // p, d["d"],
                                                        r["rotary_dim"], r["base"], r["interleaved"])))
        if "ctx" in t:
            if p == 1:  # the whole layer: the all-reduce is the identity, bias added here
                out.append(("out_proj", lambda: mtp.mtp_row_linear_partial(t["ctx"], t["Wo_t"], None, False,
                                                                           t.get("bo"), o["attn_out"],
                                                                           workspace=self.ws)))
            else:       # this rank's fp32 partial of the all-reduce
                out.append(("out_proj", lambda: mtp.mtp_row_linear_partial(t["ctx"], t["Wo_t"], o["attn_partial"],
                                                                           workspace=self.ws)))
        if d["ranks"] == "all" and p > 1:
            # every shard in turn; the all-reduce is the fp32 sum in rank order
            out.append(("mlp", lambda: mtp.mtp_mlp_forward(t["X"], t["W1t"], t.get("b1"), t["W2t"], t.get("b2"),
                                                           d["act"], p, 0, p, o["Z"], o["Yacc"], o["Y"],
                                                           workspace=self.ws)))
        else:
            # one shard (p = 1: the whole MLP): fc1 column linear with bias + activation fused, then fc2 as a
            # row-parallel partial; with p = 1 the sum over shards is the identity and b2 is added in its epilogue
            out.append(("fc1", lambda: mtp.mtp_column_linear(t["X"], t["W1t"], t.get("b1"), o["Z"], d["act"],
                                                             workspace=self.ws)))
            if p == 1:
                out.append(("fc2", lambda: mtp.mtp_row_linear_partial(o["Z"], t["W2t"], None, False, t.get("b2"),
                                                                      o["Y"], workspace=self.ws)))
            else:
                out.append(("fc2", lambda: mtp.mtp_row_linear_partial(o["Z"], t["W2t"], o["mlp_partial"],
                                                                      workspace=self.ws)))
        return out

    def step(self, mark=None):
        """Enqueue one forward.  ``mark(label)``, if given, is called before each launch and once at the end
        (label None): a caller can record stream events there to time each GEMM."""
        mark = mark or (lambda label: None)
        for label, fn in self.calls():
            mark(label)
            fn()
        mark(None)
        return self.out


class PreNormLayer:
    """A whole pre-norm layer at TP = 1, core attention aside (its context is an input): the layer spec of the
    pages ("快速入门", model implementation: input norm fused into the QKV linear, self_attn_bda,
    pre_mlp_layernorm, MLP, mlp_bda) as C-ABI calls:
        stats1 = norm(X);  qkv = norm-folded QKV linear (+ RoPE);  h1 = X + dropout(ctx . Wo^T + bo)
        stats2 = norm(h1); Z = act(norm-folded fc1(h1));           out = h1 + dropout(Z . W2^T + b2)
    The norms' scales and shifts are folded into copies of the column weights once, at construction
    (mtp_norm_fold_weights), as after each weight update.  ``extra`` holds device tensors g1, beta1, g2,
    beta2 (beta None for RMSNorm), keep1, keep2 (packed keep bits) and the float p_drop; ``kind`` is
    mtp.NORM_LAYER or mtp.NORM_RMS."""

    def __init__(self, dims: dict, inputs: dict, extra: dict, kind: int = mtp.NORM_LAYER, eps: float = 1e-5):
        import torch
        if dims.get("p", 1) != 1 or "ctx" not in inputs or "nq" not in dims:
            raise ValueError("the composed layer needs a TP = 1 dense workload with attention context")
        self.d, self.t, self.x, self.kind, self.eps = dims, inputs, extra, kind, eps
        dev = inputs["X"].device
        bf, f32 = torch.bfloat16, torch.float32
        M, H = dims["M"], dims["H"]
        ln = kind == mtp.NORM_LAYER

        def fold(Wt, g, beta, bias):
            Wf = torch.empty_like(Wt)
            cs = torch.empty(Wt.shape[0], dtype=f32, device=dev) if ln else None
            bf_ = torch.empty(Wt.shape[0], dtype=f32, device=dev)
            mtp.mtp_norm_fold_weights(Wt, g, beta if ln else None, bias, Wf, cs, bf_)
            return Wf, cs, bf_

        self.qkv_w = fold(inputs["Wqkv_t"], extra["g1"], extra["beta1"], inputs.get("bqkv"))
        self.fc1_w = fold(inputs["W1t"], extra["g2"], extra["beta2"], inputs.get("b1"))
        nq, ng, d = dims["nq"], dims["ng"], dims["d"]
        act = dims["act"]
        F = dims["F"]
        self.out = dict(stats1=torch.empty(M, 2, dtype=f32, device=dev), stats2=torch.empty(M, 2, dtype=f32, device=dev),
                        qkv=torch.empty(M, (nq + 2 * ng) * d, dtype=bf, device=dev),
                        h1=torch.empty(M, H, dtype=bf, device=dev),
                        Z=torch.empty(M, F, dtype=bf, device=dev),
                        out=torch.empty(M, H, dtype=bf, device=dev))
        if "rope" in dims:
            self.positions = torch.arange(M, dtype=torch.int32, device=dev)
        self.act = act
        self.ws = mtp.workspace_for([(M, self.out["qkv"].shape[1], H, mtp.ACT_NONE), (M, H, inputs["ctx"].shape[1],
                                     mtp.ACT_NONE), (M, inputs["W1t"].shape[0], H, act), (M, H, F, mtp.ACT_NONE)],
                                    dev)

    def calls(self):
        d, t, x, o = self.d, self.t, self.x, self.out
        out = [("norm1", lambda: mtp.mtp_norm_stats(t["X"], o["stats1"], self.kind, self.eps)),
               ("qkv", lambda: mtp.mtp_norm_column_linear(t["X"], o["stats1"], *self.qkv_w, o["qkv"],
                                                          workspace=self.ws))]
        if "rope" in d:
            r = d["rope"]
            out.append(("rope", lambda: mtp.mtp_rope_qk(o["qkv"], self.positions, d["nq"], d["ng"], d["d"],
                                                        r["rotary_dim"], r["base"], r["interleaved"])))
        out += [("attn_bda", lambda: mtp.mtp_row_linear_bda(t["ctx"], t["Wo_t"], t["X"], o["h1"], bias=t.get("bo"),
                                                             keep=x["keep1"], p_drop=x["p_drop"], workspace=self.ws)),
                ("norm2", lambda: mtp.mtp_norm_stats(o["h1"], o["stats2"], self.kind, self.eps)),
                ("fc1", lambda: mtp.mtp_norm_column_linear(o["h1"], o["stats2"], *self.fc1_w, o["Z"], self.act,
                                                           workspace=self.ws)),
                ("mlp_bda", lambda: mtp.mtp_row_linear_bda(o["Z"], t["W2t"], o["h1"], o["out"], bias=t.get("b2"),
                                                           keep=x["keep2"], p_drop=x["p_drop"], workspace=self.ws))]
        return out

    def step(self, mark=None):
        mark = mark or (lambda label: None)
        for label, fn in self.calls():
            mark(label)
            fn()
        mark(None)
        return self.out
