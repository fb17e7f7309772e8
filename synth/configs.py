"""The five synthetic workloads: shapes, tensor keys (seeds) and value distributions.

Shapes follow the model descriptions on the pages ("ai阅读megatron", 模型实现:
GPT-3 175B, LLaMA-3 70B, Mixtral 8x7B; "Megatron-LM 深度学习与源码分析文档",
part 2 section 2: fc1 width 4H/TP, heads/TP per rank).  Values are synthetic:
activations ~N(0,1), weights ~N(0, 0.02^2), biases ~N(0, 0.01^2) where a
bias exists.  Weight tensors are stored [out x in] (F.linear layout).  A
tensor's key is 1000 * workload + its number.  No data set or trained weight
is involved; the generator is defined in gen.c.
"""
from __future__ import annotations

from dataclasses import dataclass, field

ACT_NONE, ACT_GELU, ACT_SWIGLU = 0, 1, 2
W_SIGMA, B_SIGMA = 0.02, 0.01


@dataclass(frozen=True)
class T:
    """One input tensor: storage shape, generator key, distribution ('normal' with sigma, or 'f32')."""
    shape: tuple
    seed: int
    sigma: float = 1.0
    kind: str = "normal"

    @property
    def numel(self) -> int:
        n = 1
        for s in self.shape:
            n *= s
        return n


@dataclass
class Workload:
    name: str
    desc: str
    tensors: dict = field(default_factory=dict)
    dims: dict = field(default_factory=dict)
    gemms: list = field(default_factory=list)  # (label, M, N, K) as computed (N counts gate+up for SwiGLU)

    @property
    def flop(self) -> int:
        return sum(2 * m * n * k for _, m, n, k in self.gemms)


def tiny_gelu_mlp_tp2() -> Workload:
    M, H, F, p = 128, 256, 1024, 2
    w = Workload("tiny_gelu_mlp_tp2",
                 "GeLU MLP, TP=2, both shards on one device: X[128x256], fc1 2x512, fc2 2x512")
    w.dims = dict(M=M, H=H, F=F, p=p, act=ACT_GELU, ranks="all")
    w.tensors = dict(X=T((M, H), 1001), W1t=T((F, H), 1002, W_SIGMA), b1=T((F,), 1003, B_SIGMA),
                     W2t=T((H, F), 1004, W_SIGMA), b2=T((H,), 1005, B_SIGMA))
    w.gemms = [("fc1", M, F // p, H)] * p + [("fc2", M, H, F // p)] * p
    return w


def gpt345m_tp1() -> Workload:
    M, H, nh, d, F = 4096, 1024, 16, 64, 4096
    w = Workload("gpt345m_layer_tp1_4096tok",
                 "GPT-345M-shaped layer, TP=1: H=1024, 16 heads x 64, ffn 4096 GeLU, 4096 tokens")
    w.dims = dict(M=M, H=H, nq=nh, ng=nh, d=d, F=F, p=1, act=ACT_GELU, ranks="all")
    nqkv = (nh + 2 * nh) * d
    w.tensors = dict(X=T((M, H), 2001), Wqkv_t=T((nqkv, H), 2002, W_SIGMA), bqkv=T((nqkv,), 2003, B_SIGMA),
                     ctx=T((M, nh * d), 2004), Wo_t=T((H, nh * d), 2005, W_SIGMA), bo=T((H,), 2006, B_SIGMA),
                     W1t=T((F, H), 2007, W_SIGMA), b1=T((F,), 2008, B_SIGMA),
                     W2t=T((H, F), 2009, W_SIGMA), b2=T((H,), 2010, B_SIGMA))
    w.gemms = [("qkv", M, nqkv, H), ("out_proj", M, H, nh * d), ("fc1", M, F, H), ("fc2", M, H, F)]
    return w


def gpt3_175b_tp8_rank0() -> Workload:
    M, H, nh, d, p = 2048, 12288, 96, 128, 8
    F = 4 * H
    nq_l = nh // p
    w = Workload("gpt3_175b_tp8_rank0_2048tok",
                 "GPT-3 175B-shaped layer, rank 0 of TP=8: 12 heads x 128 per rank, fc1 shard 6144 GeLU, 2048 tokens")
    w.dims = dict(M=M, H=H, nq=nh, ng=nh, d=d, F=F, p=p, act=ACT_GELU, ranks="rank0")
    nqkv = 3 * nq_l * d
    F_l = F // p
    w.tensors = dict(X=T((M, H), 3001), Wqkv_t=T((nqkv, H), 3002, W_SIGMA), bqkv=T((nqkv,), 3003, B_SIGMA),
                     ctx=T((M, nq_l * d), 3004), Wo_t=T((H, nq_l * d), 3005, W_SIGMA),
                     W1t=T((F_l, H), 3007, W_SIGMA), b1=T((F_l,), 3008, B_SIGMA),
                     W2t=T((H, F_l), 3009, W_SIGMA))
    w.gemms = [("qkv", M, nqkv, H), ("out_proj", M, H, nq_l * d), ("fc1", M, F_l, H), ("fc2", M, H, F_l)]
    return w


def llama70b_tp8_rank0() -> Workload:
    M, H, nq, ng, d, p, F = 4096, 8192, 64, 8, 128, 8, 28672
    w = Workload("llama70b_gqa_swiglu_tp8_rank0_4096tok",
                 "70B-class GQA/SwiGLU layer, rank 0 of TP=8: 8 q-heads + 1 kv-group per rank, ffn 28672")
    # RoPE on the Q and K heads after the QKV GEMM (rotate half, base 5e5, full head dim), one 4096-token sequence
    w.dims = dict(M=M, H=H, nq=nq, ng=ng, d=d, F=F, p=p, act=ACT_SWIGLU, ranks="rank0",
                  rope=dict(base=500000.0, rotary_dim=d, interleaved=False))
    nqkv = (nq // p + 2 * (ng // p)) * d
    F_l = F // p
    w.tensors = dict(X=T((M, H), 4001), Wqkv_t=T((nqkv, H), 4002, W_SIGMA),
                     W1t=T((2 * F_l, H), 4007, W_SIGMA), W2t=T((H, F_l), 4009, W_SIGMA))
    w.gemms = [("qkv", M, nqkv, H), ("fc1", M, 2 * F_l, H), ("fc2", M, H, F_l)]
    return w


def moe_8x_top2() -> Workload:
    Tn, H, E, F, k = 4096, 4096, 8, 14336, 2
    w = Workload("moe_8expert_top2_4096tok",
                 "MoE expert MLP, 8 experts SwiGLU ffn 14336, top-2 of 4096 tokens, H=4096")
    w.dims = dict(T=Tn, H=H, E=E, F=F, k=k)
    # expert e's weights are rows e*2F..(e+1)*2F of W1t ([gate; up]) and rows e*H..(e+1)*H of W2t
    w.tensors = dict(X=T((Tn, H), 5001), logits=T((Tn, E), 5002, kind="f32"),
                     W1t=T((E * 2 * F, H), 5003, W_SIGMA), W2t=T((E * H, F), 5004, W_SIGMA))
    w.gemms = [("moe_fc1", Tn * k, 2 * F, H), ("moe_fc2", Tn * k, H, F)]
    return w


ALL = [tiny_gelu_mlp_tp2, gpt345m_tp1, gpt3_175b_tp8_rank0, llama70b_tp8_rank0, moe_8x_top2]


def by_index(i: int) -> Workload:
    return ALL[i]()
