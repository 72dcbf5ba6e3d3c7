"""GPU parity of the per-group FP8 FFN calls against the fp64 oracle.

Bars:
- quantisers of given inputs (rows, weight blocks) and the residual sum of
  the add & norm: bit-exact codes and scales;
- GEMM: the oracle is exact on the same codes and scales.  The block-scaled
  fp8 MFMA sums each lane's 32 products aligned to the largest of them with
  13 fraction bits below it (a product under 2^-13 of the largest vanishes;
  measured on gfx950) and adds those partial sums in fp32, so one group of 32
  loses less than 32 * 2^-13 = 2^-8 of its largest product, and the output's
  bf16 rounding adds at most half an ulp, 2^-8 |C|:
  |C - C_ref| <= 2^-8 |C_ref| + 2^-8 (1 + 2^-7) sum|a b| per element.  When
  every product's bits fit the window (exponent fields 6..9, so products
  within 2^6 of each other, each with 8 significant bits) nothing is lost,
  and the bar is the rounding alone plus fp32:
  |C - C_ref| <= 2^-8 |C_ref| + 2^-20 sum|a b|;
- outputs quantised from float32 values the kernel computes (add & norm,
  SwiGLU) decide their codes in float32 where the oracle's values are fp64,
  so codes may differ where a value sits at a rounding boundary: every
  dequantised value lies within one grid spacing of the oracle's value
  (|q - y| <= |y| / 8 + 2^(e - 9)), every group exponent within 1 of the
  oracle's, and at least 99.9 % of exponents equal;
- the chained FFN block against the oracle's chain: max |out - ref| /
  max |ref| <= 2e-2.
"""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import bits, need_gpu, say

pytestmark = pytest.mark.gpu


def _deq_rows(codes, scales):
    """[M, K] codes with [K/128, M] E8M0 scales -> fp64 values"""
    v = torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn).double().numpy()
    e = scales.T.astype(np.float64) - 127.0
    return v * np.repeat(2.0 ** e, 128, axis=1)


def _check_quantised(codes, scales, y_ref, label):
    """codes/scales (GPU, from float32 values) against fp64 values y_ref"""
    q = _deq_rows(codes, scales)
    e = np.repeat(scales.T.astype(np.float64) - 127.0, 128, axis=1)
    bound = np.abs(y_ref) / 8 + 2.0 ** (e - 9)
    viol = np.abs(q - y_ref) > bound
    assert not viol.any(), (label, int(viol.sum()), float(np.abs(q - y_ref).max()))
    M, K = y_ref.shape
    amax = np.abs(y_ref.reshape(M, K // 128, 128)).max(axis=2)          # [M, G]
    import oracle
    e_ref = np.vectorize(oracle.e8m0_exponent)(amax).T                   # [G, M]
    de = np.abs(scales.astype(np.int64) - 127 - e_ref)
    assert de.max() <= 1, (label, int(de.max()))
    assert (de == 0).mean() >= 0.999, (label, float((de == 0).mean()))


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("M,K,ld", [(1, 128, 128), (37, 384, 384), (300, 4096, 4104), (5, 12288, 12288)])
def test_fp8_quant_rows_bit_exact(orc, dtype, M, K, ld):
    D = need_gpu()
    g = torch.Generator().manual_seed(M + K)
    full = torch.randn((M, ld), generator=g) * torch.exp(torch.randn((M, 1), generator=g) * 6)
    full[:, :128][0] = 0.0                                              # one all-zero group
    if M > 3:
        full[2, 128:256] *= 1e-35                                        # subnormal-range codes
    x = full.to(dtype).cuda()
    xv = x[:, :K] if ld != K else x
    say("fp8 quant rows", dtype, M, K, ld)
    codes, scales = D.dllm_fp8_quant_rows(xv)
    torch.cuda.synchronize()
    xh = bits(x)[:, :K]
    ref_c, ref_s = orc.fp8_quant_rows(np.ascontiguousarray(xh), orc.BF16 if dtype == torch.bfloat16 else orc.F32)
    assert np.array_equal(codes.cpu().numpy(), ref_c)
    assert np.array_equal(scales.cpu().numpy(), ref_s)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_fp8_quant_weight_bit_exact(orc, dtype):
    D = need_gpu()
    N, K = 512, 640
    g = torch.Generator().manual_seed(3)
    w = torch.randn((N, K), generator=g) * 0.02
    w[128:256, 256:384] *= 1e4
    w[256:384, :128] = 0
    w = w.to(dtype).cuda()
    say("fp8 quant weight", dtype)
    codes, scales = D.dllm_fp8_quant_weight(w)
    torch.cuda.synchronize()
    ref_c, ref_s = orc.fp8_quant_weight(bits(w), orc.BF16 if dtype == torch.bfloat16 else orc.F32)
    assert np.array_equal(codes.cpu().numpy(), ref_c) and np.array_equal(scales.cpu().numpy(), ref_s)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("M,K", [(1, 128), (77, 4096), (33, 640)])
def test_fp8_addnorm_quant(orc, dtype, M, K):
    D = need_gpu()
    g = torch.Generator().manual_seed(M * 7 + K)
    x = (torch.randn((M, K), generator=g) * 2).to(dtype).cuda()
    r = torch.randn((M, K), generator=g).to(dtype).cuda()
    gm = (1 + 0.1 * torch.randn((K,), generator=g)).to(dtype).cuda()
    say("fp8 addnorm", dtype, M, K)
    res_out, codes, scales = D.dllm_fp8_addnorm_quant(x, r, gm, eps=1e-6)
    torch.cuda.synchronize()
    dt = orc.BF16 if dtype == torch.bfloat16 else orc.F32
    ref_res, y = orc.addnorm(bits(x), bits(r), bits(gm), 1e-6, dt)
    assert np.array_equal(bits(res_out), ref_res)                        # the residual stream, bit-exact
    _check_quantised(codes.cpu().numpy(), scales.cpu().numpy(), y, f"addnorm {dtype} {M}x{K}")
    # no residual: the norm of x itself
    _, codes, scales = D.dllm_fp8_addnorm_quant(x, None, gm, eps=1e-6, write_residual=False)
    torch.cuda.synchronize()
    _, y = orc.addnorm(bits(x), None, bits(gm), 1e-6, dt)
    _check_quantised(codes.cpu().numpy(), scales.cpu().numpy(), y, "addnorm no residual")


WIDE, NARROW = (0, 15), (6, 9)        # exponent fields: every binade; a 4-binade window


def _gemm_case(D, M, N, K, seed, a_lo=115, a_hi=125, w_lo=110, w_hi=120, exps=WIDE):
    a = W.fp8_codes((M, K), seed, "cuda", *exps)
    sa = W.e8m0_codes((K // 128, M), seed + 1, a_lo, a_hi, "cuda")
    w = W.fp8_codes((N, K), seed + 2, "cuda", *exps)
    sw = W.e8m0_codes((N // 128, K // 128), seed + 3, w_lo, w_hi, "cuda")
    return a, sa, w, sw


def _ref_and_abs(orc, a, sa, w, sw, rows=None):
    """the exact product and sum |a b| (the codes with their sign bits cleared)"""
    ah, sah, wh, swh = a.cpu().numpy(), sa.cpu().numpy(), w.cpu().numpy(), sw.cpu().numpy()
    ref = orc.fp8_gemm(ah, sah, wh, swh, rows=rows)
    sabs = orc.fp8_gemm(ah & 0x7F, sah, wh & 0x7F, swh, rows=rows)
    return ref, sabs


def _gemm_check(c, ref, sabs, label, narrow=False):
    c = c.double().cpu().numpy() if isinstance(c, torch.Tensor) else c
    err = np.abs(c - ref)
    acc = 2.0 ** -20 if narrow else 2.0 ** -8 * (1 + 2.0 ** -7)
    bound = 2.0 ** -8 * np.abs(ref) + acc * sabs
    assert (err <= bound).all(), (label, float((err / np.maximum(bound, 1e-300)).max()), float(err.max()))


@pytest.mark.parametrize("exps", [WIDE, NARROW], ids=["wide", "narrow"])
# K = 128, 256, 384, 640 and longer: the 64-wide slices of the product's
# LDS ring run through each of its start and end paths (2, 4, 6, 10 slices)
@pytest.mark.parametrize("M,N,K", [(1, 256, 128), (70, 256, 256), (300, 512, 384), (200, 768, 640),
                                   (256, 768, 4096), (513, 256, 12288), (2048, 1024, 1024)])
def test_fp8_gemm_parity(orc, M, N, K, exps):
    D = need_gpu()
    a, sa, w, sw = _gemm_case(D, M, N, K, seed=M + N + K, exps=exps)
    say("fp8 gemm", M, N, K, exps)
    c = D.dllm_fp8_gemm(a, sa, w, sw)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([np.arange(min(M, 40)), np.arange(max(0, M - 40), M),
                                     np.random.default_rng(M).integers(0, M, 64)]))
    ref, sabs = _ref_and_abs(orc, a, sa, w, sw, rows)
    _gemm_check(c[torch.from_numpy(rows).cuda()], ref, sabs, f"gemm {M}x{N}x{K} {exps}", narrow=exps == NARROW)


def test_fp8_gemm_scales_and_zeros(orc):
    """scale codes over 2^-37 .. 2^33 (A) and 2^-27 .. 2^23 (B) and an all-zero row"""
    D = need_gpu()
    M, N, K = 260, 512, 512
    a, sa, w, sw = _gemm_case(D, M, N, K, seed=11, a_lo=90, a_hi=160, w_lo=100, w_hi=150, exps=NARROW)
    a[5].zero_()
    say("fp8 gemm extreme scales")
    c = D.dllm_fp8_gemm(a, sa, w, sw)
    torch.cuda.synchronize()
    ref, sabs = _ref_and_abs(orc, a, sa, w, sw)
    assert torch.all(c[5] == 0)
    _gemm_check(c, ref, sabs, "gemm extreme scales")


def _swiglu_ref(orc, a, sa, w, sw, rows):
    cr = orc.fp8_gemm(a.cpu().numpy(), sa.cpu().numpy(), w.cpu().numpy(), sw.cpu().numpy(), rows=rows)
    n = cr.shape[1]
    blk = cr.reshape(len(rows), n // 256, 2, 128)
    gate, up = blk[:, :, 0, :].reshape(len(rows), -1), blk[:, :, 1, :].reshape(len(rows), -1)
    return orc.swiglu(gate, up).reshape(len(rows), n // 2)


@pytest.mark.parametrize("M,N,K", [(1, 256, 128), (65, 512, 256), (300, 512, 384), (257, 1024, 4096)])
def test_fp8_gemm_swiglu(orc, M, N, K):
    """on products within 2^6 of each other, where the fp8 MFMA loses
    nothing, so gate and up carry only fp32 error"""
    D = need_gpu()
    a, sa, w, sw = _gemm_case(D, M, N, K, seed=M * 3 + K, a_lo=112, a_hi=118, w_lo=108, w_hi=114,
                              exps=NARROW)
    say("fp8 gemm swiglu", M, N, K)
    codes, scales = D.dllm_fp8_gemm_swiglu(a, sa, w, sw)
    torch.cuda.synchronize()
    rows = np.arange(M)
    y = _swiglu_ref(orc, a, sa, w, sw, rows)
    _check_quantised(codes.cpu().numpy(), scales.cpu().numpy(), y, f"swiglu {M}x{N}x{K}")


def test_fp8_ffn_block_llada_sampled(orc):
    """the FFN of one LLaDA-8B-shaped layer on a 16 x 2048 step (32768 tokens,
    hidden 4096, SwiGLU width 12288), rows sampled: add & norm + quant, Gate-Up
    + SwiGLU + quant, FF-Out, against the oracle's chain from the same bf16
    inputs"""
    D = need_gpu()
    M = 16 * 2048
    x, res, gm, w_gu, w_out = W.ffn_inputs(M, seed=21, device="cuda")
    say("fp8 ffn block llada", M)
    cgu, sgu = D.dllm_fp8_quant_weight(w_gu)
    cout, sout = D.dllm_fp8_quant_weight(w_out)
    r_out, ca, sa = D.dllm_fp8_addnorm_quant(x, res, gm, eps=1e-6)
    ch, sh = D.dllm_fp8_gemm_swiglu(ca, sa, cgu, sgu)
    out = D.dllm_fp8_gemm(ch, sh, cout, sout)
    torch.cuda.synchronize()
    rows = np.random.default_rng(5).choice(M, 24, replace=False)
    rows.sort()
    xr, rr = bits(x[torch.from_numpy(rows).cuda()]), bits(res[torch.from_numpy(rows).cuda()])
    # the oracle's own chain: weights quantised by the oracle, activations from fp64 values
    ogu_c, ogu_s = orc.fp8_quant_weight(bits(w_gu), orc.BF16)
    oo_c, oo_s = orc.fp8_quant_weight(bits(w_out), orc.BF16)
    assert np.array_equal(cgu.cpu().numpy(), ogu_c) and np.array_equal(cout.cpu().numpy(), oo_c)
    _, y = orc.addnorm(xr, rr, bits(gm), 1e-6, orc.BF16)
    ya_c, ya_s = orc.fp8_quant_rows(y, orc.F64)
    n = 2 * W.FFN_INTER
    cr = orc.fp8_gemm(ya_c, ya_s, ogu_c, ogu_s)
    blk = cr.reshape(len(rows), n // 256, 2, 128)
    h = orc.swiglu(blk[:, :, 0, :].reshape(len(rows), -1), blk[:, :, 1, :].reshape(len(rows), -1))
    hc, hs = orc.fp8_quant_rows(h, orc.F64)
    ref = orc.fp8_gemm(hc, hs, oo_c, oo_s)
    got = out[torch.from_numpy(rows).cuda()].double().cpu().numpy()
    e = np.abs(got - ref).max() / np.abs(ref).max()
    assert e <= 2e-2, e
    # row by row as well, so that one wrong row cannot hide behind the
    # largest output.  The chains differ by the bf16 output's rounding (up to
    # 2^-9 relative per element), by the fp8 products' alignment window
    # (under 2^-8 of each 32-product group's largest term) and by the rare
    # fp8 code that float32 puts on the other side of a rounding boundary
    # than float64; measured: relative L2 error 2.1e-3 per row on average,
    # 4.2e-3 at most, over these 24 rows
    rel = np.linalg.norm(got - ref, axis=1) / np.linalg.norm(ref, axis=1)
    assert rel.max() <= 1e-2, rel.max()


def test_fp8_gemm_deterministic():
    D = need_gpu()
    a, sa, w, sw = _gemm_case(D, 600, 512, 1024, seed=31)
    say("fp8 gemm determinism")
    c1 = D.dllm_fp8_gemm(a, sa, w, sw).clone()
    c2 = D.dllm_fp8_gemm(a, sa, w, sw)
    assert torch.equal(c1, c2)
