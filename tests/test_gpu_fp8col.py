"""GPU parity of the fused MXFP4-rows -> FP8-columns conversion (expert weight
gradient) against the CPU oracle: bit-exact E4M3 bytes and fp32 scales, for ragged
expert splits (empty experts, single tokens, every start offset modulo 16, partial
groups), ragged column tiles, NaN / zero / extreme-scale blocks, every code at every
shift into the E4M3 subnormal range, and the 65536 x 7168, 256-expert buffer."""
import numpy as np
import pytest
import torch

from mxfp4_microscaling_quantization_amd import mxq, workloads
from oracle import fp8, mx
from tests.gpu_helpers import assert_equal_bits, require_gpu, u8

pytestmark = pytest.mark.gpu

SENTINEL = 0xA5


def run(codes, e8m0, offsets, ld_extra=0):
    """Runs the kernel with outputs prefilled by a sentinel; returns q8 [C, ld] and
    the scale bits [C, S]."""
    dev = require_gpu()
    R, C = codes.shape[0], codes.shape[1] * 2
    E = len(offsets) - 1
    ld = (R + 15) // 16 * 16 + ld_extra
    q8 = torch.full((C, ld), SENTINEL, dtype=torch.uint8, device=dev)
    s = torch.full((C, mxq.fp8_col_scale_slots(R, E) + 3), float("nan"), dtype=torch.float32, device=dev)
    s.view(torch.int32).fill_(0x5A5A5A5A)
    off = torch.tensor(np.asarray(offsets, dtype=np.int64), device=dev)
    mxq.mxq_fp4_row_to_fp8_col(torch.as_tensor(codes).to(dev), torch.as_tensor(e8m0).to(dev), off, out=(q8, s))
    return u8(q8), s.cpu().view(torch.int32).numpy().view(np.uint32)


def check(codes, e8m0, offsets, what, ld_extra=0):
    codes, e8m0 = np.asarray(codes), np.asarray(e8m0)
    R = codes.shape[0]
    q8, s = run(codes, e8m0, offsets, ld_extra)
    rq, rs = fp8.mxfp4_rows_to_fp8_cols(codes, e8m0, offsets)
    G = rs.shape[1]
    assert_equal_bits(q8[:, :R], rq, what + " E4M3")
    assert_equal_bits(s[:, :G], rs, what + " scales")
    assert (q8[:, R:] == SENTINEL).all(), what + ": bytes past the last token were written"
    assert (s[:, G:] == 0x5A5A5A5A).all(), what + ": scale entries past the last group were written"


def random_codes(rng, R, C, e_lo=115, e_hi=135, p_zero=0.15):
    nib = rng.integers(0, 16, (R, C)).astype(np.uint8)
    nib[rng.random((R, C)) < p_zero] &= 8
    return mx.pack_nibbles(nib), rng.integers(e_lo, e_hi, (R, C // 32)).astype(np.uint8)


def offsets_of(counts):
    return np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)


def test_single_group_and_single_expert():
    rng = np.random.default_rng(0)
    for R, C in ((128, 256), (1, 32), (16, 64), (300, 512)):
        p, e = random_codes(rng, R, C)
        check(p, e, [0, R], f"one expert {R}x{C}")


def test_ragged_experts_every_start_offset():
    # expert starts at every residue modulo 16, sizes from 0 to 300 tokens
    rng = np.random.default_rng(1)
    counts = [0, 1, 5, 0, 130, 128, 3, 17, 15, 16, 129, 255, 256, 257, 31, 300, 2, 0, 9, 14,
              35, 33, 33, 37, 35, 33, 33]
    off = offsets_of(counts)
    assert len(set((off % 16).tolist())) == 16
    p, e = random_codes(rng, int(off[-1]), 288)  # 256 + a 32-column tile
    check(p, e, off, "ragged experts", ld_extra=16)


def test_dirichlet_split():
    rng = np.random.default_rng(2)
    counts = workloads.expert_counts(2048, 64, 3)
    p, e = random_codes(rng, 2048, 320)
    check(p, e, offsets_of(counts), "dirichlet 64 experts")


def test_nan_zero_and_sign_blocks():
    rng = np.random.default_rng(3)
    R, C = 260, 96
    nib = rng.integers(0, 16, (R, C)).astype(np.uint8)
    e = rng.integers(118, 130, (R, C // 32)).astype(np.uint8)
    e[5, 1] = 255            # NaN block in the first group of expert 0
    e[200, 0] = 255          # NaN block in a later group
    nib[130:258, 64:96] &= 8  # a whole group of one column block: signed zeros
    e[130:258, 2] = 0         # with the zero-block byte
    nib[10:20, :] = 8         # rows of -0
    check(mx.pack_nibbles(nib), e, [0, 130, 258, 260], "nan / zero blocks")


def test_extreme_scale_bytes_take_the_exact_path():
    # nonzero blocks with bytes outside [10, 252]: tiny values (fp32 subnormal
    # scales) and values near the top of the fp32 range
    rng = np.random.default_rng(4)
    for lo, hi in ((0, 12), (245, 255), (0, 255)):
        p, e = random_codes(rng, 200, 64, lo, hi)
        check(p, e, [0, 77, 200], f"scale bytes {lo}..{hi - 1}")


def test_every_code_at_every_shift():
    # one group per column: a top element 6 * 2^0 in row 0, then rows whose block
    # exponent sits d = 0..20 binades lower holding all 16 codes; covers the normal
    # range, the subnormal range with its ties, and the flush to zero
    rows = []
    es = []
    top = np.zeros(32, np.uint8)
    top[:] = 7
    rows.append(top)
    es.append(127)
    for d in range(0, 21):
        r = np.arange(32, dtype=np.uint8) % 16
        rows.append(r)
        es.append(127 - d)
    nib = np.stack(rows)
    e = np.array(es, np.uint8)[:, None]
    check(mx.pack_nibbles(nib), e, [0, nib.shape[0]], "codes x shifts")


def test_full_65536x7168_256_experts_sampled():
    # the MoE token buffer (65536 tokens, hidden 7168, 256 experts from a
    # Dirichlet(0.5) split): sampled 32-column blocks compared with the oracle
    dev = require_gpu()
    w = workloads.fp8_col_experts()
    R, C = 65536, 7168
    off = torch.tensor(w.offsets, dtype=torch.int64, device=dev)
    q8, s = mxq.mxq_fp4_row_to_fp8_col(w.codes.to(dev), w.e8m0.to(dev), off)
    G = int(fp8.expert_group_offsets(w.offsets)[-1])
    rng = np.random.default_rng(5)
    blocks = sorted(set([0, C // 32 - 1]) | set(rng.choice(C // 32, 2, replace=False).tolist()))
    for b in blocks:
        pc = w.codes[:, 16 * b:16 * b + 16].numpy()
        pe = w.e8m0[:, b:b + 1].numpy()
        rq, rs = fp8.mxfp4_rows_to_fp8_cols(pc, pe, w.offsets)
        assert_equal_bits(u8(q8[32 * b:32 * b + 32]), rq, f"block {b} E4M3")
        assert_equal_bits(s[32 * b:32 * b + 32, :G].cpu().view(torch.int32).numpy().view(np.uint32), rs,
                          f"block {b} scales")


def test_overlapping_offsets_stay_inside_the_buffers():
    # malformed offsets (experts that overlap) give unspecified values but must not
    # write outside the outputs: here the experts' groups add up to more than the
    # scale slots the call sizes for, and every slot past them, and every byte past
    # the last token, must keep its sentinel
    dev = require_gpu()
    rng = np.random.default_rng(17)
    R, C = 300, 64
    codes, e8m0 = random_codes(rng, R, C)
    for offs in ([0, R, 0, R, 0, R], [0, R, 0, R], [0, 290, 10, R]):
        E = len(offs) - 1
        S = mxq.fp8_col_scale_slots(R, E)
        ld = (R + 15) // 16 * 16
        q8 = torch.full((C, ld + 16), SENTINEL, dtype=torch.uint8, device=dev)
        s_big = torch.zeros((C, S + 8), dtype=torch.float32, device=dev)
        s_big.view(torch.int32).fill_(0x5A5A5A5A)
        off = torch.tensor(np.asarray(offs, dtype=np.int64), device=dev)
        mxq.mxq_fp4_row_to_fp8_col(torch.as_tensor(codes).to(dev), torch.as_tensor(e8m0).to(dev), off,
                                   out=(q8[:, :ld], s_big[:, :S]))
        torch.cuda.synchronize()
        assert (u8(q8)[:, R:] == SENTINEL).all(), offs
        assert (s_big.cpu().view(torch.int32).numpy().view(np.uint32)[:, S:] == 0x5A5A5A5A).all(), offs


def test_wide_rows_address_tokens_in_64_bits():
    # 128 tokens of 3 * 2^25 columns: the codes of token 86 and later lie more than
    # 2^32 bytes past the group's first token, so token offsets must be formed in 64
    # bits; sampled column tiles at both ends and in the middle against the oracle
    dev = require_gpu()
    R, C = 128, 3 * 2 ** 25
    g = torch.Generator(device=dev)
    g.manual_seed(5)
    codes = torch.randint(0, 256, (R, C // 2), dtype=torch.uint8, device=dev, generator=g)
    e8m0 = torch.randint(115, 135, (R, C // 32), dtype=torch.uint8, device=dev, generator=g)
    off = torch.tensor([0, 40, R], dtype=torch.int64, device=dev)
    q8, s = mxq.mxq_fp4_row_to_fp8_col(codes, e8m0, off)
    torch.cuda.synchronize()
    for c0 in (0, C // 2 + 256 * 7, C - 256):
        sl = slice(c0, c0 + 256)
        pc = u8(codes[:, c0 // 2:(c0 + 256) // 2])
        pe = u8(e8m0[:, c0 // 32:(c0 + 256) // 32])
        rq, rs = fp8.mxfp4_rows_to_fp8_cols(pc, pe, np.array([0, 40, R], dtype=np.int64))
        assert_equal_bits(u8(q8[sl]), rq, f"wide rows E4M3, columns {c0}..")
        assert_equal_bits(s[sl, :rs.shape[1]].cpu().view(torch.int32).numpy().view(np.uint32), rs,
                          f"wide rows scales, columns {c0}..")
    del codes, e8m0, q8, s
    torch.cuda.empty_cache()
