"""Pins for the byte accounting (no GPU): per-token KV sizes the pages print."""
import numpy as np

from paged_kv_cache_65_amd import accounting as acc


def test_llama7b_mha_fp16_is_512_kib_per_token():
    # "KV Cache Explained Like You're an LLM Engineer", section "Why Recomputing
    # Attention is Inefficient": 2 x 32 x 32 x 128 x 2 = 524,288 bytes; and
    # "Inference serving: the KV-cache machine": a 2048-token context is 1 GB.
    assert acc.kv_bytes_per_token(32, 32, 128, 2) == 524_288
    assert acc.kv_bytes_per_token(32, 32, 128, 2) * 2048 == 2 ** 30


def test_llama3_8b_gqa_is_128_kib_per_token():
    # "Inference serving: the KV-cache machine": 2 x 32 x 8 x 128 x 2 B = 128 KiB/token
    assert acc.kv_bytes_per_token(32, 8, 128, 2) == 131_072


def test_70b_gqa_is_320_kib_per_token():
    # "Modern AI Infrastructure and Agentic System Design", section 9.1:
    # 2 x 80 x 8 x 128 x 2 = 327,680 bytes; 32,000 tokens ~ 10 GiB
    b = acc.kv_bytes_per_token(80, 8, 128, 2)
    assert b == 327_680
    assert abs(b * 32_000 / 2 ** 30 - 9.77) < 0.01


def test_decode_bytes_single_layer_and_shared_prefix():
    lens = np.array([2048] * 8)
    b = acc.decode_algorithmic_bytes(lens, 32, 32, 128, "f16", "f16")
    assert b["kv_unique"] == 8 * 2048 * 2 * 32 * 128 * 2
    assert b["tables"] == 4 * 8 * 128 and b["q"] == b["out"] == 8 * 32 * 128 * 2
    sh = acc.decode_algorithmic_bytes([512 + 10, 512 + 20], 32, 8, 128, "bf16", "bf16",
                                      shared_tokens=512)
    per_tok = 2 * 8 * 128 * 2
    assert sh["kv_logical"] == (522 + 532) * per_tok
    assert sh["kv_unique"] == (512 + 30) * per_tok
    assert acc.decode_flops([3, 5], 4, 64) == 4 * 64 * 4 * 8


def test_windowed_tokens_and_blocks_hand_counted():
    # L = 5, W = 2: positions 2..4 (3 tokens) in block 0.  L = 40, W = 20:
    # positions 19..39 (21 tokens) in blocks 1, 2.  L = 17, W = 0: no window,
    # 17 tokens in 2 blocks.  L = 0: nothing.  L = 33, W = 16: positions
    # 16..32 (17 tokens) in blocks 1, 2.
    toks, blks = acc.attended([5, 40, 17, 0, 33], window=0)
    assert toks.tolist() == [5, 40, 17, 0, 33] and blks.tolist() == [1, 3, 2, 0, 3]
    toks, blks = acc.attended([5, 40, 0, 33], window=2)  # L = 33: positions 30..32, blocks 1 and 2
    assert toks.tolist() == [3, 3, 0, 3] and blks.tolist() == [1, 1, 0, 2]
    toks, blks = acc.attended([40, 33], window=20)
    assert toks.tolist() == [21, 21] and blks.tolist() == [2, 3]
    toks, blks = acc.attended([33], window=16)
    assert toks.tolist() == [17] and blks.tolist() == [2]
    b = acc.decode_algorithmic_bytes([40, 33], 8, 2, 64, "bf16", "f32", window=20)
    assert b["kv_unique"] == (21 + 21) * 2 * 2 * 64 * 2
    assert b["tables"] == 4 * (2 + 3)
