"""The seeded input recipes: shapes, position tables and byte counts."""
import numpy as np

import workloads as W


def test_algorithmic_bytes_per_call():
    want = {"tiny_mrope": 6144 + 192,
            "omni_text_prefill": 603979776 + 393216 + 512,
            "qwen35_partial_mixed": 469762048 + 196608 + 1024,
            "chunked_video": 184549376 + 135168,
            "vision_2d": 603979776 + 262144}
    for name, b in want.items():
        assert W.WORKLOADS[name].algorithmic_bytes() == b


def test_qwen35_mixed_positions():
    wl = W.WORKLOADS["qwen35_partial_mixed"]
    pos = W.workload_positions(wl)
    assert pos.shape == (3, 16384) and pos.dtype == np.int32
    assert np.array_equal(pos[:, :512], np.stack([np.arange(512)] * 3))
    img = pos[:, 512:512 + 768]
    assert np.all(img[0] == 512)
    assert np.array_equal(img[1], 512 + np.repeat(np.arange(24), 32))
    assert np.array_equal(img[2], 512 + np.tile(np.arange(32), 24))
    tail = pos[:, 512 + 768:]
    assert tail[0, 0] == 544 and tail[0, -1] == 15647
    assert np.all(tail[0] == tail[1]) and np.all(tail[0] == tail[2])


def test_chunked_video_positions():
    pos = W.workload_positions(W.WORKLOADS["chunked_video"])
    assert pos.shape == (3, 11264)
    vid = pos[:, 1024:1024 + 9216]
    assert vid[:, 0].tolist() == [1024, 1024, 1024]
    assert vid[:, -1].tolist() == [1039, 1047, 1047]
    assert vid[:, 24 * 24].tolist() == [1025, 1024, 1024]      # time is slowest
    assert pos[:, 1024 + 9216].tolist() == [1048] * 3
    assert pos[0, -1] == 1048 + 1023


def test_vision_positions_merge_block_order():
    pos = W.workload_positions(W.WORKLOADS["vision_2d"])
    assert pos.shape == (2, 32768)
    # first merge block of the first image: (0,0) (0,1) (1,0) (1,1)
    assert pos[:, :4].T.tolist() == [[0, 0], [0, 1], [1, 0], [1, 1]]
    # second block starts at column 2
    assert pos[:, 4].tolist() == [0, 2]
    assert pos.max() == 63
    assert np.array_equal(pos[:, :4096], pos[:, 4096:8192])
    assert W.vision_cu_seqlens().tolist() == list(range(0, 32769, 4096))


def test_inputs_are_seeded_and_truncation_is_a_prefix_of_positions():
    a = W.make_inputs("omni_text_prefill", T=64)
    b = W.make_inputs("omni_text_prefill", T=64)
    assert np.array_equal(a["q"], b["q"]) and np.array_equal(a["wq"], b["wq"])
    assert a["q"].dtype == np.uint16 and a["q"].shape == (64, 32, 128)
    assert np.array_equal(a["pos"], np.stack([np.arange(64)] * 3))
    t = W.make_inputs("tiny_mrope")
    assert t["q"].dtype == np.float32 and t["pos"].shape == (3, 16)
    assert t["pos"].min() >= 0 and t["pos"].max() < 32
