"""The layer schedule ("图解DeepSeek V4：详细计算流程解析" section 1): 61 layers, the
first three HCA, HCA, CSA, then HCA and CSA alternating, the last layer SWA."""
import pytest

from compressed_sparse_attention_c4a_amd import schedule as S


def test_pro_schedule():
    k = S.attention_kinds()
    assert len(k) == 61
    assert k[:3] == ["hca", "hca", "csa"]
    assert k[-1] == "swa"
    assert (k.count("hca"), k.count("csa"), k.count("swa")) == (31, 29, 1)
    for a, b in zip(k[2:-2], k[3:-1]):          # strict alternation from layer 2 to layer 59
        assert {a, b} == {"hca", "csa"}


def test_short_schedules_keep_the_shape():
    assert S.attention_kinds(4) == ["hca", "hca", "csa", "swa"]
    assert S.attention_kinds(6) == ["hca", "hca", "csa", "hca", "csa", "swa"]
    with pytest.raises(ValueError):
        S.attention_kinds(3)
