"""statekv_decode_attention_noalloc, the decoding entry point that allocates
nothing (its split partials live in the library's fixed device scratch),
against statekv_decode_attention (partials in the layer's workspace): two
calls in a row, the second with fewer text queries, each equal bit for bit
to the workspace variant and within the decoding tolerance of the float64
oracle."""

import numpy as np
import pytest

import framegen
from gpu_util import O_MAXABS, O_RELRMS, o_errors, to_dev
from oracle import decode_attention

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import streaming_long_video_amd as skv  # noqa: E402
from streaming_long_video_amd import _binding as B  # noqa: E402


def _noalloc(layer, q, out):
    B.statekv_decode_attention_noalloc(layer.handle, q.data_ptr(), q.shape[0], out.data_ptr(),
                                       torch.cuda.current_stream().cuda_stream)
    return out


@pytest.mark.parametrize("name,n_frames", [("internvl3_1b_layer", 12), ("internvl3_8b_layer", 24)])
def test_noalloc_decode_matches_workspace_decode(name, n_frames):
    spec = framegen.workload(name)
    T, Hq, Hkv, d = spec.frame_tokens, spec.n_q_heads, spec.n_kv_heads, spec.head_dim
    print(f"no-alloc decode: {name}, {n_frames} frames", flush=True)
    layer = skv.Layer(Hq, Hkv, d, T, spec.state_budget, detailed_capacity=n_frames * T)
    ks, vs = [], []
    for q, k, v in framegen.frames(spec, 0, n_frames):
        layer.prefill(to_dev(q), to_dev(k), to_dev(v))
        ks.append(k), vs.append(v)
    torch.cuda.synchronize()
    dk, dv = np.concatenate(ks), np.concatenate(vs)
    for M in (4, 1):  # second call: smaller input
        qt = framegen.text_queries(spec.replace(n_frames=n_frames), M, 0)
        q_d = to_dev(qt)
        ref_gpu = layer.decode(q_d)
        out = torch.full((M, Hq, d), float("nan"), dtype=torch.float32, device="cuda")
        _noalloc(layer, q_d, out)
        torch.cuda.synchronize()
        a, b = out.cpu().numpy(), ref_gpu.cpu().numpy()
        np.testing.assert_array_equal(a, b)
        maxabs, relrms = o_errors(a, decode_attention(qt, dk, dv))
        print(f"  M={M}: identical to the workspace variant; vs oracle maxabs {maxabs:.2e} "
              f"relrms {relrms:.2e}", flush=True)
        assert maxabs <= O_MAXABS and relrms <= O_RELRMS


def test_noalloc_decode_argument_errors():
    spec = framegen.workload("tiny")
    layer = skv.Layer(spec.n_q_heads, spec.n_kv_heads, spec.head_dim, spec.frame_tokens,
                      spec.state_budget, detailed_capacity=spec.n_frames * spec.frame_tokens)
    q = torch.zeros((1, spec.n_q_heads, spec.head_dim), dtype=torch.bfloat16, device="cuda")
    out = torch.zeros((1, spec.n_q_heads, spec.head_dim), dtype=torch.float32, device="cuda")
    # nothing in D yet
    with pytest.raises(B.StateKVError) as e:
        B.statekv_decode_attention_noalloc(layer.handle, q.data_ptr(), 1, out.data_ptr())
    assert e.value.status == B.STATEKV_ERR_INVALID_ARGUMENT
    # G * M > 32
    with pytest.raises(B.StateKVError) as e:
        B.statekv_decode_attention_noalloc(layer.handle, q.data_ptr(), 17, out.data_ptr())
    assert e.value.status == B.STATEKV_ERR_UNSUPPORTED
