"""kimodo_denoise_step_static, the entry point that allocates nothing (its
scratch is a static device array), against kimodo_denoise_step with a ctx and
a workspace: the same kernels and partitions, so the same bits. Two calls in a
row on the same GPU, the second with a smaller input, so the second finds the
first call's contents in the shared array."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype_name,L,shapes", [
    ("f16", 16, ((2, 150, [150, 97]), (1, 60, [41]))),
    ("f32", 2, ((3, 100, [100, 1, 64]), (2, 37, [37, 20]))),
])
def test_static_step_equals_workspace_step(dtype_name, L, shapes):
    import torch

    from synthetic.inputs import Dims, make_noise, make_text, make_weights
    from text_motion_diffusion_amd import kimodo as K
    from text_motion_diffusion_amd.session import Session

    assert torch.cuda.is_available()
    dev = torch.device("cuda:0")
    dims = Dims(layers_root=L, layers_body=L)
    dtype = K.KIMODO_F16 if dtype_name == "f16" else K.KIMODO_F32
    w = make_weights(dims)
    if dtype == K.KIMODO_F16:
        w = [a.astype(np.float16) for a in w]
    B0, T0 = shapes[0][0], shapes[0][1]
    sess = Session(w, L, L, B0, T0, 1, dtype)
    cfg = K.make_config(L, L, B0, T0, 1, dtype)
    _, abar = K.kimodo_make_schedule(100, 1e-4, 0.02, 100)
    stream = torch.cuda.current_stream()
    for call, (B, T, lengths) in enumerate(shapes):
        t = 60 - 7 * call
        x = torch.from_numpy(make_noise(B, T, dims, seed=20 + call)).to(dev)
        text = torch.from_numpy(make_text(B, dims, seed=30 + call)).to(dev)
        print(f"{dtype_name} call {call}: B={B} T={T} lengths={lengths}", flush=True)
        want = sess.denoise_step(x, text, lengths, t, float(abar[t]), float(abar[t - 1]), 2.5)
        got = torch.full_like(x, float("nan"))
        K.kimodo_denoise_step_static(cfg, sess.weights, B, T, x, text, lengths, t, float(abar[t]),
                                     float(abar[t - 1]), 2.5, got, stream=stream)
        torch.cuda.synchronize()
        assert torch.isfinite(want).all()
        diff = (got - want).abs().max().item()
        print(f"  max |static - workspace| = {diff:.3e}", flush=True)
        assert torch.equal(got, want)
    sess.close()
