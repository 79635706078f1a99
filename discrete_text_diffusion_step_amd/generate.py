"""Block-autoregressive generation over the C ABI (host loop).

aibars.net news, block-autoregressive denoising: a 256-token block is
denoised fully, committed to the KV cache, then the next block starts.
DiffusionGemma Technical Report review, section 1 (Adaptive Stopping): the
denoising loop stops early on prediction entropy and output stability.
stop_rule "renoised" (default): stop once a step re-noises no position.
stop_rule "stable": stop once no proposal changed since the previous step;
the canvas then takes the stable proposals at every position, as a final
step would.  Either way one 4-byte device-to-host read per step; after
max_steps the final step commits every position.
"""
import math

import torch

from . import binding as B


def generate(model, kv, prompt, n_canvases, canvas_len=256, max_steps=48, seed=1, t_max=1.0, t_min=1.0,
             tau=None, adaptive=True, stream=None, commit_rule="entropy", token_rule="argmax",
             stop_rule="renoised"):
    """Commit `prompt`, then denoise and commit n_canvases canvases.

    All device work (library calls, copies, the count read-back) is issued on
    one stream: `stream` if given, else torch's current stream, so each read
    of the stop count follows the step that wrote it.
    Returns (tokens [n_canvases, canvas_len] int32 on the device, steps used per canvas).
    """
    s = stream if stream is not None else torch.cuda.current_stream()
    with torch.cuda.stream(s):
        return _generate(model, kv, prompt, n_canvases, canvas_len, max_steps, seed, t_max, t_min, tau,
                         adaptive, s, commit_rule, token_rule, stop_rule)


def _generate(model, kv, prompt, n_canvases, canvas_len, max_steps, seed, t_max, t_min, tau, adaptive, s,
              commit_rule, token_rule, stop_rule):
    V = model.cfg["vocab"]
    tau = 0.5 * math.log(V) if tau is None else tau
    dev = prompt.device
    if prompt is not None and prompt.numel() > 0:
        # a ring cache takes at most ring_tokens new positions per call
        step = getattr(kv, "ring_tokens", 0) or prompt.numel()
        for p0 in range(0, prompt.numel(), step):
            B.dg_commit_canvas(model, kv, prompt[p0:p0 + step], stream=s)
    out = torch.empty(n_canvases, canvas_len, dtype=torch.int32, device=dev)
    steps_used = []
    canvas = B.Canvas(canvas_len, model.cfg["hidden"], model.cfg["dtype"], device=dev)
    host_count = torch.empty(1, dtype=torch.int32, pin_memory=True)
    for c in range(n_canvases):
        canvas.tokens.copy_(B.dg_canvas_noise(canvas_len, V, seed, c, device=dev, stream=s))
        canvas.use_u = 0
        canvas.pred.fill_(-1)
        used = 0
        for i in range(max_steps):
            final = i == max_steps - 1
            sc = dict(vocab=V, tau=tau, t_max=t_max, t_min=t_min, n_steps=max_steps, step=i,
                      canvas_idx=c, seed=seed, final_step=final, commit_rule=commit_rule, token_rule=token_rule)
            B.dg_canvas_step(model, kv, canvas, sc, stream=s)
            used += 1
            if adaptive and not final:
                stable = stop_rule == "stable"
                if stable and i == 0:
                    continue
                host_count.copy_(canvas.n_changed if stable else canvas.n_renoised, non_blocking=True)
                s.synchronize()
                if int(host_count.item()) == 0:
                    if stable:
                        canvas.tokens.copy_(canvas.pred)
                    break
        out[c].copy_(canvas.tokens)
        B.dg_commit_canvas(model, kv, canvas.tokens, stream=s)
        steps_used.append(used)
    return out, steps_used
