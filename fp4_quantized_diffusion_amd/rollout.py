"""Stage-1 FP4 exploration rollout driven through the C ABI.

Sol-RL's first stage (project page, "Two-Stage Pipeline"; aitrends summary,
Stage-1 paragraph): re-quantize the current weights, integrate N noise seeds
with a 6-step ODE solver whose linears run FP4 x FP4, score every candidate
with a proxy reward and keep the K/2 best and K/2 worst seeds.

The velocity network stands in for the pages' trained transformers with the
shape of their MLP linears: 4 residual blocks
    h <- h + W2 GELU(W1 RMSNorm(h)),    v = h_4,  h_0 = x
(dim -> hidden -> dim, no time conditioning), then Euler steps on the
uniform grid t_i = 1 - i/steps. Per block the device work is:
    fp4_quantize(h, RMSNORM prologue)     -> A1 (MXFP4)
    fp4_gemm(A1, W1q) -> z (fp32)
    fp4_quantize(z, GELU prologue)        -> A2 (MXFP4)
    fp4_gemm(A2, W2q, residual = h) -> h  (fp32, in place)
and per step euler_step(x, v = h). With the panel layout (the default) and
row counts that are multiples of 256, the first two lines are one call,
fp4_gemm_panel_gelu_f32(A1, W1q) -> A2, which applies the GELU to the fp32
sums and the MXFP4 quantization in the GEMM's epilogue (bit-identical to the
pair, without writing z); and the last block's second GEMM and the Euler
step are one call,
fp4_gemm_panel_euler(A2, W2q, residual = h, x) -> x_next, which applies
x + dt (h + A2 W2q^T) in the GEMM's epilogue -- bit-identical to the GEMM into
v followed by euler_step, without writing v or reading it back. The hidden
activation z stays fp32, as in the float64 oracle's reading (GELU from an
LDS table of (Q, phi) at bf16 points carried to z by a fourth-order
expansion, erfc evaluated beyond |z| = 6); hidden="bf16" rounds it to bf16
first (fp4_gemm_panel_gelu, one table read per value, faster -- about 363
ms per rollout step against 388 -- but not the oracle's arithmetic: at
96 x 4096 x 3072 the final state then differs from the oracle's by about a
quarter, because the rounding moves about one hidden value in a hundred
across an FP4 decision point and the next blocks' quantizers amplify that).
The FP4 operands use the panel layout by default
(fp4_quantize with FP4_LAYOUT_PANEL, fp4_gemm_panel): the same codes and
scales, stored so that every GEMM stage load is contiguous; layout="row" runs
the row-major entry points (and a separate euler_step) instead.

Two-stream schedule (overlap=True): the candidates are split into
two halves A and B; the GEMMs run on the caller's stream and the quantizers
and Euler steps on a second stream, enqueued phase by phase so that each
quantizer of one half runs while a GEMM of the other half does:
    GEMM stream:       G1(A) G1(B) G2(A) G2(B) G1'(A) ...
    quantizer stream:  R(A) R(B) Q(A) Q(B) R'(A) R'(B) ...
(R: RMSNorm quantize, Q: GELU quantize; every edge is a device-side event
wait, no host synchronization). It stores the hidden activation as bf16, so
it needs hidden="bf16". The quantizers are VALU-bound and fit
beside the GEMM's one workgroup per CU (its waves leave VGPRs for one more
wave per SIMD), so they overlap it. Every kernel computes rows independently
of how the rows are chunked, so the result is bit-identical to the
one-stream schedule. Both streams run at the default priority. On MI355X
this schedule measured slower than the one-stream schedule of the same
(unfused) kernels for the 96 x 4096 x 3072 rollout (534 vs 523 ms per step,
where the fused one-stream path takes about 363 ms with the same bf16 hidden
activation): the GEMM runs at the card's power limit, and the overlapped
quantizers lower the clock and slow the GEMM by more than they hide; it is
kept as an option.

Every call enqueues on the current stream (and the second stream, which the
current stream waits for before returning); the only host synchronization is
the caller reading the selected indices.
"""
from . import binding as fb


class Fp4Rollout:
    def __init__(self, w1, w2, u, steps=6, k_top=12, k_bottom=12, fmt="mx", chunk=None, timer=None,
                 layout="panel", overlap=False, lora=None, fuse_reward=True, hidden="f32"):
        """w1[b]: bf16 or fp32 CUDA [hidden, dim]; w2[b]: [dim, hidden]; u: fp32 [dim].
        lora: optional (lora1, lora2), one entry per block each, None or a
        LoRA adapter (B, A, scale) of that weight; the per-iteration
        re-quantization then merges it in the same pass (fp4_quantize_lora).
        Update adapters between iterations with set_lora.
        fuse_reward: on the panel layout, take the proxy reward in the last
        GEMM of the last step (fp4_gemm_panel_euler_reward) when the shapes
        allow, instead of re-reading the final state (fp4_proxy_reward): the
        same quantity in another fp32 summation order.
        chunk: candidates per pass through the network on one stream (None =
        all); ignored by the two-stream schedule.
        overlap: two-stream schedule over two halves of the candidates (needs
        at least 2 candidates).
        timer: optional callable(name, fn) wrapping each launch (for timing);
        it is called with the launch's stream current.
        hidden: "f32" (default) keeps the first linear's output fp32 into
        GELU, the float64 oracle's reading of the hidden activation (the
        fused epilogue, fp4_gemm_panel_gelu_f32, takes GELU of the fp32 sums
        from a (Q, phi) table and a fourth-order expansion; the unfused path
        stores z as fp32). "bf16" rounds it to bf16 before GELU (the fused
        epilogue, fp4_gemm_panel_gelu, reads one table entry per value; the
        unfused path stores z as bf16): about half the epilogue arithmetic,
        but a different network -- the rounding moves hidden values across
        FP4 decision points, which the following quantizers amplify."""
        if fmt != "mx":
            raise ValueError("the rollout's fused quantize prologues are implemented for MXFP4")
        self.w1, self.w2, self.u = list(w1), list(w2), u
        self.steps, self.k_top, self.k_bottom = steps, k_top, k_bottom
        if layout not in ("panel", "row"):
            raise ValueError(f"unknown layout {layout!r}")
        self.fmt, self.chunk, self.layout = fmt, chunk, layout
        self.overlap = overlap
        self.fuse_reward = fuse_reward
        if hidden not in ("bf16", "f32"):
            raise ValueError(f"unknown hidden dtype {hidden!r}")
        if hidden == "f32" and overlap:
            raise ValueError("the two-stream schedule stores the hidden activation as bf16: pass hidden='bf16'")
        self.hidden = hidden
        self._side = None
        self.timer = timer
        self.q1 = self.q2 = None
        self._bufs = {}
        self.set_lora(lora)

    def set_lora(self, lora):
        """Adapters for the next re-quantization: None, or (lora1, lora2) as
        in the constructor."""
        n = len(self.w1)
        self.lora1, self.lora2 = ([None] * n, [None] * n) if lora is None else (list(lora[0]), list(lora[1]))
        if len(self.lora1) != n or len(self.lora2) != n:
            raise ValueError("one adapter entry (or None) per block and weight")

    def requantize(self):
        """Per-iteration weight re-quantization (all weights, on device), with
        each weight's LoRA adapter merged in when one is set."""
        def one(w, ad, prev):
            if ad is None:
                return fb.quantize(w, self.fmt, out=prev, layout=self.layout)
            b, a, scale = ad
            return fb.quantize_lora(w, b, a, scale, out=prev, layout=self.layout)

        self.q1 = [one(w, self.lora1[i], None if self.q1 is None else self.q1[i]) for i, w in enumerate(self.w1)]
        self.q2 = [one(w, self.lora2[i], None if self.q2 is None else self.q2[i]) for i, w in enumerate(self.w2)]

    def _buf(self, name, shape, dtype, device):
        import torch
        key = (name, tuple(shape), dtype)
        t = self._bufs.get(key)
        if t is None:
            t = torch.empty(shape, dtype=dtype, device=device)
            self._bufs[key] = t
        return t

    def _call(self, name, fn):
        return fn() if self.timer is None else self.timer(name, fn)

    def _gemm(self, a, b, out_dtype, residual=None, out=None):
        return self._call("gemm", lambda: fb.gemm(a, b, out_dtype, residual=residual, out=out))

    def velocity(self, x, h, step=None, reward=None):
        """h <- v(x) for x, h fp32 [rows, dim] (h_0 = x is never copied: the
        first block's GEMM takes x as its residual). step = (t_cur, t_next,
        x_out): the last block's second GEMM also takes the Euler step,
        x_out = x + (t_next - t_cur) v, and h is left at the previous block's
        value. reward = (rewards, tokens) with step: that GEMM also writes the
        proxy reward of each candidate (tokens rows each) of x_out into
        rewards (fp4_gemm_panel_euler_reward)."""
        import torch
        rows, dim = x.shape
        hidden = self.w1[0].shape[0]
        # the first linear quantizes GELU of its own output (fp4_gemm_panel_gelu)
        # when the shapes allow; otherwise z goes through HBM as bf16
        fused = self.layout == "panel" and rows % 256 == 0 and hidden % 256 == 0
        zdt = torch.bfloat16 if self.hidden == "bf16" else torch.float32
        z = None if fused else self._buf("z", (rows, hidden), zdt, x.device)
        src = x
        last = len(self.w1) - 1
        for b in range(len(self.w1)):
            a1 = self._call("quant_rmsnorm", lambda: fb.quantize(
                src, self.fmt, prologue="rmsnorm", out=self._qbuf("a1", rows, dim, x.device)))
            if fused:
                a2 = self._call("gemm", lambda: fb.gemm_gelu(a1, self.q1[b], out=self._qbuf("a2", rows, hidden,
                                                                                          x.device),
                                                             exact=self.hidden == "f32"))
            else:
                self._gemm(a1, self.q1[b], self.hidden, out=z)
                a2 = self._call("quant_gelu", lambda: fb.quantize(
                    z, self.fmt, prologue="gelu", out=self._qbuf("a2", rows, hidden, x.device)))
            if b == last and step is not None:
                t_cur, t_next, x_out = step
                if reward is not None:
                    rw, tokens = reward
                    part = self._buf("rpart", (max(rows // 256, 1) * max(dim // 256, 1) * 4,), torch.float32, x.device)
                    self._call("gemm", lambda: fb.gemm_euler_reward(a2, self.q2[b], src, x, t_cur, t_next, self.u,
                                                                    tokens, out=x_out, rewards=rw, partials=part))
                else:
                    self._call("gemm", lambda: fb.gemm_euler(a2, self.q2[b], src, x, t_cur, t_next, out=x_out))
                return x_out
            self._gemm(a2, self.q2[b], "f32", residual=src, out=h)
            src = h
        return h

    def _qbuf(self, name, rows, k, device):
        import torch
        if self.layout == "panel":
            cb, sb = fb.panel_bytes(rows, k)
            codes = self._buf(name + ".c", (cb,), torch.uint8, device)
            scales = self._buf(name + ".s", (sb,), torch.uint8, device)
            return fb.QTensor(codes, scales, None, fb.FMT_MX, k, "panel", rows)
        ldc = ((k // 2 + 15) // 16) * 16
        codes = self._buf(name + ".c", (rows, ldc), torch.uint8, device)
        scales = self._buf(name + ".s", (rows, k // 32), torch.uint8, device)
        return fb.QTensor(codes, scales, None, fb.FMT_MX, k)

    def run(self, noise, work=None):
        """noise: fp32 CUDA [n_cand, tokens, dim]. The trajectory is integrated
        in `work` (same shape; the first Euler step reads `noise` and writes
        `work`, so `noise` stays intact), or in place in `noise` if work is None.
        Returns (rewards [n_cand], top [k_top], bottom [k_bottom], r_norm)."""
        if self.overlap and noise.shape[0] >= 2:
            return self._run_two_streams(noise, work)
        return self._run_one_stream(noise, work)

    def graph(self, noise, work=None):
        """Capture one run(noise, work) -- the weight re-quantization, every
        Euler step, the reward and the selection -- in a HIP graph (through
        torch.cuda.CUDAGraph) for callers that repeat the rollout on the same
        buffers as one graph launch (a serving loop that replays captured
        work). It is not faster: from 4 x 256 x 256 up, the kernels' own time
        covers the launches, and replays ran as fast as eager rollouts.
        Returns (replay, outputs): replay() runs the whole rollout
        again as one graph launch on the current stream; outputs =
        (rewards, top, bottom, r_norm) are refreshed in place by every replay.
        noise and work stay at their addresses: write new noise into `noise`
        (and new weights into the bf16 weights given to the constructor)
        between replays. Every launch of the library is a kernel node (it
        allocates and clears no device memory itself). The rollout runs once
        eagerly first, to set up its buffers."""
        import torch
        if self.timer is not None:
            raise ValueError("a timed rollout cannot be captured: build it without timer")
        self.run(noise, work)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            out = self.run(noise, work)
        self._graph = g  # the graph's memory pool lives as long as the graph
        return g.replay, out

    def _run_two_streams(self, noise, work):
        import torch
        n_cand, tokens, dim = noise.shape
        hidden = self.w1[0].shape[0]
        dev = noise.device
        main = torch.cuda.current_stream(dev)
        if self._side is None:
            self._side = torch.cuda.Stream(device=dev)  # default priority
        side = self._side

        def mark(stream):
            e = torch.cuda.Event()
            e.record(stream)
            return e

        half = (n_cand + 1) // 2
        first = [0, half * tokens]
        rows = [half * tokens, (n_cand - half) * tokens]
        self._call("requantize", self.requantize)
        x0 = noise.view(n_cand * tokens, dim)
        x = x0 if work is None else work.view(n_cand * tokens, dim)
        h = [self._buf(f"h{c}", (rows[c], dim), torch.float32, dev) for c in (0, 1)]
        z = [self._buf(f"z{c}", (rows[c], hidden), torch.bfloat16, dev) for c in (0, 1)]
        a1 = [self._qbuf(f"a1_{c}", rows[c], dim, dev) for c in (0, 1)]
        a2 = [self._qbuf(f"a2_{c}", rows[c], hidden, dev) for c in (0, 1)]
        t = [1.0 - i / self.steps for i in range(self.steps + 1)]
        side.wait_stream(main)  # the weights are re-quantized, earlier work done
        g2 = [None, None]  # per half: its latest second GEMM (h final for the block)
        for i in range(self.steps):
            src = x0 if i == 0 else x
            xs = [src[first[c]:first[c] + rows[c]] for c in (0, 1)]
            xd = [x[first[c]:first[c] + rows[c]] for c in (0, 1)]
            for b in range(len(self.w1)):
                res = xs if b == 0 else h
                rdy = [None, None]
                with torch.cuda.stream(side):
                    for c in (0, 1):
                        if b > 0:  # block 0 reads x, written by this stream's Euler step
                            side.wait_event(g2[c])
                        self._call("quant_rmsnorm", lambda: fb.quantize(res[c], self.fmt, prologue="rmsnorm",
                                                                        out=a1[c]))
                        rdy[c] = mark(side)
                g1 = [None, None]
                for c in (0, 1):
                    main.wait_event(rdy[c])
                    self._gemm(a1[c], self.q1[b], "bf16", out=z[c])
                    g1[c] = mark(main)
                with torch.cuda.stream(side):
                    for c in (0, 1):
                        side.wait_event(g1[c])
                        self._call("quant_gelu", lambda: fb.quantize(z[c], self.fmt, prologue="gelu", out=a2[c]))
                        rdy[c] = mark(side)
                for c in (0, 1):
                    main.wait_event(rdy[c])
                    self._gemm(a2[c], self.q2[b], "f32", residual=res[c], out=h[c])
                    g2[c] = mark(main)
            with torch.cuda.stream(side):
                for c in (0, 1):
                    side.wait_event(g2[c])
                    self._call("euler", lambda: fb.euler(xs[c], h[c], t[i], t[i + 1], out=xd[c]))
        main.wait_stream(side)
        rewards = self._call("reward", lambda: fb.proxy_reward(x, n_cand, tokens, self.u))
        top, bottom, rn = self._call("select", lambda: fb.select(rewards, self.k_top, self.k_bottom))
        return rewards, top, bottom, rn

    def _run_one_stream(self, noise, work):
        import torch
        n_cand, tokens, dim = noise.shape
        chunk = self.chunk or n_cand
        self._call("requantize", self.requantize)
        x0 = noise.view(n_cand * tokens, dim)
        x = x0 if work is None else work.view(n_cand * tokens, dim)
        h = self._buf("h", (chunk * tokens, dim), torch.float32, noise.device)
        t = [1.0 - i / self.steps for i in range(self.steps + 1)]
        rewards = torch.empty(n_cand, dtype=torch.float32, device=noise.device)
        fused_reward = True
        for i in range(self.steps):
            src = x0 if i == 0 else x
            for c0 in range(0, n_cand, chunk):
                nc = min(chunk, n_cand - c0)
                r0, rows = c0 * tokens, nc * tokens
                xs, xd = src[r0:r0 + rows], x[r0:r0 + rows]
                if self.layout == "panel":  # Euler step fused into the last GEMM
                    # and, after the last step, the proxy reward too when whole wave tiles fit
                    rw = None
                    if i == self.steps - 1 and self.fuse_reward and rows % 256 == 0 and dim % 256 == 0 \
                            and tokens % 128 == 0:
                        rw = (rewards[c0:c0 + nc], tokens)
                    elif i == self.steps - 1:
                        fused_reward = False
                    self.velocity(xs, h[:rows], step=(t[i], t[i + 1], xd), reward=rw)
                else:
                    fused_reward = False
                    hc = self.velocity(xs, h[:rows])
                    self._call("euler", lambda: fb.euler(xs, hc, t[i], t[i + 1], out=xd))
        if self.steps == 0 or not fused_reward:
            rewards = self._call("reward", lambda: fb.proxy_reward(x, n_cand, tokens, self.u))
        top, bottom, rn = self._call("select", lambda: fb.select(rewards, self.k_top, self.k_bottom))
        return rewards, top, bottom, rn
