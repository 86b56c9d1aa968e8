"""Run the microbenchmarks on the current GPU and print one JSON line per unit."""
import ctypes as ct
import json
import os
import statistics
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "libmb.so")
KINDS = [("mfma_int8_32x32x32", "TOPS"), ("mfma_fp8_32x32x64", "TOPS"), ("mfma_fp16_32x32x16", "TFLOP/s"),
         ("v_exp_f32", "G exp/s")]


def build() -> str:
    """Compile mb.hip for gfx950 in-tree (always rebuilds)."""
    from quantized_attention_video_02_amd import build as b

    tmp = LIB + ".tmp"
    cmd = [b.hipcc(), *b.HIPFLAGS, "-shared", os.path.join(HERE, "mb.hip"), "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on mb.hip:\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


def main():
    import torch

    if not os.path.exists(LIB):
        build()
    L = ct.CDLL(LIB)
    L.mb_run.argtypes = [ct.c_int, ct.c_int, ct.c_int, ct.c_void_p, ct.c_void_p]
    L.mb_ops.argtypes = [ct.c_int, ct.c_int, ct.c_int]
    L.mb_ops.restype = ct.c_double
    ncu = torch.cuda.get_device_properties(0).multi_processor_count
    stream = torch.cuda.current_stream()
    for kind, (name, unit) in enumerate(KINDS):
        blocks = ncu * 12                       # 12 workgroups of 4 waves per CU
        iters = 2000 if kind < 3 else 20000
        out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
        ts = []
        for rep in range(6):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            if L.mb_run(kind, blocks, iters, ct.c_void_p(out.data_ptr()), ct.c_void_p(stream.cuda_stream)):
                raise RuntimeError(f"mb_run({name}) failed")
            e1.record(stream)
            torch.cuda.synchronize()
            if rep:
                ts.append(e0.elapsed_time(e1))
        ms = statistics.median(ts)
        rate = L.mb_ops(kind, blocks, iters) / (ms * 1e-3)
        print(json.dumps({"unit_under_test": name, "value": rate / (1e9 if kind == 3 else 1e12),
                          "unit": unit, "ms": ms, "cus": ncu}), flush=True)
    for nbytes in (1 << 30, 3 << 30):
        src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        ts = []
        for _ in range(8):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            dst.copy_(src)
            e1.record(stream)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        ms = statistics.median(ts)
        print(json.dumps({"unit_under_test": f"device copy {nbytes >> 20} MiB (read + write)",
                          "value": 2 * nbytes / (ms * 1e-3) / 1e12, "unit": "TB/s", "ms": ms}), flush=True)
        del src, dst


if __name__ == "__main__":
    main()
