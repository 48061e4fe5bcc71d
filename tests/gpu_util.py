"""Helpers shared by the GPU tests: moving the seeded numpy inputs to the
device and results back.  No arithmetic of the method lives here."""
import numpy as np

XDT = {"f16": None, "bf16": None}


def torch_dtype(name):
    import torch
    return {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}[name]


def to_dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def bits_to_dev(bits_u16, dtype_name):
    """uint16 fp16/bf16 bit patterns -> device tensor of that dtype."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits_u16).view(np.int16)).cuda()
    return t.view(torch_dtype(dtype_name))


def packed_to_dev(codes, scales, biases):
    import torch
    c = torch.from_numpy(np.ascontiguousarray(codes).view(np.int32)).cuda()
    s = torch.from_numpy(np.ascontiguousarray(scales).view(np.int16)).cuda().view(torch.float16)
    b = torch.from_numpy(np.ascontiguousarray(biases).view(np.int16)).cuda().view(torch.float16)
    return c, s, b


def packed_from_dev(codes, scales, biases):
    import torch
    c = codes.cpu().numpy().view(np.uint32)
    s = scales.view(torch.int16).cpu().numpy().view(np.uint16)
    b = biases.view(torch.int16).cpu().numpy().view(np.uint16)
    return c, s, b


def out_to_f64(y):
    """fp16/bf16/fp32 device tensor -> exact float64 numpy values."""
    import torch
    return y.to(torch.float32).cpu().numpy().astype(np.float64)


def out_bits(y):
    import torch
    if y.dtype == torch.float32:
        return y.cpu().numpy().view(np.uint32)
    return y.view(torch.int16).cpu().numpy().view(np.uint16)
