"""Input matrices shared by the GPU test files (seeded, synthetic)."""
import torch


def extreme_cases():
    """Matrices at the ends of each format: name -> (matrix, target, fixed resolution or 0)."""
    g = torch.Generator().manual_seed(77)

    def gauss(r, c, std, dtype):
        return (torch.randn(r, c, generator=g) * std).to(dtype)
    zero_row = gauss(48, 1000, 0.02, torch.bfloat16)
    zero_row[5] = 0
    spike = gauss(40, 777, 0.02, torch.bfloat16)
    spike[3, 100] = 3.0e4
    near_max = gauss(64, 1000, 8000.0, torch.float16)
    near_max[::7, ::13] = 65504.0
    near_max[1::7, 5::13] = -65504.0
    # name: (matrix, target, fixed resolution or 0)
    return {
        "bf16_tiny_1e-38": (gauss(64, 1000, 1e-38, torch.bfloat16), 4.0, 0.0),
        "bf16_huge_1e30": (gauss(64, 1000, 1e30, torch.bfloat16), 4.0, 0.0),
        "fp16_near_max_coarse": (near_max, 4.0, 1.5),
        "fp16_subnormal_inputs": (gauss(64, 1000, 3e-6, torch.float16), 4.0, 0.0),
        "one_row_of_seven": (gauss(1, 7, 0.02, torch.bfloat16), 4.0, 0.1),
        "one_zero_row": (zero_row, 4.0, 0.0),
        "all_zero": (torch.zeros(32, 512, dtype=torch.bfloat16), 4.0, 0.0),
        "one_spike_row": (spike, 3.0, 0.0),
    }
