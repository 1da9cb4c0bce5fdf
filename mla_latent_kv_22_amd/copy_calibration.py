"""Plain device copy of a known size, used to calibrate the FETCH_SIZE and
WRITE_SIZE counters of rocprofv3 against bytes actually moved.

Usage: rocprofv3 --pmc FETCH_SIZE -- python -m mla_latent_kv_22_amd.copy_calibration
"""
import torch

NBYTES = 1 << 30  # 1 GiB read + 1 GiB written per copy


def main():
    src = torch.ones(NBYTES // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(f"copied {NBYTES} bytes x 3")


if __name__ == "__main__":
    main()
