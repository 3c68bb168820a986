"""Sigma schedules for the sampler kernels (host-side numbers only).

REFINE: the three-step refiner, 0.909 -> 0.857 -> 0.667 -> 0 ("Open-H3-Regenerate-2K:
High-Resolution Video Refinement with Few-Step Diffusion", agientry.com, section
"Three steps instead of dozens", schedule equation).

In-context routes ("Open-H3-Regenerate-2K-IC:草稿留在上下文里,2K 与 4K 重绘仍对着原来的脸、口型和字",
wujieai.com, section "三步接着放大的草稿画,八步从噪声重画"): one 8-step noise table with video shift 12;
up3 mixes the upscaled draft latent to sigma 0.835 and takes the table's last three
steps, up4 mixes to 0.923 and takes four, hf8 starts from noise at sigma 1 and takes
all eight; the reference row is renoised at sigma 0.001 (99.9% draft).  The pages
print no formula for the table; it is taken as the time-shifted flow-matching table
sigma(t) = shift·t / (1 + (shift - 1)·t) on an even grid of t from 1 to 0, which puts
0.923 at t = 1/2 as the pages do.  Every step runs as fsd_euler_step with the pair of
sigmas passed at run time; the renoise start as fsd_renoise.
"""
from __future__ import annotations

REFINE = (0.909, 0.857, 0.667, 0.0)

VIDEO_SHIFT = 12.0
TABLE_STEPS = 8
ROUTES = {"up3": (0.835, 3), "up4": (0.923, 4), "hf8": (1.0, 8)}
REFERENCE_ROW_SIGMA = 0.001


def shifted_table(n_steps: int = TABLE_STEPS, shift: float = VIDEO_SHIFT) -> list:
    """The n_steps + 1 noise levels from sigma = 1 down to 0."""
    levels = []
    for k in range(n_steps, -1, -1):          # t = k / n_steps, from 1 down to 0
        t = k / n_steps
        levels.append(shift * t / (1.0 + (shift - 1.0) * t))
    return levels


def route(name: str) -> list:
    """Noise levels of an IC route: its start, then the last steps of the table."""
    if name not in ROUTES:
        raise ValueError(f"unknown route {name!r}; one of {sorted(ROUTES)}")
    start, steps = ROUTES[name]
    table = shifted_table()
    return [start] + table[-steps:]
