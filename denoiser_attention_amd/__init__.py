"""TwoTower denoising-step kernels for AMD MI355X (gfx950)."""
