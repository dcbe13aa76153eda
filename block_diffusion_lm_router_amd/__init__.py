"""MI355X-native hot path of a block-diffusion LM denoising step (HIP, gfx950)."""
