"""MI355X-native SVDQuant W4A4 linear layer (gfx950 HIP kernels behind a
C-ABI library).  The binding lives in `svdq`; the seeded synthetic inputs in
`synth`.  Importing the package loads nothing; the HIP library is loaded on
first use and its absence is an error, never a fallback."""
