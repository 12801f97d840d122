// fa_bwd_d256.hip -- head-dim-256 instantiations of the backward (dQ and dK/dV) kernels.
//
// The source is fa_bwd.hip itself, compiled a second time with only its
// head-dim-256 launchers, and with the matrix instructions selected in their
// VGPR form (the build passes -mllvm -amdgpu-mfma-vgpr-form for this unit).
// At one wavefront per SIMD the default selection puts the accumulators in
// AGPRs and the compiler then copies the whole output accumulator between
// AGPRs and VGPRs on every loop iteration (and spills in the backward); the
// VGPR form removes those copies.  Head dims 64 and 128 keep the default.
#define FA_D256_UNIT 1
#include "fa_bwd.hip"
