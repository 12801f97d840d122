// fa_fwd_d256.hip -- head-dim-256 instantiations of the forward (plain, key-split, dropout,
// block-sparse) kernels.
//
// The source is fa_fwd.hip itself, compiled a second time with only its
// head-dim-256 launchers.  These kernels run one wavefront per SIMD with the
// whole register file: the output accumulator (128 registers per lane) lives
// in AGPRs, the matrix instructions' default form, which leaves the VGPRs to
// the Q fragments (64 registers, read from there for every K block instead
// of from LDS) and the fragments in flight.  The rare rescale of the
// accumulator is done in place in the AGPRs (FA_FWD_ACC_AGPR): were it done
// on VGPR copies, the compiler would give the accumulator one register class
// for the whole loop and copy it between AGPRs and VGPRs at every step.
#define FA_D256_UNIT 1
#define FA_FWD_ACC_AGPR 1
#include "fa_fwd.hip"
