// fa_bwd_d128nc.hip -- head-dim-128 backward kernels without the causal mask.
//
// The source is fa_bwd.hip itself, compiled a second time with only its
// non-causal head-dim-128 launcher and with the matrix instructions in their
// VGPR form (-mllvm -amdgpu-mfma-vgpr-form, set by the build for this unit).
// The dK/dV kernel runs one wavefront per SIMD at this head dim; measured, the
// VGPR form makes its non-causal instantiations faster and spill-free while
// the causal ones are faster in the default form, which fa_bwd.hip keeps.
#define FA_D128NC_UNIT 1
#include "fa_bwd.hip"
