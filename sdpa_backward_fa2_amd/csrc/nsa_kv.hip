// The selected-attention dK/dV kernel (nsa_kv_kernel) in a translation unit of
// its own: the build gives it scheduler options that suit it and not the rest
// of nsa.hip's kernels.  The other kernels and the entry points are left out
// of this unit.
#define SDPA_NSA_KV_UNIT
#include "nsa.hip"
