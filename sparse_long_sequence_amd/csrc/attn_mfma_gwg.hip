// Band + global attention with the global rows in workgroups of their own (the GWG
// kernels): the kernel source of attn_mfma.hip, instantiated here with GWG = true, in
// a translation unit of its own so that the code of the other attention kernels does
// not change with these instantiations.
#define LF_ATTN_GWG_TU 1
#include "attn_mfma.hip"
