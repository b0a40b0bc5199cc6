// Band + global attention in the 4-wave layout (128-row workgroups, a 4-slot ring of
// 75 KB, two workgroups per CU) used for long sequences: the kernel source of
// attn_mfma.hip, instantiated here with LF_ATTN_WAVES = 4 in a translation unit of
// its own.
#define LF_ATTN_WAVES 4
#define LF_ATTN_W4_TU 1
#include "attn_mfma.hip"
