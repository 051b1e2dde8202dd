// Kernels of the lds family with bf16 inputs.
#define DG_FAMILY_VARIANT dg::V_LDS
#define DG_FAMILY_DTYPE dg::DT_BF16
#define DG_FAMILY_LAUNCH launch_lds_bf16
#define DG_FAMILY_LAUNCH_GROUPED launch_lds_bf16_grouped
#include "inst_family.inc"
