// Kernels of the mfma family with bf16 inputs.
#define DG_FAMILY_VARIANT dg::V_MFMA
#define DG_FAMILY_DTYPE dg::DT_BF16
#define DG_FAMILY_LAUNCH launch_mfma_bf16
#define DG_FAMILY_LAUNCH_GROUPED launch_mfma_bf16_grouped
#include "inst_family.inc"
