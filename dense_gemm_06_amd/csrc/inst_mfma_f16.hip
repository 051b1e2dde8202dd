// Kernels of the mfma family with f16 inputs.
#define DG_FAMILY_VARIANT dg::V_MFMA
#define DG_FAMILY_DTYPE dg::DT_F16
#define DG_FAMILY_LAUNCH launch_mfma_f16
#define DG_FAMILY_LAUNCH_GROUPED launch_mfma_f16_grouped
#include "inst_family.inc"
