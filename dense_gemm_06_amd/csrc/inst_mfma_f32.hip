// Kernels of the mfma family with f32 inputs.
#define DG_FAMILY_VARIANT dg::V_MFMA
#define DG_FAMILY_DTYPE dg::DT_F32
#define DG_FAMILY_LAUNCH launch_mfma_f32
#define DG_FAMILY_LAUNCH_GROUPED launch_mfma_f32_grouped
#include "inst_family.inc"
