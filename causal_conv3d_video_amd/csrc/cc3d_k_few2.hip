// The few-output-channel kernel for C_out = 2.
#define CC3D_FEW_COUT 2
#include "cc3d_few.inc"
