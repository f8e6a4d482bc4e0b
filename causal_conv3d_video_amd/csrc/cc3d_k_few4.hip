// The few-output-channel kernel for C_out = 4.
#define CC3D_FEW_COUT 4
#include "cc3d_few.inc"
