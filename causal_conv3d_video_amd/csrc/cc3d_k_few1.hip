// The few-output-channel kernel for C_out = 1.
#define CC3D_FEW_COUT 1
#include "cc3d_few.inc"
