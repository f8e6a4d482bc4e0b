// The few-output-channel kernel for C_out = 3.
#define CC3D_FEW_COUT 3
#include "cc3d_few.inc"
