// The few-output-channel kernel for C_out = 5.
#define CC3D_FEW_COUT 5
#include "cc3d_few.inc"
