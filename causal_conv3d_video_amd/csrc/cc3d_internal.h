// Internal plan representation shared by the planner and the launcher.
#pragma once
#include "cc3d.h"

#include <atomic>
#include <cstdint>

// Kernel variants the planner can pick.  The bf16 ones are implicit-GEMM
// MFMA kernels (block tile = block_m output pixels x block_n output channels).
enum cc3d_kernel_id : int32_t {
  CC3D_K_F32_DIRECT = 0,     // fp32, any spatial parameters, one output per thread
  CC3D_K_BF16_S3_N32 = 3,    // 3x3 spatial, 256 px (8x32) x 32 channels, any C_out
  CC3D_K_BF16_S1_N192 = 4,   // 1x1 spatial, 256 px (8x32) x 192 channels
  CC3D_K_BF16_S1_N32 = 5,    // 1x1 spatial, 256 px (8x32) x 32 channels, any C_out
  CC3D_K_BF16_S3_N96_X2 = 6, // 3x3 spatial, 256 px (8x32) x 96 channels, two workgroups per CU
  CC3D_K_BF16_S3_N96_G32W8 = 10, // 3x3 spatial, 512 px (16x32) x 96 channels, halo staged by 32
                                 // channels, 8 waves (two per SIMD, 2 rows each)
  CC3D_K_BF16_S3_FEW = 11,   // 3x3 spatial, k_t = 3, d_t = 1, C_out <= 5, C_in in {32, 64, 96}:
                             // R x 128 px patches walked through time, halo rows streamed
  CC3D_K_BF16_GEN_N64 = 12,  // any spatial kernel size, stride, dilation and padding:
                             // 256 px (8x32) x 64 channels, input pixels gathered per spatial tap
  CC3D_K_BF16_S3_N64_G32W8 = 13, // as CC3D_K_BF16_S3_N96_G32W8 with 768 px (24x32) x 64 channels
                                 // (3 rows per wave)
  CC3D_K_BF16_GEN_N96 = 14,  // as CC3D_K_BF16_GEN_N64 with 96 output channels per tile
  CC3D_K_BF16_S3D2_N64_G32W8 = 15, // the group-staged kernel on 3x3 taps at spatial dilation 2,
                                   // padding 2: 512 px (16x32) x 64 channels
  CC3D_K_BF16_S3S2_N96_G32W4 = 16, // the group-staged kernel on 3x3 taps at spatial stride 2,
                                   // padding 1: 128 output px (4x32) x 96 channels, 4 waves
  CC3D_K_BF16_S3S2_N64_G32W8 = 17, // as CC3D_K_BF16_S3S2_N96_G32W4 with 64 channels, 8 waves (each
                                   // group's two 16-channel halves on two waves of the same rows)
  CC3D_K_BF16_S1_N192_RD = 18, // 1x1 spatial, 256 consecutive px of the flattened frame x 192
                               // channels, pixels loaded straight into registers
};

// A plan is host metadata only, immutable once built.
struct cc3d_plan {
  cc3d_desc_t d{};
  cc3d_plan_info_t info{};
  int32_t tile_h = 0;      // output rows per workgroup patch
  int32_t tile_w = 0;      // output columns per workgroup patch
  int32_t tiles_y = 0, tiles_x = 0, nblk_n = 0;
  int32_t cin_chunk = 0;   // input channels per pipeline stage
  int32_t pack_kind = 0;   // packed weight image: 0 none (fp32), 1 stage-ordered tiles, 2 a copy of W
  int64_t x_bytes = 0, cache_bytes = 0, w_bytes = 0, b_bytes = 0, out_bytes = 0, cache_out_bytes = 0;
  int32_t elem = 0;        // bytes per element
};

namespace cc3d {
extern std::atomic<uint64_t> g_fast_path, g_unsupported, g_invalid, g_device_error;
}
