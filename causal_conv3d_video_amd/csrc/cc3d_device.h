// Shared by the kernel translation units and the launcher: the kernel
// argument block, the device helpers every kernel uses, and the per-family
// launch functions each kernel file defines.
#pragma once
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdint>
#include <type_traits>
#include <utility>

#include "cc3d_internal.h"

namespace cc3d {

constexpr int kMaxFrameIv = 4;   // active-frame intervals (one per temporal tap, k_t <= 4)
constexpr int kMaxTapsBf16 = 4;  // temporal taps the bf16 kernels track per tile

// Kernel arguments of one launch (passed by value).
struct ConvArgs {
  const void* x;
  const void* cache;
  const void* w;    // weights as the caller stores them: [C_out][k_t][k_h][k_w][C_in]
  const void* b;
  void* out;
  const void* wpk;  // halo-staged kernels: weights packed in stage order, or null to
                    // gather each stage's weights from w in place
  int n, tx, tc, h, wd, cin, cout, to, ho, wo;
  int kt, kh, kw, sh, sw, dh, dw, ph, pw;
  int tz;
  int st;  // temporal stride: output frame o reads source frame o*st + delta[k]
  int delta[CC3D_MAX_KT];
  int tiles_x, tiles_y, nblk_n, ntiles;
  int has_bias;
  // Group-staged kernel.  Output frames with at least one active tap, as
  // disjoint intervals [act_lo, act_lo + act_n) (its tiles enumerate only
  // these, ta_n frames in all, nat tiles), the other frames (output = bias),
  // and this launch's slot of the scheduler counter table (a tile counter
  // per XCD and a count of finished workgroups, all zero at launch; the
  // launch leaves them zero).
  int act_lo[kMaxFrameIv], act_n[kMaxFrameIv], nact_iv, ta_n;
  int ina_lo[kMaxFrameIv + 1], ina_n[kMaxFrameIv + 1], nina_iv;
  int nat;
  int sched_slot;
  // Few-output-channel kernel: output rows per patch (1..16), and 8-bit
  // pixel codes instead of bf16 output,
  // code = trunc(clamp(fma(y, px_scale, px_offset) * 255, 0, 255)) in fp32.
  int tile_h;
  // Few-output-channel and group-staged kernels: they also write the
  // cache-out (source frames co_lo .. tz - 1 into cache_out[n][0 .. tz -
  // co_lo)); co_lo = tz when not.
  void* cache_out;
  int co_lo;
  int out_u8;
  float px_scale, px_offset;
  // Split reduction (conv_bf16_mfma): each tile's stages are divided among
  // `splits` work units (tile-major, split-minor; ntiles counts the units).
  // With splits > 1 every unit writes its fp32 partial sums to the
  // workspace at ws + ws_part, counts itself in the tile's arrival counter
  // at ws (an int per tile, zero at launch), and the last unit to arrive sums
  // the partials in split order -- the same order whichever unit arrives
  // last -- adds the bias and stores the tile; it leaves the counter zero.
  int splits;
  void* ws;
  int64_t ws_part;
};

// Scheduler counter table of the group-staged kernel (a static device array
// of its translation unit): slots [0, kSchedEager) are handed out to eager
// launches in turn, slots [kSchedEager, kSchedSlots) to launches recorded
// during stream capture, so a captured launch, which keeps its slot for every
// replay, never shares one with an eager launch.
constexpr int kSchedEager = 1024;
constexpr int kSchedSlots = 2048;
int next_sched_slot(bool capturing);

// Launch functions of the kernel families.  `tiles` is the number of work
// units, `cus` the compute units of the device.  Kernels whose weights are
// packed read a.wpk when it is set and gather from a.w otherwise.
hipError_t launch_mfma_family(int kernel_id, int cin_chunk, const ConvArgs& a, int64_t tiles, int cus,
                              hipStream_t s);
hipError_t launch_g32_family(int kernel_id, const ConvArgs& a, int64_t tiles, int cus, hipStream_t s);
template <int COUT>
hipError_t launch_few_cout(const ConvArgs& a, int64_t tiles, int cus, hipStream_t s);  // C_out = COUT (1..5)
hipError_t launch_gen_family(int kernel_id, const ConvArgs& a, int64_t tiles, hipStream_t s);
hipError_t launch_s1rd(const ConvArgs& a, int64_t tiles, int cus, hipStream_t s);
hipError_t launch_f32_direct(const ConvArgs& a, int64_t tiles, hipStream_t s);
hipError_t launch_copy_tail(const void* x, const void* cache, void* dst, int64_t frame_bytes, int n, int tx, int tc,
                            int frames, bool vec16, hipStream_t s);
// Writes the stage-ordered weight image of the halo-staged kernels (block_n
// output channels per tile, ks x ks spatial taps, cin_chunk channels per
// stage) from w into dst.
hipError_t pack_stage_weights(int block_n, int ks, int cin_chunk, const ConvArgs& a, void* dst, hipStream_t s);

}  // namespace cc3d

namespace {

using cc3d::ConvArgs;
using cc3d::kMaxFrameIv;
using cc3d::kMaxTapsBf16;

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ __attribute__((unused)) float bf16_to_f32(unsigned short h) {
  return __uint_as_float(static_cast<unsigned>(h) << 16);
}

// Round to nearest, ties to even (hardware conversion on gfx950).
__device__ __forceinline__ __attribute__((unused)) unsigned short f32_to_bf16(float f) {
  return __builtin_bit_cast(unsigned short, static_cast<__bf16>(f));
}

// Two fp32 values rounded to nearest even and packed as bf16, lo in bits
// 0-15 (one v_cvt_pk_bf16_f32).
__device__ __forceinline__ __attribute__((unused)) unsigned pack_bf16x2(float lo, float hi) {
  const f32x2_t f = {lo, hi};
  return __builtin_bit_cast(unsigned, __builtin_convertvector(f, bf16x2_t));
}

__device__ __forceinline__ __attribute__((unused)) int tap_delta(const ConvArgs& a, int k) {
  int d = 0;
#pragma unroll
  for (int q = 0; q < CC3D_MAX_KT; ++q)
    if (q == k) d = a.delta[q];
  return d;
}

// A kernel's argument block (its first and only argument), read through a pointer the compiler cannot
// see through: fields read this way (by the per-tile bookkeeping, which runs
// once per tile) are loaded where they are used instead of being held in
// scalar registers across the MFMA loop.
typedef const __attribute__((address_space(4))) ConvArgs* KArgs;
__device__ __forceinline__ KArgs kargs() {
  KArgs p = (KArgs)(__builtin_amdgcn_kernarg_segment_ptr());
  asm volatile("" : "+s"(p));
  return p;
}

// Wave-uniform copy of a pointer (kept in scalar registers).
__device__ __forceinline__ __attribute__((unused)) const void* uniform_ptr(const void* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint64_t lo = uint32_t(__builtin_amdgcn_readfirstlane(int(uint32_t(v))));
  const uint64_t hi = uint32_t(__builtin_amdgcn_readfirstlane(int(uint32_t(v >> 32))));
  return reinterpret_cast<const void*>((hi << 32) | lo);
}

// XOR swizzle of the 16-byte pieces of one LDS row (a halo pixel, or one
// (output channel, spatial tap) row of weights).  A 16-byte LDS read is
// served 16 lanes at a time from a 256-byte window of banks, so the reads of
// 16 consecutive rows at the same piece must land in 16 distinct 16-byte
// slots: with PZ pieces per row, rows r and r + 16/PZ would collide, and
// XOR-ing the piece index with bits of r above log2(16/PZ) separates them.
template <int PZ>
__device__ __forceinline__ int swz(int row) {
  if constexpr (PZ == 2) return (row >> 3) & 1;
  else if constexpr (PZ == 4) return (row >> 2) & 3;
  else return (row >> 1) & 7;
}

// Geometry shared by the MFMA kernels and the weight packer.  A stage's
// weight tile is planar: 16-byte piece q (8 input channels) outermost, then
// output channel, then spatial tap -- slot q*PLANE + col*S + s.  Lanes that
// read consecutive output channels at one (q, s) then step S slots apart; S
// (1 or 9) is odd, so any 16 consecutive lanes hit 16 distinct 16-byte slots
// of a 256-byte bank window, and the slot is linear in the lane.
template <int BN, int KS, int CB>
struct WTile {
  static constexpr int S = KS * KS;
  static constexpr int PZ = CB / 8;                       // 16-byte pieces per row
  static constexpr int PLANE = BN * S;                    // slots per piece plane
  static constexpr int WCH = PZ * PLANE;                  // used slots
  static constexpr int WSLOTS = (WCH + 63) / 64 * 64;     // slots per stage tile (whole wave loads)
};

// Byte offset, relative to the start of a stage's weights in W, of the
// 16-byte piece that weight-tile slot `id` holds, or an offset past any
// buffer's range for padding slots (the range check then writes zeros).  A
// stage (channel block nb, chunk cc, tap k) starts at element
// ((nb*BN*kt + k)*S)*cin + cc*CB of W; slot (q, col, s) lies
// (col*kt*S + s)*cin + q*8 elements further.  Output channels past C_out
// fall past the end of W, which the buffer's record count excludes.
template <int BN, int KS, int CB>
__device__ __forceinline__ int w_gather_offset(int id, int kt, int cin) {
  using T = WTile<BN, KS, CB>;
  if (id >= T::WCH) return int(0x80000000u);
  const int q = id / T::PLANE, rem = id % T::PLANE;
  const int col = rem / T::S, s = rem % T::S;
  return ((col * kt * T::S + s) * cin + q * 8) * 2;
}

// Calls f(std::integral_constant<int, i>) for i = I, I+1, .. N-1, unrolled,
// while f returns true (each call nested in the previous one's branch).
template <int I, int N, typename F>
__device__ __forceinline__ void static_for_while(F&& f) {
  if constexpr (I < N) {
    if (f(std::integral_constant<int, I>{})) static_for_while<I + 1, N>(f);
  }
}

// Host side: one launch of `kernel` with the argument block.
inline hipError_t launch_conv(const void* kernel, const ConvArgs& a, int64_t grid, hipStream_t s, int threads = 256) {
  ConvArgs arg = a;
  void* args[] = {&arg};
  return hipLaunchKernel(kernel, dim3(unsigned(grid)), dim3(unsigned(threads)), args, 0, s);
}

// Host side: launch a persistent kernel with as many workgroups as fit on
// the device at once (the per-CU occupancy is queried once per kernel).
template <const void* (*KernelOf)()>
hipError_t launch_persistent(const ConvArgs& a, int64_t tiles, int cus, int threads, hipStream_t s) {
  const void* kernel = KernelOf();
  static std::atomic<int> per_cu{0};
  int occ = per_cu.load(std::memory_order_relaxed);
  if (occ <= 0) {
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kernel, threads, 0) != hipSuccess || occ <= 0) occ = 1;
    per_cu.store(occ, std::memory_order_relaxed);
  }
  return launch_conv(kernel, a, std::min<int64_t>(tiles, int64_t(cus) * occ), s, threads);
}

}  // namespace
