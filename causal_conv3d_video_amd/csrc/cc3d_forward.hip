// Kernels and launcher of the cached causal Conv3D on gfx950 (MI355X).
//
// The operation ("Cache-Aware Conv3D Lowering Across Embedded World-Model
// Decoders", lowering section): output frame o sums, over the active
// temporal taps k, the bias-free spatial Conv2D of source frame o + delta_k of
// Z = [C; X] with the weight slice W[:, :, k], and adds the bias once.  The
// paper evaluates each active tap as its own batched Conv2D; here every
// active tap, every spatial tap and every input channel is one K reduction of
// an implicit GEMM held in MFMA accumulators, and Z is read in place from the
// cache and input buffers (no concatenation, no per-tap weight copies).
//
//   GEMM view per output frame:  D[co][pixel] = sum_K  W[co][K] * Z[K][pixel]
//   K = (active tap k, spatial tap (a, c), input channel ci)
//
// The kernels (all channels-last, fp32 accumulation, bias added once in
// fp32 and rounded to nearest even at the end; the launcher picks one per
// plan, see cc3d_plan.cpp):
//   * conv_bf16_g32: large 3x3 maps, also at spatial dilation 2 ("same")
//     and at spatial stride 2.  One persistent workgroup per compute unit (8
//     waves; 4 or 8 at stride 2) with per-XCD tile counters; a tile is one output
//     frame x a 16x32 or 24x32 output patch (4x32 at stride 2) x 96 or 64
//     output channels.  The halo of one (active tap, 32-channel group) is
//     staged once into LDS and serves 9 spatial taps x 2 sub-stages of 16
//     channels; v_mfma_f32_32x32x16_bf16 with the weights as A and the halo
//     pixels as B.
//   * conv_bf16_mfma: smaller 3x3 maps (two workgroups per compute unit),
//     other C_out, and the 1x1 / (k_t,1,1) convs.
//   * conv_bf16_few: C_out <= 5 (the RGB head).  Walks time per patch,
//     streaming whole halo rows; the (temporal tap, output channel) pairs are
//     the MFMA columns, rotated across lanes after each frame.
//   * conv_bf16_gen: any other spatial kernel size, stride, dilation or
//     padding, gathering each spatial tap's input pixels.
//   * conv_f32_direct: the fp32 path, one output per thread.
//   * copy_tail_frames: the cache-out (the head kernel writes its own).
// Operands reach LDS through direct-to-LDS buffer loads; the buffer range
// check writes the zero padding.  LDS layouts are XOR-swizzled so that the
// 16-byte operand reads of a fragment hit distinct banks.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdint>
#include <mutex>
#include <type_traits>
#include <utility>

#include "cc3d_internal.h"

namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

constexpr int kMaxFrameIv = 4;  // active-frame intervals (one per temporal tap, k_t <= 4)

struct ConvArgs {
  const void* x;
  const void* cache;
  const void* w;
  const void* b;
  void* out;
  const void* wpk;  // bf16 kernels: weights repacked in stage order
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
  // and this launch's scheduler counters: a tile counter per XCD and a count
  // of finished workgroups, all zero at launch.
  int act_lo[kMaxFrameIv], act_n[kMaxFrameIv], nact_iv, ta_n;
  int ina_lo[kMaxFrameIv + 1], ina_n[kMaxFrameIv + 1], nina_iv;
  int nat;
  int* sched;
  // Few-output-channel kernel: output rows per patch (1..16), and 8-bit
  // pixel codes instead of bf16 output,
  // code = trunc(clamp(fma(y, px_scale, px_offset) * 255, 0, 255)) in fp32.
  int tile_h;
  // Few-output-channel kernel: it also writes the cache-out (source frames
  // co_lo .. tz - 1 into cache_out[n][0 .. tz - co_lo)); co_lo = tz when not.
  void* cache_out;
  int co_lo;
  int out_u8;
  float px_scale, px_offset;
};

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

__device__ __forceinline__ int tap_delta(const ConvArgs& a, int k) {
  int d = 0;
#pragma unroll
  for (int q = 0; q < CC3D_MAX_KT; ++q)
    if (q == k) d = a.delta[q];
  return d;
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

// Geometry shared by the MFMA kernel and the weight packer.  A stage's
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

// Weight packer: writes, for every (output-channel block nb, input-channel
// chunk cc, tap k) in that order, the exact 16-byte slot image of the LDS
// weight tile the MFMA kernel consumes in that stage (planar, zeros beyond
// C_out), so a stage's weights are one contiguous run that streams into LDS
// with fully used cache lines.
template <int BN, int KS, int CB>
__global__ __launch_bounds__(256) void pack_weights(const unsigned short* __restrict__ w,
                                                    uint4* __restrict__ wpk, int cout, int kt, int cin,
                                                    int nblk_n, int64_t total) {
  using T = WTile<BN, KS, CB>;
  const int nch = cin / CB;
  for (int64_t idx = int64_t(blockIdx.x) * 256 + threadIdx.x; idx < total; idx += int64_t(gridDim.x) * 256) {
    const int id = int(idx % T::WSLOTS);
    const int64_t tile = idx / T::WSLOTS;
    const int k = int(tile % kt);
    const int rest = int(tile / kt);
    const int cc = rest % nch, nb = rest / nch;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (id < T::WCH) {
      const int q = id / T::PLANE, rem = id % T::PLANE;
      const int col = rem / T::S, s = rem % T::S;
      const int co = nb * BN + col;
      if (co < cout)
        v = *reinterpret_cast<const uint4*>(w + ((int64_t(co) * kt + k) * T::S + s) * cin + cc * CB + q * 8);
    }
    wpk[idx] = v;
  }
}

constexpr int kMaxTapsBf16 = 4;  // temporal taps the bf16 kernels track per tile

template <int BN, int TH, int WM, int WN, int KS, int CB, int NBUF, int OCC>
__global__ __launch_bounds__(WM * WN * 64) __attribute__((amdgpu_waves_per_eu(OCC, OCC))) void conv_bf16_mfma(ConvArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)  // the host pass only needs the launch stub
  using WT = WTile<BN, KS, CB>;
  constexpr int TW = 32;                       // patch width = MFMA pixel block
  constexpr int PAD = (KS - 1) / 2;
  constexpr int HP = TH + KS - 1, WP = TW + KS - 1, S = KS * KS;
  constexpr int PZ = CB / 8;                   // 16-byte pieces per pixel per stage
  constexpr int ZCH = HP * WP * PZ;
  constexpr int ZSLOTS = (ZCH + 63) / 64 * 64; // 16-byte LDS slots of the halo tile
  constexpr int NW = WM * WN, NT = NW * 64;    // waves, threads per workgroup
  constexpr int ZIT = (ZSLOTS + NT - 1) / NT;
  constexpr int WSLOTS = WT::WSLOTS, WIT = (WSLOTS + NT - 1) / NT;
  constexpr int RW = TH / WM;                  // patch rows per wave
  constexpr int CW = BN / (32 * WN);           // 32-channel blocks per wave
  // each LDS buffer holds one stage (halo + weights), and at a tile's end the
  // idle buffer stages the epilogue's output rows (4 waves x 32 pixels)
  constexpr int EROW = CW * 32 * 2 + 16;       // epilogue LDS bytes per pixel (padded)
  constexpr int STAGE = (ZSLOTS + WSLOTS) > (NW * 32 * EROW + 15) / 16 ? (ZSLOTS + WSLOTS)
                                                                        : (NW * 32 * EROW + 15) / 16;
  // load instructions one wave issues per stage (waves past a tile's last
  // 64-slot block issue fewer)
  constexpr auto lps_of = [](int w) {
    int n = 0;
    for (int it = 0; it < ZIT; ++it) n += it * NT + w * 64 < ZSLOTS;
    for (int it = 0; it < WIT; ++it) n += it * NT + w * 64 < WSLOTS;
    return n;
  };
  constexpr int LPS = ZIT + WIT;               // upper bound over the waves
  static_assert((NW == 4 || NW == 8) && TH % WM == 0 && BN % (32 * WN) == 0, "wave tiling");
  static_assert(PZ == 2 || PZ == 4 || PZ == 8, "stage channels");
  constexpr int WG_PER_CU = OCC * 4 / NW > 0 ? OCC * 4 / NW : 1;  // OCC is waves per SIMD
  static_assert(NBUF >= 2 && (NBUF * STAGE * 16 + 2 * BN * 4) * WG_PER_CU <= 160 * 1024, "LDS budget");
  static_assert(LPS * (NBUF - 2) <= 63, "vmcnt range");

  __shared__ uint4 lds[NBUF * STAGE];
  __shared__ float bias_lds[2][BN];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const int g = lane >> 5, l32 = lane & 31;

  // Persistent schedule.  Workgroups are dispatched round-robin over the 8
  // XCDs (workgroup b runs on XCD b % 8); each XCD owns one contiguous range
  // of tiles, which its workgroups walk together, so the tiles that run at
  // the same time on one XCD are neighbours: adjacent patches, and the output
  // frames of one patch that read the same source frames, meet in one L2.
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int nblk_here = (int(gridDim.x) >> 3) + (xcd < int(gridDim.x & 7) ? 1 : 0);
  const int tq = a.ntiles >> 3, tr = a.ntiles & 7;
  const int t_begin = xcd * tq + min(xcd, tr);
  const int t_end = t_begin + tq + (xcd < tr ? 1 : 0);
  int ctile = t_begin + slot;
  if (ctile >= t_end) return;  // uniform over the workgroup
  auto next_tile = [&](int t) { return t + nblk_here < t_end ? t + nblk_here : -1; };

  const int nch = a.cin / CB;
  const int64_t frame_el = int64_t(a.h) * a.wd * a.cin;
  const int frame_bytes = int(frame_el * 2);
  const unsigned short* __restrict__ xs = static_cast<const unsigned short*>(a.x);
  const unsigned short* __restrict__ cs = static_cast<const unsigned short*>(a.cache);
  const unsigned char* __restrict__ wpk = static_cast<const unsigned char*>(a.wpk);
  const unsigned short* __restrict__ bs = static_cast<const unsigned short*>(a.b);
  unsigned short* __restrict__ os = static_cast<unsigned short*>(a.out);

  // A tile: one output frame o of batch item nn, a TH x 32 patch at (y0, x0),
  // output channels [n0, n0 + BN); its active taps k[0..nact) read source
  // frames z[i] = o + delta_k[i] of Z = [cache; x].
  struct Tile {
    int o, nb, nn, x0, y0, n0, nact;
    int k0, k1, k2, k3;  // active taps, in order
    int z0, z1, z2, z3;  // their source frames
  };
  auto decode = [&](int t) {
    Tile c;
    c.o = t % a.to;
    t /= a.to;
    c.nb = t % a.nblk_n;
    t /= a.nblk_n;
    const int tile_x = t % a.tiles_x;
    t /= a.tiles_x;
    const int tile_y = t % a.tiles_y;
    c.nn = t / a.tiles_y;
    c.x0 = tile_x * TW;
    c.y0 = tile_y * TH;
    c.n0 = c.nb * BN;
    c.nact = 0;
    c.k0 = c.k1 = c.k2 = c.k3 = 0;
    c.z0 = c.z1 = c.z2 = c.z3 = 0;
#pragma unroll
    for (int k = 0; k < kMaxTapsBf16; ++k) {
      const int z = c.o * a.st + a.delta[k];
      if (k < a.kt && z >= 0 && z < a.tz) {
        if (c.nact == 0) { c.k0 = k; c.z0 = z; }
        else if (c.nact == 1) { c.k1 = k; c.z1 = z; }
        else if (c.nact == 2) { c.k2 = k; c.z2 = z; }
        else { c.k3 = k; c.z3 = z; }
        ++c.nact;
      }
    }
    return c;
  };
  auto pick = [](int i, int v0, int v1, int v2, int v3) { return i == 0 ? v0 : i == 1 ? v1 : i == 2 ? v2 : v3; };
  // wave-uniform copy of a pointer (kept in scalar registers)
  auto uniform = [](const void* p) {
    const uint64_t v = reinterpret_cast<uint64_t>(p);
    const uint64_t lo = uint32_t(__builtin_amdgcn_readfirstlane(int(uint32_t(v))));
    const uint64_t hi = uint32_t(__builtin_amdgcn_readfirstlane(int(uint32_t(v >> 32))));
    return reinterpret_cast<const void*>((hi << 32) | lo);
  };

  // Byte offset, within a frame, of every halo slot this thread fills (slot
  // id = it*256 + tid); slots in the spatial zero padding get an offset past
  // the buffer's record count, and the range check of the buffer load then
  // writes zeros into LDS.
  constexpr int OOB = int(0x80000000u);
  int zoff[ZIT];
  auto halo_offsets = [&](const Tile& c) {
#pragma unroll
    for (int it = 0; it < ZIT; ++it) {
      const int id = tid + NT * it;
      int off = OOB;
      if (id < ZCH) {
        const int pix = id / PZ;
        const int q = (id % PZ) ^ swz<PZ>(pix);
        const int y = c.y0 - PAD + pix / WP, x = c.x0 - PAD + pix % WP;
        if (y >= 0 && y < a.h && x >= 0 && x < a.wd) off = ((y * a.wd + x) * a.cin + q * 8) * 2;
      }
      zoff[it] = off;
    }
  };

  // Stage (cc, ti) of a tile: input-channel chunk cc, active tap ti.  Stage
  // order is tap major, chunk minor: consecutive stages read consecutive
  // 32-byte pieces of the same halo pixels, so the 128-byte lines fetched
  // for one stage serve the next stages from L2.
  // A stage's loads are prepared once (buffer descriptors, LDS targets) and
  // then issued one 64-slot wave instruction at a time, spread over the first
  // steps of the previous stage's MFMA loop: a burst of all of them would fill
  // the vector-memory queue and stall the wave at issue instead of overlapping.
  struct StageLoad {
    const unsigned short* fp;  // halo source: frame base + chunk offset
    const unsigned char* wp;   // packed weight tile
    int buf;                   // LDS buffer
  };
  auto prep_stage = [&](const Tile& c, int cc, int ti, int buf) {
    const int z = pick(ti, c.z0, c.z1, c.z2, c.z3), k = pick(ti, c.k0, c.k1, c.k2, c.k3);
    StageLoad l;
    l.fp = static_cast<const unsigned short*>(uniform((z < a.tc ? cs + (int64_t(c.nn) * a.tc + z) * frame_el
                                                                 : xs + (int64_t(c.nn) * a.tx + (z - a.tc)) * frame_el) +
                                                      cc * CB));
    l.wp = static_cast<const unsigned char*>(uniform(wpk + ((int64_t(c.nb) * nch + cc) * a.kt + k) * (WSLOTS * 16)));
    l.buf = __builtin_amdgcn_readfirstlane(buf);
    return l;
  };
  constexpr int NLOAD = ZIT + WIT;  // load instructions of one stage, per thread
  // slots are filled 64 at a time (one wave instruction); a wave whose
  // 64-slot block lies past the tile issues nothing
  auto issue_piece = [&](const StageLoad& l, int j) {
    uint4* zb = lds + l.buf * STAGE;
    if (j < ZIT) {
      if (ZSLOTS % NT == 0 || j * NT + wave * 64 < ZSLOTS) {
        const __amdgpu_buffer_rsrc_t zr =
            __builtin_amdgcn_make_buffer_rsrc(const_cast<unsigned short*>(l.fp), 0, frame_bytes, 0x00020000);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(zr, (__attribute__((address_space(3))) void*)(zb + j * NT + wave * 64),
                                                 16, zoff[j], 0, 0, 0);
      }
    } else {
      const int it = j - ZIT;
      if (WSLOTS % NT == 0 || it * NT + wave * 64 < WSLOTS) {
        const __amdgpu_buffer_rsrc_t wr =
            __builtin_amdgcn_make_buffer_rsrc(const_cast<unsigned char*>(l.wp), 0, WSLOTS * 16, 0x00020000);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(wr,
                                                 (__attribute__((address_space(3))) void*)(zb + ZSLOTS + it * NT + wave * 64),
                                                 16, (it * NT + tid) * 16, 0, 0, 0);
      }
    }
  };
  auto load_stage = [&](const Tile& c, int cc, int ti, int buf) {
    const StageLoad l = prep_stage(c, cc, ti, buf);
#pragma unroll
    for (int j = 0; j < NLOAD; ++j) issue_piece(l, j);
  };

  f32x16_t acc[CW][RW];
  auto zero_acc = [&]() {
#pragma unroll
    for (int q = 0; q < CW; ++q)
#pragma unroll
      for (int r = 0; r < RW; ++r)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[q][r][v] = 0.f;
  };

  // One stage = (CB/16) x KS x KS steps; a step is one spatial tap (ta, tcol)
  // of one 16-channel slice kk and issues CW x RW MFMAs.  Steps are grouped
  // by (kk, tcol): the RW+KS-1 halo rows of a group serve all KS row taps ta.
  // Operand fragments of step i+1 are read from LDS into a second register
  // set before step i's MFMAs issue, so LDS latency hides behind MFMA work;
  // sched_barrier keeps the compiler from sinking the reads to their uses.
  constexpr int NSTEP = (CB / 16) * KS * KS;
  constexpr int ZR = RW + KS - 1;           // halo rows per group
  auto read_z = [&](const uint4* zb, int grp, bf16x8_t* zf) {
    const int q = (grp / KS) * 2 + g, tcol = grp % KS;
#pragma unroll
    for (int r = 0; r < ZR; ++r) {
      const int pix = (wm * RW + r) * WP + l32 + tcol;
      zf[r] = __builtin_bit_cast(bf16x8_t, zb[pix * PZ + (q ^ swz<PZ>(pix))]);
    }
  };
  auto read_w = [&](const uint4* wb, int step, bf16x8_t* wf) {
    const int grp = step / KS, ta = step % KS;
    const int q = (grp / KS) * 2 + g, s = ta * KS + grp % KS;
#pragma unroll
    for (int c = 0; c < CW; ++c)
      wf[c] = __builtin_bit_cast(bf16x8_t, wb[q * WT::PLANE + ((wn * CW + c) * 32 + l32) * S + s]);
  };
  // Steps over which the next stage's load instructions are spread: the first
  // half of the stage, so they have the second half to land.
  constexpr int ISSUE_STEPS = NSTEP > 1 ? (NSTEP + 1) / 2 : 1;
  auto compute = [&](int buf, bool has_next, const StageLoad& next) {
    const uint4* zb = lds + buf * STAGE;
    const uint4* wb = zb + ZSLOTS;
    bf16x8_t zf[2][ZR], wf[2][CW];
    read_z(zb, 0, zf[0]);
    read_w(wb, 0, wf[0]);
#pragma unroll
    for (int i = 0; i < NSTEP; ++i) {
      if (i + 1 < NSTEP) {
        read_w(wb, i + 1, wf[(i + 1) & 1]);
        if ((i + 1) % KS == 0) read_z(zb, (i + 1) / KS, zf[((i + 1) / KS) & 1]);
      }
      __builtin_amdgcn_sched_barrier(0);
      const int ta = i % KS, zsel = (i / KS) & 1;
#pragma unroll
      for (int c = 0; c < CW; ++c)
#pragma unroll
        for (int r = 0; r < RW; ++r)
          acc[c][r] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[i & 1][c], zf[zsel][r + ta], acc[c][r], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
      if (has_next && i < ISSUE_STEPS) {
#pragma unroll
        for (int j = 0; j < NLOAD; ++j)
          if (j * ISSUE_STEPS / NLOAD == i) issue_piece(next, j);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Epilogue.  The lane holding pixel column l32 of a patch row has channels
  // (v/4)*8 + g*4 + (v%4) of each 32-channel block.  The bias (fp32, from the
  // tile's LDS slot) is added once, the sum rounded to nearest even to bf16,
  // and each patch row of this wave -- 32 pixels x CW*32 channels -- goes
  // through a private LDS region (the just-consumed stage buffer) so that
  // global stores are whole 16-byte pieces of contiguous channel runs.
  constexpr int EPIX = CW * 4;                   // 16-byte pieces per pixel
  constexpr int EIT = (32 * EPIX + 63) / 64;     // store rounds per patch row
  static_assert(NW * 32 * EROW <= STAGE * 16, "epilogue staging fits a stage buffer");
  const bool vec_ok = (a.cout & 7) == 0;
  auto epilogue = [&](const Tile& c, int par, int buf) {
    unsigned char* eb = reinterpret_cast<unsigned char*>(lds + buf * STAGE) + wave * 32 * EROW;
    const int cbase = c.n0 + wn * CW * 32;     // first channel of this wave
#pragma unroll
    for (int r = 0; r < RW; ++r) {
      const int y = c.y0 + wm * RW + r;
      if (y >= a.ho) continue;                  // uniform over the wave
#pragma unroll
      for (int q = 0; q < CW; ++q) {
#pragma unroll
        for (int v4 = 0; v4 < 4; ++v4) {
          const int cl = q * 32 + v4 * 8 + g * 4;
          const float4 bv = *reinterpret_cast<const float4*>(&bias_lds[par][wn * CW * 32 + cl]);
          uint2 pk;
          pk.x = unsigned(f32_to_bf16(acc[q][r][v4 * 4 + 0] + bv.x)) |
                 (unsigned(f32_to_bf16(acc[q][r][v4 * 4 + 1] + bv.y)) << 16);
          pk.y = unsigned(f32_to_bf16(acc[q][r][v4 * 4 + 2] + bv.z)) |
                 (unsigned(f32_to_bf16(acc[q][r][v4 * 4 + 3] + bv.w)) << 16);
          *reinterpret_cast<uint2*>(eb + l32 * EROW + cl * 2) = pk;
        }
      }
      unsigned short* orow = os + ((int64_t(c.nn) * a.to + c.o) * a.ho + y) * int64_t(a.wo) * a.cout;
#pragma unroll
      for (int it = 0; it < EIT; ++it) {
        const int piece = it * 64 + lane;
        if (piece < 32 * EPIX) {
          const int px = piece / EPIX, ch = (piece % EPIX) * 8;
          const int xo = c.x0 + px, co = cbase + ch;
          const uint4 v = *reinterpret_cast<const uint4*>(eb + px * EROW + ch * 2);
          if (xo < a.wo && co < a.cout) {
            unsigned short* op = orow + int64_t(xo) * a.cout + co;
            if (vec_ok) {
              *reinterpret_cast<uint4*>(op) = v;
            } else {
              const unsigned short* hv = reinterpret_cast<const unsigned short*>(&v);
#pragma unroll
              for (int e = 0; e < 8; ++e)
                if (co + e < a.cout) op[e] = hv[e];
            }
          }
        }
      }
    }
  };
  auto bias_value = [&](const Tile& c) {
    return (a.has_bias && tid < BN && c.n0 + tid < a.cout) ? bs[c.n0 + tid] : (unsigned short)0;
  };

  // Load cursor: runs NBUF-1 stages ahead of the compute cursor over the
  // flattened (tile, stage) sequence, crossing tile boundaries, so a tile's
  // first stages load while the previous tile finishes and writes its
  // outputs.  Stage position p uses LDS buffer p % NBUF.
  int ltile = ctile, lcc = 0, lti = 0;
  Tile lt = decode(ltile);
  auto lt_advance_tile = [&]() {
    lcc = 0;
    lti = 0;
    for (;;) {
      ltile = next_tile(ltile);
      if (ltile < 0) return;
      lt = decode(ltile);
      if (lt.nact > 0) break;
    }
    halo_offsets(lt);
  };
  if (lt.nact > 0) halo_offsets(lt);
  else lt_advance_tile();
  auto advance_load = [&]() {
    if (++lcc == nch) {
      lcc = 0;
      if (++lti == lt.nact) lt_advance_tile();
    }
  };
  auto issue = [&](int buf) {  // whole stage at once (pipeline prologue)
    if (ltile < 0) return false;
    load_stage(lt, lcc, lti, buf);
    advance_load();
    return true;
  };

  // Wait until this wave's loads of all but the NBUF-2 newest stages have
  // landed (vmcnt counts the wave's own outstanding loads, in issue order).
  auto wait_newer_stages = [&]() {
    if constexpr (NBUF > 2) {
      switch (wave) {
        case 0: asm volatile("s_waitcnt vmcnt(%0)" ::"n"(lps_of(0) * (NBUF - 2)) : "memory"); break;
        case 1: asm volatile("s_waitcnt vmcnt(%0)" ::"n"(lps_of(1) * (NBUF - 2)) : "memory"); break;
        case 2: asm volatile("s_waitcnt vmcnt(%0)" ::"n"(lps_of(2) * (NBUF - 2)) : "memory"); break;
        case 3: asm volatile("s_waitcnt vmcnt(%0)" ::"n"(lps_of(3) * (NBUF - 2)) : "memory"); break;
        case 4: asm volatile("s_waitcnt vmcnt(%0)" ::"n"(lps_of(4) * (NBUF - 2)) : "memory"); break;
        case 5: asm volatile("s_waitcnt vmcnt(%0)" ::"n"(lps_of(5) * (NBUF - 2)) : "memory"); break;
        case 6: asm volatile("s_waitcnt vmcnt(%0)" ::"n"(lps_of(6) * (NBUF - 2)) : "memory"); break;
        default: asm volatile("s_waitcnt vmcnt(%0)" ::"n"(lps_of(7) * (NBUF - 2)) : "memory"); break;
      }
    } else {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
  };

  int issued = 0;
#pragma unroll
  for (int i = 0; i < NBUF - 1; ++i)
    if (issue(i)) ++issued;
  if (NBUF > 2 && issued == NBUF - 1) wait_newer_stages();
  else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();

  int pos = 0, par = 0;
  Tile ct = decode(ctile);
  for (;;) {
    zero_acc();
    const int nst = ct.nact * nch;
    if (nst == 0) {
      // no active tap: the output is the bias alone
      if (tid < BN) bias_lds[par][tid] = bf16_to_f32(bias_value(ct));
      __syncthreads();
      epilogue(ct, par, pos % NBUF);
      __syncthreads();
    } else {
      for (int st = 0; st < nst; ++st, ++pos) {
        unsigned short bval = 0;
        if (st == 0) bval = bias_value(ct);  // issued before this stage's loads
        const bool more = ltile >= 0;
        const StageLoad nl = prep_stage(lt, lcc, lti, (pos + NBUF - 1) % NBUF);
        compute(pos % NBUF, more, nl);
        if (more) advance_load();  // after the pieces: they read this tile's halo offsets
        if (st == 0 && tid < BN) bias_lds[par][tid] = bf16_to_f32(bval);
        // wait until stage pos+1 has landed (the NBUF-2 newer stages may stay
        // in flight); the barrier then publishes everyone's loads and the
        // bias, and retires this stage's LDS reads
        if (NBUF > 2 && more) wait_newer_stages();
        else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
      }
      // the buffer of the last stage is idle until the next stage's loads are
      // issued: stage the outputs through it, then make sure every wave is
      // done with it before those loads go out
      epilogue(ct, par, (pos - 1) % NBUF);
      __syncthreads();
    }
    par ^= 1;
    ctile = next_tile(ctile);
    if (ctile < 0) break;
    ct = decode(ctile);
  }
#endif
}

// bf16 kernel for 3x3 spatial taps with the halo staged by 32-channel groups.
//
// The stage loads of the kernel above fetch 32 bytes (16 channels) of every
// halo pixel per stage; the vector memory pipeline pays per 128-byte line
// touched by a wave instruction, so three quarters of each halo line fetch are
// wasted there and the halo stream alone keeps that pipeline about as busy as
// the MFMAs keep the matrix cores.  This kernel stages the halo of a
// (temporal tap, 32-channel group) once -- 64 bytes per pixel -- and runs the
// group's two 16-channel weight sub-stages against it, and its tiles are
// 16 x 32 output pixels, so each weight byte fetched feeds twice the MFMA work.
// One workgroup per compute unit: WM = 4 waves (one per SIMD, each a 4-row x
// 32-pixel x BN-channel register tile) or WM = 8 (two per SIMD, 2 rows each).
//
// LDS: two halo buffers (group g and g+1) and two weight buffers (sub-stages 0
// and 1 of a group).  Schedule of group g (buffers H[g%2], W[0], W[1]):
//   sub-stage 0: MFMAs on H[g%2] x W[0]; meanwhile load W[1] <- weights of
//                (g, second 16 channels), then H[(g+1)%2] <- halo of g+1;
//                wait for W[1] only; barrier.
//   sub-stage 1: MFMAs on H[g%2] x W[1]; meanwhile load W[0] <- weights of
//                (g+1, first 16 channels); wait for everything; barrier.
// The group sequence runs across tile boundaries, so the next tile's first
// loads overlap the current tile's last MFMAs and its epilogue.
//
// DD is the spatial dilation of the 3x3 taps (1, or 2 for the dilated
// "same" conv, padding 2): the halo grows by DD on every side, and column
// tap c, row tap ta read halo column l + c*DD, halo row r + ta*DD.
//
// SS is the spatial stride (1, or 2 with padding 1 and no dilation, the
// encoder's downsampling conv).  At stride 2 output pixel (r, l) of the tile
// reads input row 2r + ta and input column 2l + c of the halo, which spans
// 2*TH + 1 rows by 2*32 + 1 columns.  Each halo row is stored with its even
// input columns first (33 of them), then its odd ones (32): column tap c then
// reads the 32 consecutive stored pixels from l + c/2 (c even) or 33 + l
// (c = 1), the same conflict-free fragment pattern as at stride 1.
//
// KSP = 2 splits each group's two 16-channel halves between two waves of
// the same rows (waves w and w + WM/2), so a tile of TH rows runs WM waves
// with one barrier per group instead of two; the group's two weight halves
// are staged together (double-buffered: the next group's load during this
// one), and the waves of the second half add their sums into those of the
// first through LDS before the epilogue.
template <int BN, int TH, int WM, int DD = 1, int SS = 1, int KSP = 1>
__global__ __launch_bounds__(WM * 64) __attribute__((amdgpu_waves_per_eu(WM / 4, WM / 4))) void conv_bf16_g32(ConvArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)
  using WT = WTile<BN, 3, 16>;
  static_assert(SS == 1 || (SS == 2 && DD == 1), "stride 2 runs undilated");
  constexpr int TW = 32, S = 9;
  constexpr int HP = SS * (TH - 1) + 2 * DD + 1;             // halo rows
  constexpr int WP = SS == 1 ? TW + 2 * DD : 2 * TW + 1;     // halo columns
  constexpr int PZ = 4;                          // 16-byte pieces per halo pixel
  constexpr int ZCH = HP * WP * PZ;
  constexpr int ZSLOTS = (ZCH + 63) / 64 * 64;
  constexpr int NW = WM, NT = NW * 64;
  constexpr int WSLOTS = WT::WSLOTS;
  constexpr int ZIT = (ZSLOTS + NT - 1) / NT, WIT = (WSLOTS + NT - 1) / NT;
  constexpr int RW = TH / (WM / KSP), CW = BN / 32;
  constexpr int ZR = SS * (RW - 1) + 2 * DD + 1; // halo rows a wave reads per column tap
  constexpr int EROW = CW * 32 * 2 + 16;         // epilogue LDS bytes per pixel (padded)
  static_assert((WM == 4 || WM == 8) && TH % (WM / KSP) == 0 && BN % 32 == 0, "wave tiling");
  static_assert(KSP == 1 || (KSP == 2 && WM == 8), "channel-half split");
  // epilogue staging: waves 0-3 use the idle weight buffer, waves 4-7 the idle halo buffer
  static_assert(4 * 32 * EROW <= WSLOTS * 16 && (NW - 4) * 32 * EROW <= ZSLOTS * 16, "epilogue staging");
  static_assert((2 * ZSLOTS + 2 * KSP * WSLOTS) * 16 + 2 * BN * 4 <= 160 * 1024, "LDS budget");
  // channel-half split: the second half's sums pass through an idle halo buffer
  static_assert(KSP == 1 || (WM / 2) * CW * RW * 16 * 64 * 4 <= ZSLOTS * 16, "partial sums");
  constexpr auto zcnt = [](int w) {  // halo load instructions of wave w per group
    int n = 0;
    for (int it = 0; it < ZIT; ++it) n += it * NT + w * 64 < ZSLOTS;
    return n;
  };
  static_assert(zcnt(0) + WIT <= 63, "vmcnt range");

  __shared__ uint4 zl[2 * ZSLOTS];
  __shared__ uint4 wl[2 * KSP * WSLOTS];
  __shared__ float bias_lds[2][BN];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5, l32 = lane & 31;
  // row group and channel half of this wave (the row group is the wave
  // itself unless the halves are split between waves)
  const int wr = KSP == 1 ? wave : wave & (WM / 2 - 1);
  const int wj = KSP == 1 ? 0 : wave / (WM / 2);

  // Persistent schedule over the tiles of the output frames with an active
  // tap.  Each XCD owns one contiguous range of them (neighbouring tiles
  // share source frames in its L2).  A workgroup's first two tiles are
  // fixed; it claims each later one while the tile before it runs, from its
  // XCD's counter and, once that range is used up, from the other XCDs'
  // counters, so XCDs that run at different clocks still finish together.
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  auto xcd_wgs = [&](int x) { return (int(gridDim.x) >> 3) + (x < int(gridDim.x & 7) ? 1 : 0); };
  auto xcd_begin = [&](int x) { return x * (a.nat >> 3) + min(x, a.nat & 7); };
  auto xcd_len = [&](int x) { return (a.nat >> 3) + (x < (a.nat & 7) ? 1 : 0); };
  auto fixed_tile = [&](int k) {  // k-th fixed tile (k = 0, 1) of this workgroup, or -1
    const int r = slot + k * xcd_wgs(xcd);
    return r < xcd_len(xcd) ? xcd_begin(xcd) + r : -1;
  };
  auto claim = [&](int x) {  // next claim number on XCD x's counter
    return __hip_atomic_fetch_add(a.sched + x, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  };
  auto claimed = [&](int x, int v) {  // the tile of claim v on XCD x, or -1 once its range is used up
    const int r = 2 * xcd_wgs(x) + v;
    return r < xcd_len(x) ? xcd_begin(x) + r : -1;
  };
  int ctile = fixed_tile(0), tnext = fixed_tile(1), tnn = -1;  // this tile, the next two
  int steal = 0;  // (thread 0) offset of the XCD whose counter it claims from
  __shared__ int claim_lds;

  const int ngrp = a.cin / 32;                   // 32-channel groups per tap
  const int nch = a.cin / 16;                    // 16-channel weight sub-stages per tap
  const int64_t frame_el = int64_t(a.h) * a.wd * a.cin;
  const int frame_bytes = int(frame_el * 2);
  const unsigned short* __restrict__ xs = static_cast<const unsigned short*>(a.x);
  const unsigned short* __restrict__ cs = static_cast<const unsigned short*>(a.cache);
  const unsigned char* __restrict__ wpk = static_cast<const unsigned char*>(a.wpk);
  const unsigned short* __restrict__ bs = static_cast<const unsigned short*>(a.b);
  unsigned short* __restrict__ os = static_cast<unsigned short*>(a.out);

  struct Tile {
    int o, nb, nn, x0, y0, n0, nact;
    int k0, k1, k2, k3;
    int z0, z1, z2, z3;
  };
  auto act_frame = [&](int j) {  // the j-th output frame with an active tap
    int o = a.act_lo[0] + j;
#pragma unroll
    for (int i = 0; i + 1 < kMaxFrameIv; ++i)
      if (i + 1 < a.nact_iv && j >= a.act_n[i]) {
        j -= a.act_n[i];
        o = a.act_lo[i + 1] + j;
      }
    return o;
  };
  auto decode = [&](int t) {
    Tile c;
    c.o = act_frame(t % a.ta_n);
    t /= a.ta_n;
    c.nb = t % a.nblk_n;
    t /= a.nblk_n;
    const int tile_x = t % a.tiles_x;
    t /= a.tiles_x;
    const int tile_y = t % a.tiles_y;
    c.nn = t / a.tiles_y;
    c.x0 = tile_x * TW;
    c.y0 = tile_y * TH;
    c.n0 = c.nb * BN;
    c.nact = 0;
    c.k0 = c.k1 = c.k2 = c.k3 = 0;
    c.z0 = c.z1 = c.z2 = c.z3 = 0;
#pragma unroll
    for (int k = 0; k < kMaxTapsBf16; ++k) {
      const int z = c.o * a.st + a.delta[k];
      if (k < a.kt && z >= 0 && z < a.tz) {
        if (c.nact == 0) { c.k0 = k; c.z0 = z; }
        else if (c.nact == 1) { c.k1 = k; c.z1 = z; }
        else if (c.nact == 2) { c.k2 = k; c.z2 = z; }
        else { c.k3 = k; c.z3 = z; }
        ++c.nact;
      }
    }
    return c;
  };
  auto pick = [](int i, int v0, int v1, int v2, int v3) { return i == 0 ? v0 : i == 1 ? v1 : i == 2 ? v2 : v3; };
  auto uniform = [](const void* p) {
    const uint64_t v = reinterpret_cast<uint64_t>(p);
    const uint64_t lo = uint32_t(__builtin_amdgcn_readfirstlane(int(uint32_t(v))));
    const uint64_t hi = uint32_t(__builtin_amdgcn_readfirstlane(int(uint32_t(v >> 32))));
    return reinterpret_cast<const void*>((hi << 32) | lo);
  };

  // Byte offsets within a frame of the halo slots this thread fills (slot id
  // = it*NT + tid; 4 slots of 16 bytes per pixel, XOR-swizzled); slots in the
  // spatial zero padding get an offset past the buffer's record count, and
  // the buffer load's range check writes zeros for them.
  constexpr int OOB = int(0x80000000u);
  int zoff[ZIT];
  auto halo_offsets = [&](const Tile& c) {
#pragma unroll
    for (int it = 0; it < ZIT; ++it) {
      const int id = tid + NT * it;
      int off = OOB;
      if (id < ZCH) {
        const int pix = id / PZ;
        const int q = (id % PZ) ^ swz<PZ>(pix);
        const int col = pix % WP;
        // input column of the stored pixel: at stride 2 the even ones, then the odd
        const int u = SS == 1 ? col : col <= TW ? 2 * col : 2 * (col - TW - 1) + 1;
        const int y = SS * c.y0 - DD + pix / WP, x = SS * c.x0 - DD + u;
        if (y >= 0 && y < a.h && x >= 0 && x < a.wd) off = ((y * a.wd + x) * a.cin + q * 8) * 2;
      }
      zoff[it] = off;
    }
  };

  // A group position: tile, active-tap index, 32-channel group.
  struct Grp {
    int t, ti, gz;
  };
  auto halo_src = [&](const Tile& c, int ti, int gz) {
    const int z = pick(ti, c.z0, c.z1, c.z2, c.z3);
    return static_cast<const unsigned short*>(uniform((z < a.tc ? cs + (int64_t(c.nn) * a.tc + z) * frame_el
                                                                : xs + (int64_t(c.nn) * a.tx + (z - a.tc)) * frame_el) +
                                                     gz * 32));
  };
  auto wsrc = [&](const Tile& c, int ti, int cc) {
    const int k = pick(ti, c.k0, c.k1, c.k2, c.k3);
    return static_cast<const unsigned char*>(uniform(wpk + ((int64_t(c.nb) * nch + cc) * a.kt + k) * (WSLOTS * 16)));
  };
  auto issue_z = [&](const unsigned short* fp, int zb, int it) {
    if (ZSLOTS % NT == 0 || it * NT + wave * 64 < ZSLOTS) {
      const __amdgpu_buffer_rsrc_t r =
          __builtin_amdgcn_make_buffer_rsrc(const_cast<unsigned short*>(fp), 0, frame_bytes, 0x00020000);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          r, (__attribute__((address_space(3))) void*)(zl + zb * ZSLOTS + it * NT + wave * 64), 16, zoff[it], 0, 0, 0);
    }
  };
  auto issue_w = [&](const unsigned char* wp, int wb, int it) {
    if (WSLOTS % NT == 0 || it * NT + wave * 64 < WSLOTS) {
      const __amdgpu_buffer_rsrc_t r =
          __builtin_amdgcn_make_buffer_rsrc(const_cast<unsigned char*>(wp), 0, WSLOTS * 16, 0x00020000);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          r, (__attribute__((address_space(3))) void*)(wl + wb * WSLOTS + it * NT + wave * 64), 16, (it * NT + tid) * 16,
          0, 0, 0);
    }
  };

  f32x16_t acc[CW][RW];
  auto zero_acc = [&]() {
#pragma unroll
    for (int q = 0; q < CW; ++q)
#pragma unroll
      for (int r = 0; r < RW; ++r)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[q][r][v] = 0.f;
  };

  // One sub-stage = 9 steps, one per spatial tap (ta, tcol), grouped by
  // column tap: the halo rows read for a column tap serve its 3 row taps.
  // Fragments of step i+1 are read before step i's MFMAs issue.
  // Sub-stage J multiplies the 16 channels [16J, 16J+16) of the group.
  constexpr int NSTEP = 9;
  auto read_z = [&](const uint4* zb, int tcol, int J, bf16x8_t* zf) {
    const int q = 2 * J + g;
    const int col = SS == 1 ? tcol * DD : (tcol & 1) ? TW + 1 : tcol >> 1;
#pragma unroll
    for (int r = 0; r < ZR; ++r) {
      const int pix = (wr * RW * SS + r) * WP + l32 + col;
      zf[r] = __builtin_bit_cast(bf16x8_t, zb[pix * PZ + (q ^ swz<PZ>(pix))]);
    }
  };
  auto read_w = [&](const uint4* wb, int step, bf16x8_t* wf) {
    const int s = (step % 3) * 3 + step / 3;
#pragma unroll
    for (int c = 0; c < CW; ++c) wf[c] = __builtin_bit_cast(bf16x8_t, wb[g * WT::PLANE + (c * 32 + l32) * S + s]);
  };
  // issue(k) is called once for k = 0..NL-1, spread over the first ISS steps
  // A wave whose rows all lie below the image (the last patch row of a map
  // whose height is not a multiple of TH) only issues its share of the loads.
  auto compute = [&](const uint4* zb, const uint4* wb, bool rows_in, auto J, auto NLc, auto ISSc, auto&& issue) {
    constexpr int NL = decltype(NLc)::value, ISS = decltype(ISSc)::value;
    if (!rows_in) {
#pragma unroll
      for (int k = 0; k < NL; ++k) issue(k);
      return;
    }
    bf16x8_t zf[2][ZR], wf[2][CW];
    read_z(zb, 0, J, zf[0]);
    read_w(wb, 0, wf[0]);
#pragma unroll
    for (int i = 0; i < NSTEP; ++i) {
      if (i + 1 < NSTEP) {
        read_w(wb, i + 1, wf[(i + 1) & 1]);
        if ((i + 1) % 3 == 0) read_z(zb, (i + 1) / 3, J, zf[((i + 1) / 3) & 1]);
      }
      __builtin_amdgcn_sched_barrier(0);
      const int ta = i % 3, zsel = (i / 3) & 1;
#pragma unroll
      for (int c = 0; c < CW; ++c)
#pragma unroll
        for (int r = 0; r < RW; ++r)
          acc[c][r] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[i & 1][c], zf[zsel][SS * r + ta * DD], acc[c][r], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int k = 0; k < NL; ++k)
        if (k * ISS / NL == i) issue(k);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Epilogue: bias added once in fp32 (all of this lane's bias values are
  // read before the first staging write), round to nearest even, staged per
  // wave through an idle weight buffer (waves 0-3) or the idle halo
  // buffer (waves 4-7) so global stores are whole 16-byte runs of channels.
  // C_out is a multiple of BN here: every channel of the tile exists, and
  // only the pixel column is range-checked.
  constexpr int EPIX = CW * 4;
  constexpr int EIT = (32 * EPIX + 63) / 64;
  auto epilogue = [&](const Tile& c, int par, int hidle, int widle) {
    unsigned char* eb = wave < 4 ? reinterpret_cast<unsigned char*>(wl + widle * WSLOTS) + wave * 32 * EROW
                                 : reinterpret_cast<unsigned char*>(zl + hidle * ZSLOTS) + (wave - 4) * 32 * EROW;
    float4 bias[CW][4];
#pragma unroll
    for (int q = 0; q < CW; ++q)
#pragma unroll
      for (int v4 = 0; v4 < 4; ++v4)
        bias[q][v4] = *reinterpret_cast<const float4*>(&bias_lds[par][q * 32 + v4 * 8 + g * 4]);
#pragma unroll
    for (int r = 0; r < RW; ++r) {
      const int y = c.y0 + wr * RW + r;
      if (y >= a.ho) continue;
#pragma unroll
      for (int q = 0; q < CW; ++q) {
#pragma unroll
        for (int v4 = 0; v4 < 4; ++v4) {
          const float4 bv = bias[q][v4];
          const f32x16_t& v = acc[q][r];
          uint2 pk;
          pk.x = pack_bf16x2(v[v4 * 4 + 0] + bv.x, v[v4 * 4 + 1] + bv.y);
          pk.y = pack_bf16x2(v[v4 * 4 + 2] + bv.z, v[v4 * 4 + 3] + bv.w);
          *reinterpret_cast<uint2*>(eb + l32 * EROW + (q * 32 + v4 * 8 + g * 4) * 2) = pk;
        }
      }
      unsigned short* orow = os + ((int64_t(c.nn) * a.to + c.o) * a.ho + y) * int64_t(a.wo) * a.cout + c.n0;
#pragma unroll
      for (int it = 0; it < EIT; ++it) {
        const int piece = it * 64 + lane;
        if (piece < 32 * EPIX) {
          const int px = piece / EPIX, ch = (piece % EPIX) * 8;
          const int xo = c.x0 + px;
          const uint4 v = *reinterpret_cast<const uint4*>(eb + px * EROW + ch * 2);
          // streaming store: the output is not read again by this kernel
          if (xo < a.wo)
            __builtin_nontemporal_store(__builtin_bit_cast(u32x4_t, v),
                                        reinterpret_cast<u32x4_t*>(orow + int64_t(xo) * a.cout + ch));
        }
      }
    }
  };
  auto bias_value = [&](const Tile& c) {
    return (a.has_bias && tid < BN && c.n0 + tid < a.cout) ? bs[c.n0 + tid] : (unsigned short)0;
  };

  // Load cursor: the group after the one being computed; it moves on at the
  // end of each group, after the barrier that publishes a claimed tile.  Its
  // tile is the current one or the next (tnext); the tile after that is the
  // one claimed during the current tile's first group (tnn), which a tile of
  // a single group already needs.  zoff holds the halo offsets of its tile.
  Grp nx{ctile, 0, 0};
  Tile nt{};
  bool nx_ok = ctile >= 0;
  if (nx_ok) {
    nt = decode(ctile);
    halo_offsets(nt);
  }
  auto nx_advance = [&]() {
    if (++nx.ti == nt.nact) {
      nx.ti = 0;
      if (++nx.gz == ngrp) {
        nx.gz = 0;
        nx.t = nx.t == ctile ? tnext : tnn;
        if (nx.t < 0) {
          nx_ok = false;
          return;
        }
        nt = decode(nx.t);
        halo_offsets(nt);
      }
    }
  };

  auto wait_halo_in_flight = [&]() {  // all but this wave's halo loads of the last group
    switch (wave) {
      case 0: asm volatile("s_waitcnt vmcnt(%0)" ::"n"(zcnt(0)) : "memory"); break;
      case 1: asm volatile("s_waitcnt vmcnt(%0)" ::"n"(zcnt(1)) : "memory"); break;
      case 2: asm volatile("s_waitcnt vmcnt(%0)" ::"n"(zcnt(2)) : "memory"); break;
      case 3: asm volatile("s_waitcnt vmcnt(%0)" ::"n"(zcnt(3)) : "memory"); break;
      case 4: asm volatile("s_waitcnt vmcnt(%0)" ::"n"(zcnt(4 % NW)) : "memory"); break;
      case 5: asm volatile("s_waitcnt vmcnt(%0)" ::"n"(zcnt(5 % NW)) : "memory"); break;
      case 6: asm volatile("s_waitcnt vmcnt(%0)" ::"n"(zcnt(6 % NW)) : "memory"); break;
      default: asm volatile("s_waitcnt vmcnt(%0)" ::"n"(zcnt(7 % NW)) : "memory"); break;
    }
  };

  // Wait for every vector memory operation.  The inline-asm waits are
  // invisible to the compiler's own wait-count tracking; the builtin after
  // it tells the compiler they have completed, so it does not drain loads
  // again where it reuses the register of an earlier load or atomic.
  auto vm_drain = [&]() {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xF70);  // vmcnt(0), other counters unconstrained
  };

  // Workgroup barrier with explicit waits only: the caller has waited for
  // the loads that must have landed; this waits for the wave's own LDS
  // accesses.  (__syncthreads() would also drain every load in flight,
  // including the next group's halo.)
  auto barrier = [&]() {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };

  if constexpr (KSP == 2) {
    // prologue: the first group's halo and both weight halves (group buffer 0)
    int wcur = 0;  // weight group buffer of the current group: halves 2*wcur, 2*wcur+1
    if (nx_ok) {
      const unsigned short* fp = halo_src(nt, nx.ti, nx.gz);
      const unsigned char* w0p = wsrc(nt, nx.ti, nx.gz * 2);
      const unsigned char* w1p = wsrc(nt, nx.ti, nx.gz * 2 + 1);
#pragma unroll
      for (int it = 0; it < ZIT; ++it) issue_z(fp, 0, it);
#pragma unroll
      for (int it = 0; it < WIT; ++it) issue_w(w0p, 0, it);
#pragma unroll
      for (int it = 0; it < WIT; ++it) issue_w(w1p, 1, it);
      nx_advance();
      vm_drain();
      barrier();
    }
    int hpar = 0, par = 0;
    if (ctile >= 0) {
      Tile ct = decode(ctile);
      for (;;) {
        zero_acc();
        const bool claims = tnext >= 0;
        const int ngt = ct.nact * ngrp;
        const bool rows_in = ct.y0 + wr * RW < a.ho;  // wave-uniform
        for (int gi = 0; gi < ngt; ++gi) {
          const uint4* zb = zl + hpar * ZSLOTS;
          unsigned short bval = 0;
          if (gi == 0) bval = bias_value(ct);
          const bool more = nx_ok;
          // in the first group thread 0 claims a tile (published at the barrier)
          const int cx = (xcd + steal) & 7;
          int v = 0;
          if (gi == 0 && claims && tid == 0) v = claim(cx);
          {
            // load the next group's weight halves and halo into the free buffers
            const unsigned char* wn0 = more ? wsrc(nt, nx.ti, nx.gz * 2) : wpk;
            const unsigned char* wn1 = more ? wsrc(nt, nx.ti, nx.gz * 2 + 1) : wpk;
            const unsigned short* fpn = more ? halo_src(nt, nx.ti, nx.gz) : xs;
            const int hn = __builtin_amdgcn_readfirstlane(hpar ^ 1);
            const int wn = __builtin_amdgcn_readfirstlane((wcur ^ 1) * 2);
            compute(zb, wl + (wcur * 2 + wj) * WSLOTS, rows_in, wj, std::integral_constant<int, 2 * WIT + ZIT>{},
                    std::integral_constant<int, NSTEP>{}, [&](int k) {
                      if (!more) return;
                      if (k < WIT) issue_w(wn0, wn, k);
                      else if (k < 2 * WIT) issue_w(wn1, wn + 1, k - WIT);
                      else issue_z(fpn, hn, k - 2 * WIT);
                    });
          }
          asm volatile("" ::: "memory");  // the claim is read only after the group
          if (gi == 0 && claims && tid == 0) {
            int t = claimed(cx, v);
            while (t < 0 && steal < 7) {
              ++steal;
              const int x = (xcd + steal) & 7;
              t = claimed(x, claim(x));
            }
            claim_lds = t;
          }
          if (gi == 0 && tid < BN) bias_lds[par][tid] = bf16_to_f32(bval);
          vm_drain();
          barrier();
          if (gi == 0 && claims) tnn = __builtin_amdgcn_readfirstlane(claim_lds);
          if (more) nx_advance();
          hpar ^= 1;
          wcur ^= 1;
        }
        // the second half's sums join the first's through the idle halo buffer
        float* red = reinterpret_cast<float*>(zl + (hpar ^ 1) * ZSLOTS);
        if (wj == 1) {
#pragma unroll
          for (int c = 0; c < CW; ++c)
#pragma unroll
            for (int r = 0; r < RW; ++r)
#pragma unroll
              for (int e = 0; e < 16; ++e) red[(((wr * CW + c) * RW + r) * 16 + e) * 64 + lane] = acc[c][r][e];
        }
        barrier();
        if (wj == 0) {
#pragma unroll
          for (int c = 0; c < CW; ++c)
#pragma unroll
            for (int r = 0; r < RW; ++r)
#pragma unroll
              for (int e = 0; e < 16; ++e) acc[c][r][e] += red[(((wr * CW + c) * RW + r) * 16 + e) * 64 + lane];
          // (the output stores may stay in flight across the barrier below)
          epilogue(ct, par, hpar ^ 1, (wcur ^ 1) * 2);
        }
        barrier();
        par ^= 1;
        ctile = tnext;
        tnext = tnn;
        tnn = -1;
        if (ctile < 0) break;
        ct = decode(ctile);
      }
    }
  } else {
    // prologue: the first group's halo and first weight sub-stage
    int hpar = 0;
    if (nx_ok) {
      const unsigned short* fp = halo_src(nt, nx.ti, nx.gz);
      const unsigned char* wp = wsrc(nt, nx.ti, nx.gz * 2);
#pragma unroll
      for (int it = 0; it < ZIT; ++it) issue_z(fp, 0, it);
#pragma unroll
      for (int it = 0; it < WIT; ++it) issue_w(wp, 0, it);
      nx_advance();
      vm_drain();
      barrier();
    }

    int par = 0;
    if (ctile >= 0) {
      Tile ct = decode(ctile);
      for (;;) {
        zero_acc();
        const bool claims = tnext >= 0;  // claim the tile after tnext while this one runs
        const int ngt = ct.nact * ngrp;  // >= 1: only frames with an active tap have tiles
        const bool rows_in = ct.y0 + wr * RW < a.ho;  // wave-uniform
        for (int gi = 0; gi < ngt; ++gi) {
          // group-major order: the active taps of one 32-channel group run back
          // to back, so a source frame's group is reused by the output frames of
          // the neighbouring tiles within a few groups, while it is still in L2
          const int gz = gi / ct.nact, ti = gi - gz * ct.nact;
          const uint4* zb = zl + hpar * ZSLOTS;
          unsigned short bval = 0;
          if (gi == 0) bval = bias_value(ct);
          const bool more = nx_ok;
          // sub-stage 0: load W[1] <- (this group, second half), H[next] <- next group
          {
            const unsigned char* wp1 = wsrc(ct, ti, gz * 2 + 1);
            const unsigned short* fpn = more ? halo_src(nt, nx.ti, nx.gz) : xs;
            const int hn = __builtin_amdgcn_readfirstlane(hpar ^ 1);
            compute(zb, wl, rows_in, std::integral_constant<int, 0>{}, std::integral_constant<int, WIT + ZIT>{},
                    std::integral_constant<int, NSTEP>{}, [&](int k) {
                      if (k < WIT) issue_w(wp1, 1, k);
                      else if (more) issue_z(fpn, hn, k - WIT);
                    });
          }
          if (more) wait_halo_in_flight();
          else vm_drain();
          if (gi == 0 && tid < BN) bias_lds[par][tid] = bf16_to_f32(bval);
          barrier();
          // sub-stage 1: load W[0] <- next group, first half.  In the first
          // group, thread 0 also claims a tile (the atomic's latency hides
          // behind the sub-stage; the claim is published at its barrier).
          const int cx = (xcd + steal) & 7;
          int v = 0;
          if (gi == 0 && claims && tid == 0) v = claim(cx);
          {
            const unsigned char* wpn = more ? wsrc(nt, nx.ti, nx.gz * 2) : wpk;
            compute(zb, wl + WSLOTS, rows_in, std::integral_constant<int, 1>{}, std::integral_constant<int, WIT>{},
                    std::integral_constant<int, (NSTEP + 1) / 2>{}, [&](int k) {
                      if (more) issue_w(wpn, 0, k);
                    });
          }
          asm volatile("" ::: "memory");  // the claim is read only after the sub-stage
          if (gi == 0 && claims && tid == 0) {
            int t = claimed(cx, v);
            while (t < 0 && steal < 7) {
              ++steal;
              const int x = (xcd + steal) & 7;
              t = claimed(x, claim(x));
            }
            claim_lds = t;
          }
          vm_drain();
          barrier();
          if (gi == 0 && claims) tnn = __builtin_amdgcn_readfirstlane(claim_lds);
          if (more) nx_advance();
          hpar ^= 1;
        }
        // (the output stores may stay in flight across this barrier)
        epilogue(ct, par, hpar ^ 1, 1);
        barrier();
        par ^= 1;
        ctile = tnext;
        tnext = tnn;
        tnn = -1;
        if (ctile < 0) break;
        ct = decode(ctile);
      }
    }
  }

  // Output frames without an active tap hold the bias: every workgroup
  // writes a strided share of them (C_out % 8 == 0: 16-byte runs).
  {
    const int64_t fpx = int64_t(a.ho) * a.wo;
    const int cpp = a.cout >> 3;
#pragma unroll 1
    for (int i = 0; i < a.nina_iv; ++i) {
      const int64_t per_n = int64_t(a.ina_n[i]) * fpx * cpp;
      for (int64_t e = int64_t(blockIdx.x) * NT + tid; e < per_n * a.n; e += int64_t(gridDim.x) * NT) {
        const int nn = int(e / per_n);
        const int64_t r = e - nn * per_n;
        const int cc = int(r % cpp);
        unsigned short v8[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) v8[q] = a.has_bias ? bs[cc * 8 + q] : (unsigned short)0;
        uint4 val;
        __builtin_memcpy(&val, v8, 16);
        *reinterpret_cast<uint4*>(os + ((int64_t(nn) * a.to + a.ina_lo[i]) * fpx + r / cpp) * a.cout + cc * 8) = val;
      }
    }
  }

  // The last workgroup to finish clears the counters for the next launch
  // that uses them (its claims and every other workgroup's are done: each
  // workgroup counts itself after its last claim).
  if (tid == 0) {
    const int done = __hip_atomic_fetch_add(a.sched + 8, 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    if (done == int(gridDim.x) - 1)
      for (int x = 0; x < 9; ++x) __hip_atomic_store(a.sched + x, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
#endif
}

// Calls f(std::integral_constant<int, i>) for i = I, I+1, .. N-1, unrolled,
// while f returns true (each call nested in the previous one's branch).
template <int I, int N, typename F>
__device__ __forceinline__ void static_for_while(F&& f) {
  if constexpr (I < N) {
    if (f(std::integral_constant<int, I>{})) static_for_while<I + 1, N>(f);
  }
}

// bf16 kernel for few output channels (C_out <= 5; the decoder's RGB head):
// 3x3 spatial taps, k_t = 3, unit temporal dilation, C_in = 32 * NCH.
//
// With three output channels a GEMM tile over output channels is almost all
// padding, and the work is bound by reading the input once.  One
// v_mfma_f32_16x16x32_bf16 multiplies 16 pixels x 32 channels of source frame
// z by a 32 x 16 weight block whose 16 columns are (temporal tap k, output
// channel co) pairs, so a single pass over frame z produces its contributions
// to the three output frames o = z + p_l - k.  The accumulator column for tap
// slot k holds output frame z + p_l - k: after frame z the slot-2 columns hold
// a finished output frame, which is written (bias added once, rounded to
// nearest even), and a lane shift by C_out within each 16-lane row (DPP
// row_shr) moves slot k to slot k+1 for the next frame.  Weights stay in
// registers for the whole kernel.
//
// Each workgroup owns a patch of a.tile_h (<= 16) output rows by 128 columns
// (eight waves of 16 columns each) and walks the source frames of Z = [C; X]
// in time order.  A stage is one halo row of one frame: 130 pixels with all
// C_in channels, a single contiguous run of the channels-last input, copied
// to LDS in memory order (so every load instruction reads 1 KB of
// consecutive bytes, and each cache line is used whole by one stage).  Halo
// row hr feeds output rows hr - kh for the three row taps kh; the
// accumulators of every output row of the patch stay in registers while the
// frame's halo rows stream through.
template <int COUT, int NCH, bool CO>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void conv_bf16_few(ConvArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int TW = 128, WP = TW + 2;       // output columns, halo columns
  constexpr int PP = 4 * NCH;                // 16-byte pieces per pixel
  constexpr int THMAX = 16;                  // accumulator rows
  constexpr int ZSLOTS = (WP * PP + 63) / 64 * 64;
  constexpr int NT = 512, ZIT = (ZSLOTS + NT - 1) / NT;
  static_assert(3 * COUT <= 16 && NCH >= 1 && NCH <= 3, "few-channel kernel shape");
  // A ring of halo-row buffers, as many as LDS holds (up to eight): all but
  // one in flight while one is multiplied.
  constexpr int NBUF = std::min(8, int(160 * 1024 / (ZSLOTS * 16)));
  static_assert(NBUF >= 4 && NBUF * ZSLOTS * 16 <= 160 * 1024, "LDS budget");
  __shared__ uint4 zl[NBUF * ZSLOTS];
  constexpr auto zcnt = [](int w) {  // halo load instructions of wave w per stage
    int n = 0;
    for (int it = 0; it < ZIT; ++it) n += it * NT + w * 64 < ZSLOTS;
    return n;
  };
  constexpr int NCO = CO ? NCH : 0;  // cache-out stores per wave and stage
  static_assert((NBUF - 2) * (zcnt(0) + NCO) <= 63, "vmcnt range");
  static_assert(zcnt(1) == zcnt(7), "waves 1-7 issue alike");

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int m = lane & 15, q = lane >> 4;   // A operand: pixel m, 8-channel piece q; D: column m
  const int th = a.tile_h, hrows = th + 2;  // output rows per patch, halo rows per frame

  // persistent schedule over patches, one contiguous range per XCD
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int nblk_here = (int(gridDim.x) >> 3) + (xcd < int(gridDim.x & 7) ? 1 : 0);
  const int tq = a.ntiles >> 3, tr = a.ntiles & 7;
  const int t_begin = xcd * tq + min(xcd, tr);
  const int t_end = t_begin + tq + (xcd < tr ? 1 : 0);
  int ctile = t_begin + slot;
  if (ctile >= t_end) return;
  auto next_tile = [&](int t) { return t + nblk_here < t_end ? t + nblk_here : -1; };

  const int64_t frame_el = int64_t(a.h) * a.wd * a.cin;
  const int row_el = a.wd * a.cin, row_bytes = row_el * 2;
  const unsigned short* __restrict__ xs = static_cast<const unsigned short*>(a.x);
  const unsigned short* __restrict__ cs = static_cast<const unsigned short*>(a.cache);
  const int p_l = -a.delta[0];              // delta_0 = -p_l
  const int z_lo = max(0, -p_l);            // first source frame any output reads

  // weights: B fragments [chunk][spatial tap], prepacked by the launcher
  bf16x8_t wreg[NCH][9];
  {
    const uint4* wp = static_cast<const uint4*>(a.wpk);
#pragma unroll
    for (int ch = 0; ch < NCH; ++ch)
#pragma unroll
      for (int s = 0; s < 9; ++s) wreg[ch][s] = __builtin_bit_cast(bf16x8_t, wp[(ch * 9 + s) * 64 + lane]);
  }
  // bias of the output channel this lane emits (lanes of tap slot 2)
  const int emit_co = m - 2 * COUT;
  const bool emits = emit_co >= 0 && emit_co < COUT;
  const float bias = (a.has_bias && emits) ? bf16_to_f32(static_cast<const unsigned short*>(a.b)[emit_co]) : 0.f;

  auto uniform = [](const void* p) {
    const uint64_t v = reinterpret_cast<uint64_t>(p);
    const uint64_t lo = uint32_t(__builtin_amdgcn_readfirstlane(int(uint32_t(v))));
    const uint64_t hi = uint32_t(__builtin_amdgcn_readfirstlane(int(uint32_t(v >> 32))));
    return reinterpret_cast<const void*>((hi << 32) | lo);
  };
  struct Patch {
    int nn, x0, y0;
  };
  auto decode = [&](int t) {
    Patch p;
    p.x0 = (t % a.tiles_x) * TW;
    t /= a.tiles_x;
    p.y0 = (t % a.tiles_y) * th;
    p.nn = t / a.tiles_y;
    return p;
  };
  // LDS slot of (halo pixel px, piece j) in a halo-row buffer: memory order,
  // with the 8-channel piece within each 32-channel chunk XOR-swizzled by
  // pixel so that 16 consecutive pixels at one piece hit 16 distinct 16-byte
  // bank groups (a pixel is PP slots, a multiple of 4).
  constexpr int OOB = int(0x80000000u);
  int zoff[ZIT];
  auto halo_offsets = [&](const Patch& c) {
#pragma unroll
    for (int it = 0; it < ZIT; ++it) {
      const int s = tid + NT * it;
      int off = OOB;
      if (s < WP * PP) {
        const int px = s / PP, j = s % PP;
        const int x = c.x0 - 1 + px;
        if (x >= 0 && x < a.wd) off = (x * a.cin + ((j & ~3) | ((j & 3) ^ swz<4>(px))) * 8) * 2;
      }
      zoff[it] = off;
    }
  };
  auto frame_ptr = [&](const Patch& c, int z) {
    return static_cast<const unsigned short*>(uniform(z < a.tc ? cs + (int64_t(c.nn) * a.tc + z) * frame_el
                                                               : xs + (int64_t(c.nn) * a.tx + (z - a.tc)) * frame_el));
  };
  // halo row y of the frame at fp into buffer buf
  auto issue_stage = [&](const unsigned short* fp, int y, int buf) {
    const bool yin = y >= 0 && y < a.h;
    // a halo row outside the map reads as zeros: an empty buffer range
    const __amdgpu_buffer_rsrc_t r =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(uniform(fp + (yin ? y : 0) * row_el)), 0,
                                          __builtin_amdgcn_readfirstlane(yin ? row_bytes : 0), 0x00020000);
#pragma unroll
    for (int it = 0; it < ZIT; ++it)
      if (ZSLOTS % NT == 0 || it * NT + wave * 64 < ZSLOTS)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            r, (__attribute__((address_space(3))) void*)(zl + buf * ZSLOTS + it * NT + wave * 64), 16, zoff[it], 0, 0, 0);
  };
  auto barrier = [&]() {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };

  f32x4_t acc[THMAX];
  // the A operand of column tap c for this lane: halo pixel wave*16 + m + c,
  // piece q of a chunk (plus 4 * chunk slots)
  int lane_slot[3];
#pragma unroll
  for (int c = 0; c < 3; ++c) {
    const int px = wave * 16 + m + c;
    lane_slot[c] = px * PP + (q ^ swz<4>(px));
  }
  // one stage: halo row HR of a frame, every chunk and column tap, into
  // output rows HR - kh.  Rows at or past the patch height (which only the
  // last two halo rows reach) collect values that are never written.
  auto compute = [&](const uint4* zb, auto hr_c) {
    constexpr int HR = decltype(hr_c)::value;
    bf16x8_t af[2][3];
#pragma unroll
    for (int c = 0; c < 3; ++c) af[0][c] = __builtin_bit_cast(bf16x8_t, zb[lane_slot[c]]);
#pragma unroll
    for (int ch = 0; ch < NCH; ++ch) {
      if (ch + 1 < NCH)
#pragma unroll
        for (int c = 0; c < 3; ++c) af[(ch + 1) & 1][c] = __builtin_bit_cast(bf16x8_t, zb[lane_slot[c] + (ch + 1) * 4]);
#pragma unroll
      for (int c = 0; c < 3; ++c)
#pragma unroll
        for (int kh = 0; kh < 3; ++kh)
          if (HR - kh >= 0 && HR - kh < THMAX)
            acc[HR - kh] =
                __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[ch & 1][c], wreg[ch][kh * 3 + c], acc[HR - kh], 0, 0, 0);
    }
  };
  // Write output frame o from the tap-slot-2 columns (bias added once) with
  // 16-bit buffer stores: a per-lane byte offset within the output row (out
  // of range for lanes that hold no output), the row offset in a scalar.
  //
  // With out_u8 the frame is written as 8-bit pixel codes (one byte per
  // channel, same layout): the step after the head, on the device, before
  // any copy to the host.  The code is decided in fp32 from the unrounded
  // sum: trunc(clamp(fma(y, scale, offset) * 255, 0, 255)).
  const int esz = a.out_u8 ? 1 : 2;  // bytes per output element
  int eoff[4];
  auto emit_offsets = [&](const Patch& c) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int x = c.x0 + wave * 16 + q * 4 + v;
      eoff[v] = (emits && x < a.wo) ? (x * COUT + emit_co) * esz : OOB;
    }
  };
  // Cache-out rows.  The last frames of Z (from a.co_lo on) are also the
  // carry to the next call.  Each stage of such a frame whose halo row is
  // one of the patch's own rows writes that row's 128 interior pixels from
  // LDS to cache_out, in memory order, so the carried frames are not read
  // from HBM a second time.  In the instantiation that writes the cache-out
  // (CO) every stage issues NCH 16-byte stores per wave (out of range where
  // there is nothing to write), which keeps the wait counts fixed; the other
  // issues none.
  int cslot[NCH], coff[NCH];
#pragma unroll
  for (int it = 0; it < NCH; ++it) {
    const int s = it * NT + tid, px = s / PP, jm = s % PP;  // piece jm of pixel x0 + px
    cslot[it] = (px + 1) * PP + ((jm & ~3) | ((jm & 3) ^ swz<4>(px + 1)));
  }
  auto co_offsets = [&](const Patch& c) {
#pragma unroll
    for (int it = 0; it < NCH; ++it) {
      const int s = it * NT + tid, px = s / PP, jm = s % PP;
      const int x = c.x0 + px;
      coff[it] = x < a.wd ? (x * a.cin + jm * 8) * 2 : OOB;
    }
  };
  const int nco = a.tz - a.co_lo;  // frames carried
  // cof: the cache-out frame of the frame being multiplied (or null), own:
  // the patch's rows inside the map; halo row hr is output row hr - 1
  auto store_cache = [&](const unsigned short* cof, int own, int y0, int hr, const uint4* zb) {
    if constexpr (!CO) return;
    // (fresh copies of own and y0 per stage: the comparisons and row
    // offsets of loop-invariant values for each unrolled row would be
    // hoisted, and held in scalar registers, which then spill)
    int own_now, y0_now;
    asm volatile("s_mov_b32 %0, %1" : "=s"(own_now) : "s"(own));
    asm volatile("s_mov_b32 %0, %1" : "=s"(y0_now) : "s"(y0));
    const bool act = cof != nullptr && unsigned(hr - 1) < unsigned(own_now);  // uniform
    const unsigned short* rp = act ? cof + (y0_now + hr - 1) * int64_t(row_el) : xs;
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<void*>(uniform(rp)), 0, __builtin_amdgcn_readfirstlane(act ? row_bytes : 0), 0x00020000);
#pragma unroll
    for (int it = 0; it < NCH; ++it) {
      uint4 v = make_uint4(0, 0, 0, 0);
      if (act) v = zb[cslot[it]];
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, v), r, coff[it], 0, 0);
    }
  };
  const int frame_out_bytes = a.ho * a.wo * COUT * esz;
  auto emit = [&](const Patch& c, int o) {
    if (o < 0 || o >= a.to) return;  // uniform
    unsigned char* of = static_cast<unsigned char*>(a.out) + ((int64_t(c.nn) * a.to + o) * a.ho * int64_t(a.wo) * COUT) * esz;
    const __amdgpu_buffer_rsrc_t r_out = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<void*>(uniform(of)), 0, __builtin_amdgcn_readfirstlane(frame_out_bytes), 0x00020000);
    const int rows = __builtin_amdgcn_readfirstlane(min(th, a.ho - c.y0));
    const int y0 = __builtin_amdgcn_readfirstlane(c.y0);
    if (a.out_u8) {  // uniform
#pragma unroll
      for (int r = 0; r < THMAX; ++r) {
        if (r < rows) {  // uniform (a loop exit here would index acc at run time)
          const int y = y0 + r;
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const float p = __builtin_fmaf(acc[r][v] + bias, a.px_scale, a.px_offset) * 255.f;
            const unsigned code = unsigned(fminf(fmaxf(p, 0.f), 255.f));  // truncates
            __builtin_amdgcn_raw_buffer_store_b8((unsigned char)code, r_out, eoff[v], y * a.wo * COUT, 0);
          }
        }
      }
      return;
    }
#pragma unroll
    for (int r = 0; r < THMAX; ++r) {
      if (r < rows) {  // uniform
        const int y = y0 + r;
#pragma unroll
        for (int v = 0; v < 4; ++v)
          __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16(acc[r][v] + bias), r_out, eoff[v], y * a.wo * COUT * 2, 0);
      }
    }
  };
  auto rotate = [&]() {  // tap slot k -> k+1 (columns are lanes within 16-lane rows)
#pragma unroll
    for (int r = 0; r < THMAX; ++r)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        // (a vector element is copied to a scalar first: bit-casting the
        // element expression itself does not read that element)
        const float cur = acc[r][v];
        acc[r][v] = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(cur), 0x110 | COUT, 0xF, 0xF, true));
      }
  };

  // Load cursor: the next stage to issue, NBUF - 1 stages ahead of the one
  // multiplied, across patch boundaries.  Stage i goes to buffer i % NBUF.
  int ltile = ctile, lz = z_lo, ly = 0;  // ly: halo row, 0 .. hrows - 1
  Patch lp = decode(ltile);
  halo_offsets(lp);
  const unsigned short* lfp = frame_ptr(lp, lz);
  int issued = 0, ibuf = 0;  // stages issued, and the next one's buffer
  auto issue_next = [&]() {
    issue_stage(lfp, lp.y0 - 1 + ly, ibuf);
    ++issued;
    ibuf = ibuf + 1 == NBUF ? 0 : ibuf + 1;
    if (++ly == hrows) {
      ly = 0;
      if (++lz == a.tz) {
        lz = z_lo;
        ltile = next_tile(ltile);
        if (ltile >= 0) {
          lp = decode(ltile);
          halo_offsets(lp);
        }
      }
      if (ltile >= 0) lfp = frame_ptr(lp, lz);
    }
  };
  // Wait for stage pos.  Each stage's loads are issued right after its NCO
  // cache-out stores, so with NBUF - 2 later stages in flight all but their
  // loads and stores must be done (memory operations complete in order; the
  // output stores at frame ends only add to the count).
  auto wait_stage = [&](int ahead) {
    if (ahead < NBUF - 2) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      return;
    }
    if (wave == 0) asm volatile("s_waitcnt vmcnt(%0)" ::"n"((NBUF - 2) * (zcnt(0) + NCO)) : "memory");
    else asm volatile("s_waitcnt vmcnt(%0)" ::"n"((NBUF - 2) * (zcnt(1) + NCO)) : "memory");
  };
  Patch cp = decode(ctile);
  emit_offsets(cp);
  co_offsets(cp);
  // the stores ahead of the first loads write nothing
  for (int i = 0; i < NBUF - 1 && ltile >= 0; ++i) {
    store_cache(nullptr, 0, 0, 0, zl);
    issue_next();
  }
  int pos = 0, cbuf = 0;  // stage multiplied next, and its buffer
  for (;;) {
#pragma unroll
    for (int r = 0; r < THMAX; ++r) acc[r] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    // output frames no tap reaches (p_l > 2) are the bias alone
    for (int o = 0; o < min(a.to, p_l - 2); ++o) emit(cp, o);
    const int own = __builtin_amdgcn_readfirstlane(min(th, a.h - cp.y0));
    for (int zi = 0; zi < a.tz - z_lo; ++zi) {
      const int z = z_lo + zi;
      const unsigned short* cof =
          z >= a.co_lo ? static_cast<const unsigned short*>(uniform(static_cast<const unsigned short*>(a.cache_out) +
                                                                    (int64_t(cp.nn) * nco + (z - a.co_lo)) * frame_el))
                       : nullptr;
      // halo rows 0 .. hrows - 1 (uniform), nested so that each test runs
      // only where the previous row was taken
      static_for_while<0, THMAX + 2>([&](auto hr_c) {
        if (decltype(hr_c)::value >= hrows) return false;
        wait_stage(issued - pos - 1);
        barrier();  // stage pos has landed everywhere; buffer (pos - 1) % NBUF is free
        store_cache(cof, own, cp.y0, decltype(hr_c)::value, zl + cbuf * ZSLOTS);
        if (ltile >= 0) issue_next();
        compute(zl + cbuf * ZSLOTS, hr_c);
        ++pos;
        cbuf = cbuf + 1 == NBUF ? 0 : cbuf + 1;
        return true;
      });
      emit(cp, z_lo + zi + p_l - 2);
      rotate();
    }
    ctile = next_tile(ctile);
    if (ctile < 0) break;
    cp = decode(ctile);
    emit_offsets(cp);
    co_offsets(cp);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#endif
}

// bf16 kernel for any spatial kernel size, stride, dilation and padding
// (k_t <= 4, C_in % 16 == 0): an implicit GEMM over stages (active temporal
// tap, spatial tap, 32-channel chunk).  A stage gathers, for every output
// pixel of the tile, the 16-byte channel pieces of the input pixel that tap
// reads, straight into LDS (the buffer range check writes zeros for the
// padding and for channels past C_in), and the 32 x 32 weight block from the
// copy of W in the workspace ([C_out][k_t][k_h][k_w][C_in] as it is).  No
// halo is shared between spatial taps, so the input is read k_h * k_w times
// from L2: the kernel covers the shapes the halo-staged ones do not.
// Tile: 8 x 32 output pixels x BN (64 or 96) output channels; wave w owns
// rows 2w and 2w + 1 (2 x BN/32 accumulators of 32 x 32).  The gathered
// pixels dominate the staged bytes, so the wider tile stages fewer bytes per
// MFMA (470 against 640).
template <int BN>
__global__ __launch_bounds__(256) void conv_bf16_gen(ConvArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int TH = 8, TW = 32, CW = BN / 32, NT = 256, PPX = 4;  // pieces per pixel: 32 channels
  constexpr int ASL = TH * TW * PPX, BSL = BN * PPX;               // LDS slots per stage
  constexpr int BIT = (BSL + NT - 1) / NT;                         // weight load rounds
  constexpr int NB = 3;                                            // stage buffers (ring)
  static_assert(BN % 32 == 0 && BSL % 64 == 0, "tile width");
  constexpr auto bcnt = [](int w) {  // weight load instructions of wave w per stage
    int n = 0;
    for (int it = 0; it < BIT; ++it) n += it * NT + w * 64 < BSL;
    return n;
  };
  __shared__ uint4 al[NB * ASL];
  __shared__ uint4 bl[NB * BSL];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5, l32 = lane & 31;

  int t = blockIdx.x;
  const int o = t % a.to;
  t /= a.to;
  const int nb = t % a.nblk_n;
  t /= a.nblk_n;
  const int x0 = (t % a.tiles_x) * TW;
  t /= a.tiles_x;
  const int y0 = (t % a.tiles_y) * TH;
  const int nn = t / a.tiles_y;
  const int n0 = nb * BN;

  // active temporal taps of output frame o
  int ktap[kMaxTapsBf16], ztap[kMaxTapsBf16], nact = 0;
#pragma unroll
  for (int k = 0; k < kMaxTapsBf16; ++k) {
    ktap[k] = ztap[k] = 0;
    const int z = o * a.st + a.delta[k];
    if (k < a.kt && z >= 0 && z < a.tz) {
#pragma unroll
      for (int i = 0; i < kMaxTapsBf16; ++i)
        if (i == nact) {
          ktap[i] = k;
          ztap[i] = z;
        }
      ++nact;
    }
  }
  const int nchk = (a.cin + 31) / 32, nsp = a.kh * a.kw;
  const int nst = nact * nsp * nchk;
  const int64_t frame_el = int64_t(a.h) * a.wd * a.cin;
  const int frame_bytes = int(frame_el * 2);
  const int w_bytes = a.cout * a.kt * nsp * a.cin * 2;
  const unsigned short* __restrict__ xs = static_cast<const unsigned short*>(a.x);
  const unsigned short* __restrict__ cs = static_cast<const unsigned short*>(a.cache);
  unsigned short* __restrict__ os = static_cast<unsigned short*>(a.out);
  const __amdgpu_buffer_rsrc_t r_w =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(a.wpk), 0, w_bytes, 0x00020000);
  constexpr int OOB = int(0x80000000u);
  auto pick = [](const int* v, int i) {
    int r = v[0];
#pragma unroll
    for (int j = 1; j < kMaxTapsBf16; ++j)
      if (j == i) r = v[j];
    return r;
  };

  // Slot s of a stage buffer holds piece q of pixel px with s = px*4 + (q ^ (px & 3))
  // (the XOR spreads the 32 pixels one fragment read touches over the banks);
  // the direct-to-LDS load writes lane i's 16 bytes at slot base + i, so the
  // thread owning slot s loads that pixel's piece.
  auto issue = [&](int st, int buf) {
    const int cc = st % nchk, sp = (st / nchk) % nsp, ti = st / (nchk * nsp);
    const int ta = sp / a.kw, tcol = sp % a.kw;
    const int k = pick(ktap, ti), z = pick(ztap, ti);
    const unsigned short* fp =
        z < a.tc ? cs + (int64_t(nn) * a.tc + z) * frame_el : xs + (int64_t(nn) * a.tx + (z - a.tc)) * frame_el;
    const __amdgpu_buffer_rsrc_t r_z =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<unsigned short*>(fp), 0, frame_bytes, 0x00020000);
#pragma unroll
    for (int it = 0; it < ASL / NT; ++it) {
      const int sl = it * NT + tid, px = sl >> 2, q = (sl & 3) ^ (px & 3);
      const int oy = y0 + (px >> 5), ox = x0 + (px & 31);
      const int iy = oy * a.sh - a.ph + ta * a.dh, ix = ox * a.sw - a.pw + tcol * a.dw, ch = cc * 32 + q * 8;
      const bool in = oy < a.ho && ox < a.wo && iy >= 0 && iy < a.h && ix >= 0 && ix < a.wd && ch < a.cin;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          r_z, (__attribute__((address_space(3))) void*)(al + buf * ASL + it * NT + wave * 64), 16,
          in ? ((iy * a.wd + ix) * a.cin + ch) * 2 : OOB, 0, 0, 0);
    }
#pragma unroll
    for (int it = 0; it < BIT; ++it) {
      const int sl = it * NT + tid;
      if (it * NT + wave * 64 < BSL) {  // wave-uniform
        const int co = sl >> 2, q = (sl & 3) ^ (co & 3), ch = cc * 32 + q * 8;
        const bool in = n0 + co < a.cout && ch < a.cin;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            r_w, (__attribute__((address_space(3))) void*)(bl + buf * BSL + it * NT + wave * 64), 16,
            in ? ((((n0 + co) * a.kt + k) * nsp + sp) * a.cin + ch) * 2 : OOB, 0, 0, 0);
      }
    }
  };
  auto barrier = [&]() {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };

  // Ring of three stage buffers, one barrier per stage: stage st + 2 is
  // issued after the barrier of stage st, when every wave has finished
  // stage st - 1, the last reader of its buffer.
  f32x16_t acc[CW][2];
#pragma unroll
  for (int cb = 0; cb < CW; ++cb)
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[cb][r][v] = 0.f;
  if (nst > 0) issue(0, 0);
  if (nst > 1) issue(1, 1);
  for (int st = 0; st < nst; ++st) {
    const int buf = st % NB;
    // stage st has landed once only stage st + 1's loads are in flight
    if (st + 1 < nst) {
      static_assert(bcnt(0) == BIT && bcnt(3) >= BIT - 1, "two weight load counts");
      if (bcnt(wave) == BIT) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(ASL / NT + BIT) : "memory");
      else asm volatile("s_waitcnt vmcnt(%0)" ::"n"(ASL / NT + BIT - 1) : "memory");
    } else {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    barrier();
    if (st + 2 < nst) issue(st + 2, (st + 2) % NB);
    const uint4* ab = al + buf * ASL;
    const uint4* bb = bl + buf * BSL;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int q = kk * 2 + g;  // 8-channel piece of this lane's k range
      bf16x8_t wf[CW], pf[2];
#pragma unroll
      for (int cb = 0; cb < CW; ++cb) {
        const int co = cb * 32 + l32;
        wf[cb] = __builtin_bit_cast(bf16x8_t, bb[co * 4 + (q ^ (co & 3))]);
      }
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const int px = (wave * 2 + r) * 32 + l32;
        pf[r] = __builtin_bit_cast(bf16x8_t, ab[px * 4 + (q ^ (px & 3))]);
      }
#pragma unroll
      for (int cb = 0; cb < CW; ++cb)
#pragma unroll
        for (int r = 0; r < 2; ++r)
          acc[cb][r] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[cb], pf[r], acc[cb][r], 0, 0, 0);
    }
  }

  // epilogue: bias once in fp32, round to nearest even, channels-last stores
  const unsigned short* __restrict__ bs = static_cast<const unsigned short*>(a.b);
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int oy = y0 + wave * 2 + r, ox = x0 + l32;
    if (oy >= a.ho || ox >= a.wo) continue;
    unsigned short* op = os + (((int64_t(nn) * a.to + o) * a.ho + oy) * a.wo + ox) * a.cout;
#pragma unroll
    for (int cb = 0; cb < CW; ++cb)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int co = n0 + cb * 32 + (v >> 2) * 8 + g * 4 + (v & 3);
        if (co < a.cout) op[co] = f32_to_bf16(acc[cb][r][v] + (a.has_bias ? bf16_to_f32(bs[co]) : 0.f));
      }
  }
#endif
}

// Packs the weights of the few-channel kernel into its B fragments: for
// chunk ch, spatial tap s and lane l, the 8 weights of column n = l % 16
// ((tap k, channel co) = (n / C_out, n % C_out), zero past 3 C_out) and
// input channels ch*32 + (l/16)*8 + [0, 8).
template <int COUT, int NCH>
__global__ __launch_bounds__(64) void pack_weights_few(const unsigned short* __restrict__ w, uint4* __restrict__ wpk,
                                                       int cin) {
  const int ch = blockIdx.x / 9, s = blockIdx.x % 9, lane = threadIdx.x;
  const int n = lane & 15, kq = lane >> 4;
  uint4 v = make_uint4(0, 0, 0, 0);
  if (n < 3 * COUT) {
    const int k = n / COUT, co = n % COUT;
    v = *reinterpret_cast<const uint4*>(w + ((int64_t(co) * 3 + k) * 9 + s) * cin + ch * 32 + kq * 8);
  }
  wpk[(ch * 9 + s) * 64 + lane] = v;
}

// fp32 path: one output element per thread, direct loops in the order of the
// definition (taps, rows, columns, channels) with fp32 fused multiply-add.
__global__ __launch_bounds__(256) void conv_f32_direct(ConvArgs a) {
  const int64_t total = int64_t(a.n) * a.to * a.ho * a.wo * a.cout;
  const int64_t idx = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (idx >= total) return;
  int64_t r = idx;
  const int co = int(r % a.cout);
  r /= a.cout;
  const int j = int(r % a.wo);
  r /= a.wo;
  const int i = int(r % a.ho);
  r /= a.ho;
  const int o = int(r % a.to);
  const int nn = int(r / a.to);
  const float* xs = static_cast<const float*>(a.x);
  const float* cs = static_cast<const float*>(a.cache);
  const float* ws = static_cast<const float*>(a.w);
  const int64_t frame_el = int64_t(a.h) * a.wd * a.cin;
  float acc = a.has_bias ? static_cast<const float*>(a.b)[co] : 0.f;
  for (int k = 0; k < a.kt; ++k) {
    const int t = o * a.st + tap_delta(a, k);
    if (t < 0 || t >= a.tz) continue;
    const float* fp = t < a.tc ? cs + (int64_t(nn) * a.tc + t) * frame_el
                               : xs + (int64_t(nn) * a.tx + (t - a.tc)) * frame_el;
    for (int ta = 0; ta < a.kh; ++ta) {
      const int u = i * a.sh - a.ph + ta * a.dh;
      if (u < 0 || u >= a.h) continue;
      for (int tb = 0; tb < a.kw; ++tb) {
        const int v = j * a.sw - a.pw + tb * a.dw;
        if (v < 0 || v >= a.wd) continue;
        const float* zp = fp + (int64_t(u) * a.wd + v) * a.cin;
        const float* wp = ws + ((int64_t(co) * a.kt + k) * a.kh * a.kw + ta * a.kw + tb) * a.cin;
        for (int ci = 0; ci < a.cin; ++ci) acc = fmaf(zp[ci], wp[ci], acc);
      }
    }
  }
  static_cast<float*>(a.out)[idx] = acc;
}

// Cache-out writer: copies the last L frames of Z = [C; X] of every batch
// item into cache_out[n][0..L).  Frames are contiguous byte ranges.
__global__ __launch_bounds__(256) void copy_tail_frames(const unsigned char* __restrict__ x,
                                                        const unsigned char* __restrict__ cache,
                                                        unsigned char* __restrict__ dst,
                                                        int64_t frame_bytes, int n, int tx, int tc,
                                                        int L, int vec16) {
  const int tz = tx + tc;
  for (int f = blockIdx.y; f < n * L; f += gridDim.y) {
    const int nn = f / L, j = f - nn * L;
    const int zf = tz - L + j;
    const unsigned char* src = zf < tc ? cache + (int64_t(nn) * tc + zf) * frame_bytes
                                       : x + (int64_t(nn) * tx + (zf - tc)) * frame_bytes;
    unsigned char* d = dst + int64_t(f) * frame_bytes;
    const int64_t stride = int64_t(gridDim.x) * 256;
    int64_t done = 0;
    if (vec16) {
      const int64_t n16 = frame_bytes / 16;
      for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < n16; i += stride)
        reinterpret_cast<uint4*>(d)[i] = reinterpret_cast<const uint4*>(src)[i];
      done = n16 * 16;
    }
    for (int64_t i = done + int64_t(blockIdx.x) * 256 + threadIdx.x; i < frame_bytes; i += stride)
      d[i] = src[i];
  }
}

bool overlaps(const void* p, int64_t pb, const void* q, int64_t qb) {
  if (!p || !q || pb <= 0 || qb <= 0) return false;
  const auto a0 = reinterpret_cast<uintptr_t>(p), b0 = reinterpret_cast<uintptr_t>(q);
  return a0 < b0 + uint64_t(qb) && b0 < a0 + uint64_t(pb);
}

bool aligned(const void* p, uintptr_t al) { return (reinterpret_cast<uintptr_t>(p) & (al - 1)) == 0; }

cc3d_status_t invalid() {
  cc3d::g_invalid.fetch_add(1, std::memory_order_relaxed);
  return CC3D_ERR_INVALID_ARG;
}

hipError_t launch_conv(const void* kernel, const ConvArgs& a, int64_t grid, hipStream_t s, int threads = 256) {
  ConvArgs arg = a;
  void* args[] = {&arg};
  return hipLaunchKernel(kernel, dim3(unsigned(grid)), dim3(unsigned(threads)), args, 0, s);
}

// Compute units of the current device (cached per device).
int device_cus(int dev) {
  static std::atomic<int> cus[64];
  if (dev < 0 || dev >= 64) return 256;
  int v = cus[dev].load(std::memory_order_relaxed);
  if (v <= 0) {
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) v = 256;
    cus[dev].store(v, std::memory_order_relaxed);
  }
  return v;
}

// bf16 path: optionally repack the weights into the plan's workspace, then
// run the persistent conv kernel with min(tiles, compute units) workgroups,
// one per compute unit.
// Repack the weights into the stage-ordered layout of the bf16 kernels.
template <int BN, int KS, int CB>
hipError_t pack_bf16(const ConvArgs& a, hipStream_t s) {
  using T = WTile<BN, KS, CB>;
  const unsigned short* w = static_cast<const unsigned short*>(a.w);
  uint4* wpk = static_cast<uint4*>(const_cast<void*>(a.wpk));
  int cout = a.cout, kt = a.kt, cin = a.cin, nblk = a.nblk_n;
  int64_t total = int64_t(kt) * (cin / CB) * nblk * T::WSLOTS;
  const unsigned pgrid = unsigned(std::min<int64_t>((total + 255) / 256, 4096));
  void* pargs[] = {&w, &wpk, &cout, &kt, &cin, &nblk, &total};
  return hipLaunchKernel(reinterpret_cast<const void*>(&pack_weights<BN, KS, CB>), dim3(pgrid), dim3(256), pargs, 0,
                         s);
}

// Launch a persistent bf16 kernel with as many workgroups as fit on the
// device at once (the per-CU occupancy is queried once per kernel).
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

template <int BN, int TH, int WM, int WN, int KS, int CB, int NBUF, int OCC>
const void* mfma_kernel() {
  return reinterpret_cast<const void*>(&conv_bf16_mfma<BN, TH, WM, WN, KS, CB, NBUF, OCC>);
}
template <int BN, int TH, int WM, int DD, int SS, int KSP>
const void* g32_kernel() {
  return reinterpret_cast<const void*>(&conv_bf16_g32<BN, TH, WM, DD, SS, KSP>);
}
template <int COUT, int NCH, bool CO>
const void* few_kernel() {
  return reinterpret_cast<const void*>(&conv_bf16_few<COUT, NCH, CO>);
}

// The few-output-channel kernel packs its weights as register fragments.
template <int COUT, int NCH>
hipError_t launch_few(ConvArgs a, int64_t tiles, int cus, bool pack, bool conv, hipStream_t s) {
  if (pack) {
    const unsigned short* w = static_cast<const unsigned short*>(a.w);
    uint4* wpk = static_cast<uint4*>(const_cast<void*>(a.wpk));
    int cin = a.cin;
    void* pargs[] = {&w, &wpk, &cin};
    const hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&pack_weights_few<COUT, NCH>), dim3(NCH * 9),
                                         dim3(64), pargs, 0, s);
    if (e != hipSuccess) return e;
  }
  if (!conv) return hipSuccess;
  if (a.cache_out) return launch_persistent<&few_kernel<COUT, NCH, true>>(a, tiles, cus, 512, s);
  return launch_persistent<&few_kernel<COUT, NCH, false>>(a, tiles, cus, 512, s);
}
template <int COUT>
hipError_t launch_few_cin(ConvArgs a, int64_t tiles, int cus, bool pack, bool conv, hipStream_t s) {
  switch (a.cin / 32) {
    case 1: return launch_few<COUT, 1>(a, tiles, cus, pack, conv, s);
    case 2: return launch_few<COUT, 2>(a, tiles, cus, pack, conv, s);
    default: return launch_few<COUT, 3>(a, tiles, cus, pack, conv, s);
  }
}

template <int BN, int TH, int WM, int WN, int KS, int CB, int NBUF, int OCC>
hipError_t launch_bf16(ConvArgs a, int64_t tiles, int cus, bool pack, bool conv, hipStream_t s) {
  if (pack) {
    const hipError_t e = pack_bf16<BN, KS, CB>(a, s);
    if (e != hipSuccess) return e;
  }
  if (!conv) return hipSuccess;
  return launch_persistent<&mfma_kernel<BN, TH, WM, WN, KS, CB, NBUF, OCC>>(a, tiles, cus, WM * WN * 64, s);
}

// The general-spatial kernel reads W as it is, from a copy in the workspace
// (so the packed-weights path works the same way); one workgroup per tile.
template <int BN>
hipError_t launch_gen(ConvArgs a, int64_t tiles, bool pack, bool conv, hipStream_t s) {
  if (pack) {
    const size_t w_bytes = size_t(a.cout) * a.kt * a.kh * a.kw * a.cin * 2;
    const hipError_t e = hipMemcpyAsync(const_cast<void*>(a.wpk), a.w, w_bytes, hipMemcpyDeviceToDevice, s);
    if (e != hipSuccess) return e;
  }
  if (!conv) return hipSuccess;
  return launch_conv(reinterpret_cast<const void*>(&conv_bf16_gen<BN>), a, tiles, s, 256);
}

// The group-staged 3x3 kernel (16-channel weight sub-stages, same packing).
template <int BN, int TH, int WM, int DD = 1, int SS = 1, int KSP = 1>
hipError_t launch_g32(ConvArgs a, int64_t tiles, int cus, bool pack, bool conv, hipStream_t s) {
  if (pack) {
    const hipError_t e = pack_bf16<BN, 3, 16>(a, s);
    if (e != hipSuccess) return e;
  }
  if (!conv) return hipSuccess;
  return launch_persistent<&g32_kernel<BN, TH, WM, DD, SS, KSP>>(a, tiles, cus, WM * 64, s);
}

}  // namespace

namespace {

enum RunMode { kPackAndRun, kPackOnly, kRunPacked };

// The output frames with at least one active tap (the union of the taps'
// output intervals [o_lo, o_hi)) as sorted disjoint intervals, their
// complement in [0, T_o), and the number of tiles over the active frames.
bool frame_intervals(const cc3d_plan* plan, ConvArgs& a) {
  const cc3d_plan_info_t& in = plan->info;
  std::pair<int, int> iv[CC3D_MAX_KT];
  int n = 0;
  for (int k = 0; k < plan->d.k_t; ++k)
    if (in.taps[k].active) iv[n++] = {in.taps[k].o_lo, in.taps[k].o_hi};
  std::sort(iv, iv + n);
  a.nact_iv = 0;
  a.ta_n = 0;
  for (int i = 0; i < n; ++i) {
    if (a.nact_iv > 0 && iv[i].first <= a.act_lo[a.nact_iv - 1] + a.act_n[a.nact_iv - 1]) {
      const int hi = std::max(a.act_lo[a.nact_iv - 1] + a.act_n[a.nact_iv - 1], iv[i].second);
      a.act_n[a.nact_iv - 1] = hi - a.act_lo[a.nact_iv - 1];
    } else {
      if (a.nact_iv == kMaxFrameIv) return false;
      a.act_lo[a.nact_iv] = iv[i].first;
      a.act_n[a.nact_iv] = iv[i].second - iv[i].first;
      ++a.nact_iv;
    }
  }
  a.nina_iv = 0;
  int prev = 0;
  for (int i = 0; i <= a.nact_iv; ++i) {
    const int lo = i < a.nact_iv ? a.act_lo[i] : in.t_out;
    if (lo > prev) {
      a.ina_lo[a.nina_iv] = prev;
      a.ina_n[a.nina_iv] = lo - prev;
      ++a.nina_iv;
    }
    if (i < a.nact_iv) {
      prev = a.act_lo[i] + a.act_n[i];
      a.ta_n += a.act_n[i];
    }
  }
  const int64_t nat = int64_t(a.n) * a.ta_n * a.tiles_y * a.tiles_x * a.nblk_n;
  if (nat > INT32_MAX) return false;
  a.nat = int(nat);
  return true;
}

// Pixel output of the head: 8-bit codes instead of bf16 (see ConvArgs).
struct PixelOut {
  float scale, offset;
};

cc3d_status_t run_plan(cc3d_plan_t plan, const void* x, const void* cache_in, const void* w, const void* b,
                       void* out, void* cache_out, void* stream, RunMode mode, const PixelOut* px = nullptr) {
  if (!plan) return invalid();
  const cc3d_desc_t& d = plan->d;
  const cc3d_plan_info_t& in = plan->info;
  if (px && in.kernel_id != CC3D_K_BF16_S3_FEW) {
    cc3d::g_unsupported.fetch_add(1, std::memory_order_relaxed);
    return CC3D_ERR_UNSUPPORTED;
  }
  const int64_t out_bytes = px ? plan->out_bytes / plan->elem : plan->out_bytes;
  const bool bf16 = d.dtype == CC3D_BF16;
  const bool needs_w = mode != kRunPacked;
  const bool runs = mode != kPackOnly;
  if (!bf16 && mode != kPackAndRun) return invalid();
  if (d.t_cache == 0) cache_in = nullptr;
  if (!d.has_bias) b = nullptr;
  if (!needs_w) w = nullptr;
  if (!runs) {
    x = cache_in = b = nullptr;
    out = cache_out = nullptr;
  }
  if ((needs_w && !w) ||
      (runs && (!x || !out || (d.t_cache > 0 && !cache_in) || (d.has_bias && !b))))
    return invalid();
  const uintptr_t al = bf16 ? 16 : 4;
  if (!aligned(x, al) || !aligned(cache_in, al) || !aligned(w, al) || (!px && !aligned(out, al)) ||
      !aligned(cache_out, al) || !aligned(b, uintptr_t(plan->elem)))
    return invalid();
  if (overlaps(out, out_bytes, x, plan->x_bytes) || overlaps(out, out_bytes, cache_in, plan->cache_bytes) ||
      overlaps(out, out_bytes, w, plan->w_bytes) || overlaps(out, out_bytes, b, plan->b_bytes) ||
      overlaps(out, out_bytes, cache_out, plan->cache_out_bytes) ||
      overlaps(cache_out, plan->cache_out_bytes, x, plan->x_bytes) ||
      overlaps(cache_out, plan->cache_out_bytes, cache_in, plan->cache_bytes) ||
      overlaps(cache_out, plan->cache_out_bytes, w, plan->w_bytes) ||
      overlaps(cache_out, plan->cache_out_bytes, b, plan->b_bytes))
    return invalid();

  ConvArgs a{};
  a.x = x;
  a.cache = cache_in;
  a.w = w;
  a.b = b;
  a.out = out;
  a.n = d.n;
  a.tx = d.t_x;
  a.tc = d.t_cache;
  a.h = d.h;
  a.wd = d.w;
  a.cin = d.c_in;
  a.cout = d.c_out;
  a.to = in.t_out;
  a.ho = in.h_out;
  a.wo = in.w_out;
  a.kt = d.k_t;
  a.kh = d.k_h;
  a.kw = d.k_w;
  a.sh = d.s_h;
  a.sw = d.s_w;
  a.dh = d.d_h;
  a.dw = d.d_w;
  a.ph = d.p_h;
  a.pw = d.p_w;
  a.tz = in.t_z;
  for (int k = 0; k < CC3D_MAX_KT; ++k) a.delta[k] = k < d.k_t ? in.taps[k].delta : 0;
  a.st = d.s_t;
  a.tiles_x = plan->tiles_x;
  a.tiles_y = plan->tiles_y;
  a.tile_h = plan->tile_h;
  // the few-output-channel kernel writes the cache-out itself
  const bool fused_co = in.kernel_id == CC3D_K_BF16_S3_FEW && cache_out && in.t_cache_out > 0;
  a.cache_out = fused_co ? cache_out : nullptr;
  a.co_lo = fused_co ? a.tz - in.t_cache_out : a.tz;
  a.nblk_n = plan->nblk_n;
  a.ntiles = int(in.tiles);
  a.has_bias = d.has_bias;
  if (px) {
    a.out_u8 = 1;
    a.px_scale = px->scale;
    a.px_offset = px->offset;
  }
  if ((in.kernel_id == CC3D_K_BF16_S3_N96_G32W8 || in.kernel_id == CC3D_K_BF16_S3_N64_G32W8 ||
       in.kernel_id == CC3D_K_BF16_S3D2_N64_G32W8 || in.kernel_id == CC3D_K_BF16_S3S2_N96_G32W4 ||
       in.kernel_id == CC3D_K_BF16_S3S2_N64_G32W8) &&
      !frame_intervals(plan, a))
    return invalid();

  int cus = 256;
  if (bf16) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) {
      cc3d::g_device_error.fetch_add(1, std::memory_order_relaxed);
      return CC3D_ERR_DEVICE;
    }
    std::lock_guard<std::mutex> lock(plan->mu);
    if (!plan->wpk) {
      if (mode == kRunPacked) return invalid();  // nothing packed yet
      if (hipMalloc(&plan->wpk, size_t(in.workspace_bytes)) != hipSuccess) {
        plan->wpk = nullptr;
        cc3d::g_device_error.fetch_add(1, std::memory_order_relaxed);
        return CC3D_ERR_DEVICE;
      }
      // the scheduler counters start at zero (each launch leaves its slot so)
      if (hipMemset(static_cast<char*>(plan->wpk) + plan->sched_off, 0,
                    size_t(in.workspace_bytes - plan->sched_off)) != hipSuccess ||
          hipDeviceSynchronize() != hipSuccess) {
        (void)hipFree(plan->wpk);
        plan->wpk = nullptr;
        cc3d::g_device_error.fetch_add(1, std::memory_order_relaxed);
        return CC3D_ERR_DEVICE;
      }
      plan->wpk_device = dev;
    } else if (plan->wpk_device != dev) {
      return invalid();
    }
    a.wpk = plan->wpk;
    a.sched = reinterpret_cast<int*>(static_cast<char*>(plan->wpk) + plan->sched_off) +
              int64_t(plan->sched_seq.fetch_add(1, std::memory_order_relaxed) % kSchedSlots) * kSchedInts;
    cus = device_cus(dev);
  }

  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hipSuccess;
  const bool pack = mode != kRunPacked;
  switch (in.kernel_id) {
    case CC3D_K_F32_DIRECT:
      e = launch_conv(reinterpret_cast<const void*>(&conv_f32_direct), a, in.tiles, s);
      break;
    case CC3D_K_BF16_S3_N96_X2: e = launch_bf16<96, 8, 4, 1, 3, 16, 2, 2>(a, in.tiles, cus, pack, runs, s); break;
    case CC3D_K_BF16_S3_N32: e = launch_bf16<32, 8, 4, 1, 3, 16, 3, 2>(a, in.tiles, cus, pack, runs, s); break;
    case CC3D_K_BF16_S3_N96_G32W8:
      e = launch_g32<96, 16, 8>(a, std::max<int64_t>(a.nat, 1), cus, pack, runs, s);
      break;
    case CC3D_K_BF16_S3_N64_G32W8:
      e = launch_g32<64, 24, 8>(a, std::max<int64_t>(a.nat, 1), cus, pack, runs, s);
      break;
    case CC3D_K_BF16_S3D2_N64_G32W8:
      e = launch_g32<64, 16, 8, 2>(a, std::max<int64_t>(a.nat, 1), cus, pack, runs, s);
      break;
    case CC3D_K_BF16_S3S2_N96_G32W4:
      e = launch_g32<96, 4, 4, 1, 2>(a, std::max<int64_t>(a.nat, 1), cus, pack, runs, s);
      break;
    case CC3D_K_BF16_S3S2_N64_G32W8:
      e = launch_g32<64, 4, 8, 1, 2, 2>(a, std::max<int64_t>(a.nat, 1), cus, pack, runs, s);
      break;
    case CC3D_K_BF16_GEN_N64: e = launch_gen<64>(a, in.tiles, pack, runs, s); break;
    case CC3D_K_BF16_GEN_N96: e = launch_gen<96>(a, in.tiles, pack, runs, s); break;
    case CC3D_K_BF16_S3_FEW:
      switch (d.c_out) {
        case 1: e = launch_few_cin<1>(a, in.tiles, cus, pack, runs, s); break;
        case 2: e = launch_few_cin<2>(a, in.tiles, cus, pack, runs, s); break;
        case 3: e = launch_few_cin<3>(a, in.tiles, cus, pack, runs, s); break;
        case 4: e = launch_few_cin<4>(a, in.tiles, cus, pack, runs, s); break;
        default: e = launch_few_cin<5>(a, in.tiles, cus, pack, runs, s); break;
      }
      break;
    case CC3D_K_BF16_S1_N192:
      if (plan->cin_chunk == 64) e = launch_bf16<192, 8, 2, 2, 1, 64, 2, 1>(a, in.tiles, cus, pack, runs, s);
      else e = launch_bf16<192, 8, 2, 2, 1, 32, 3, 1>(a, in.tiles, cus, pack, runs, s);
      break;
    case CC3D_K_BF16_S1_N32:
      if (plan->cin_chunk == 64) e = launch_bf16<32, 8, 4, 1, 1, 64, 3, 1>(a, in.tiles, cus, pack, runs, s);
      else if (plan->cin_chunk == 32) e = launch_bf16<32, 8, 4, 1, 1, 32, 3, 2>(a, in.tiles, cus, pack, runs, s);
      else e = launch_bf16<32, 8, 4, 1, 1, 16, 3, 2>(a, in.tiles, cus, pack, runs, s);
      break;
    default:
      return invalid();
  }
  if (e == hipSuccess && runs && cache_out && in.t_cache_out > 0 && !fused_co) {
    const int64_t frame_bytes = int64_t(d.h) * d.w * d.c_in * plan->elem;
    int vec16 = (frame_bytes % 16 == 0) && aligned(x, 16) && aligned(cache_in, 16) && aligned(cache_out, 16);
    const int64_t units = vec16 ? frame_bytes / 16 : frame_bytes;
    int n = d.n, tx = d.t_x, tc = d.t_cache, L = in.t_cache_out;
    const int frames = n * L;
    const unsigned gx = unsigned(std::max<int64_t>(1, std::min<int64_t>((units + 1023) / 1024, 2048)));
    const unsigned gy = unsigned(std::min(frames, 65535));
    const unsigned char* xp = static_cast<const unsigned char*>(x);
    const unsigned char* cp = static_cast<const unsigned char*>(cache_in);
    unsigned char* dp = static_cast<unsigned char*>(cache_out);
    int64_t fb = frame_bytes;
    void* args[] = {&xp, &cp, &dp, &fb, &n, &tx, &tc, &L, &vec16};
    e = hipLaunchKernel(reinterpret_cast<const void*>(&copy_tail_frames), dim3(gx, gy), dim3(256), args, 0, s);
  }
  if (e != hipSuccess) {
    cc3d::g_device_error.fetch_add(1, std::memory_order_relaxed);
    return CC3D_ERR_DEVICE;
  }
  if (runs) cc3d::g_fast_path.fetch_add(1, std::memory_order_relaxed);
  return CC3D_OK;
}

}  // namespace

extern "C" cc3d_status_t causal_conv3d_forward(cc3d_plan_t plan, const void* x, const void* cache_in,
                                               const void* w, const void* b, void* out, void* cache_out,
                                               void* stream) {
  return run_plan(plan, x, cache_in, w, b, out, cache_out, stream, kPackAndRun);
}

extern "C" cc3d_status_t causal_conv3d_pack_weights(cc3d_plan_t plan, const void* w, void* stream) {
  return run_plan(plan, nullptr, nullptr, w, nullptr, nullptr, nullptr, stream, kPackOnly);
}

extern "C" cc3d_status_t causal_conv3d_forward_packed(cc3d_plan_t plan, const void* x, const void* cache_in,
                                                      const void* b, void* out, void* cache_out, void* stream) {
  return run_plan(plan, x, cache_in, nullptr, b, out, cache_out, stream, kRunPacked);
}

extern "C" cc3d_status_t causal_conv3d_forward_u8(cc3d_plan_t plan, const void* x, const void* cache_in,
                                                  const void* w, const void* b, void* out, void* cache_out,
                                                  float scale, float offset, void* stream) {
  if (!(scale == scale) || !(offset == offset)) return invalid();  // NaN
  const PixelOut px{scale, offset};
  return run_plan(plan, x, cache_in, w, b, out, cache_out, stream, w ? kPackAndRun : kRunPacked, &px);
}

// Per-signature variant choice: every bf16 variant that can run the call is
// timed on the caller's buffers and the fastest is kept.
extern "C" cc3d_status_t causal_conv3d_plan_autotune(const cc3d_desc_t* desc, const void* x, const void* cache_in,
                                                     const void* w, const void* b, void* out, int launches,
                                                     void* stream, cc3d_plan_t* out_plan, float* best_ms) {
  // (nullptr: the default variant, whose geometry may be none of these)
  static const char* const kCandidates[] = {nullptr,
                                            "bf16_s3_n96_p16x32_g32",
                                            "bf16_s3_n64_p24x32_g32",
                                            "bf16_s3_n96_p8x32_x2",
                                            "bf16_s3_n32_p8x32",
                                            "bf16_s3_few_p16x128",
                                            "bf16_s3_few_p12x128",
                                            "bf16_s3_few_p8x128",
                                            "bf16_s1_n192_p8x32",
                                            "bf16_s1_n32_p8x32",
                                            "bf16_s3d2_n64_p16x32_g32",
                                            "bf16_s3s2_n96_p4x32_g32",
                                            "bf16_s3s2_n64_p4x32_g32",
                                            "bf16_gen_n96_p8x32",
                                            "bf16_gen_n64_p8x32"};
  if (!out_plan) return invalid();
  *out_plan = nullptr;
  if (best_ms) *best_ms = 0.f;
  if (!desc || launches < 1) return invalid();
  if (desc->dtype != CC3D_BF16) return causal_conv3d_plan(desc, out_plan);  // one fp32 kernel
  hipEvent_t e0 = nullptr, e1 = nullptr;
  if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) {
    if (e0) (void)hipEventDestroy(e0);
    cc3d::g_device_error.fetch_add(1, std::memory_order_relaxed);
    return CC3D_ERR_DEVICE;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  cc3d_plan_t best = nullptr;
  float best_t = 0.f;
  cc3d_status_t st = CC3D_ERR_UNSUPPORTED;
  for (const char* name : kCandidates) {
    cc3d_plan_t p = nullptr;
    const cc3d_status_t ps = name ? causal_conv3d_plan_variant(desc, name, &p) : causal_conv3d_plan(desc, &p);
    if (ps == CC3D_ERR_UNSUPPORTED) continue;
    if (ps != CC3D_OK) {
      st = ps;
      break;
    }
    // first call packs the weights and warms up; then time the conv alone
    cc3d_status_t rs = causal_conv3d_forward(p, x, cache_in, w, b, out, nullptr, stream);
    if (rs == CC3D_OK && hipEventRecord(e0, s) != hipSuccess) rs = CC3D_ERR_DEVICE;
    for (int i = 0; i < launches && rs == CC3D_OK; ++i)
      rs = causal_conv3d_forward_packed(p, x, cache_in, b, out, nullptr, stream);
    float ms = 0.f;
    if (rs == CC3D_OK && (hipEventRecord(e1, s) != hipSuccess || hipEventSynchronize(e1) != hipSuccess ||
                          hipEventElapsedTime(&ms, e0, e1) != hipSuccess))
      rs = CC3D_ERR_DEVICE;
    if (rs != CC3D_OK) {
      (void)hipStreamSynchronize(s);
      causal_conv3d_plan_destroy(p);
      st = rs;
      break;
    }
    ms /= float(launches);
    if (!best || ms < best_t) {
      if (best) causal_conv3d_plan_destroy(best);
      best = p;
      best_t = ms;
    } else {
      causal_conv3d_plan_destroy(p);
    }
    st = CC3D_OK;
  }
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  if (st != CC3D_OK || !best) {
    if (best) causal_conv3d_plan_destroy(best);
    return st == CC3D_OK ? CC3D_ERR_UNSUPPORTED : st;
  }
  *out_plan = best;
  if (best_ms) *best_ms = best_t;
  return CC3D_OK;
}

// Frees a plan's device workspace (called by causal_conv3d_plan_destroy).
void cc3d_release_workspace(cc3d_plan_t plan) {
  std::lock_guard<std::mutex> lock(plan->mu);
  if (plan->wpk) {
    int cur = -1;
    const bool switch_dev = hipGetDevice(&cur) == hipSuccess && cur != plan->wpk_device;
    if (switch_dev) (void)hipSetDevice(plan->wpk_device);
    (void)hipFree(plan->wpk);
    if (switch_dev) (void)hipSetDevice(cur);
    plan->wpk = nullptr;
  }
}
