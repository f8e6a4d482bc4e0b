// conv_bf16_g32: the group-staged kernel of the large 3x3 maps (also at
// spatial dilation 2 and at spatial stride 2).
#include "cc3d_device.h"

namespace {

// The scheduler counters of every launch of this kernel on the device:
// cc3d::kSchedSlots slots of kSchedInts ints (a tile counter per XCD, the
// count of finished workgroups, then the cache-out chunk counter).  Zero when the code object is loaded;
// each launch leaves its slot zero when it completes.
constexpr int kSchedInts = 16;
__device__ __attribute__((unused)) int g32_sched[cc3d::kSchedSlots * kSchedInts];
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
//
// WPK: the weight sub-stages come from the packed image (a.wpk), one
// contiguous run each; otherwise each slot's 16-byte piece is gathered from W
// as the caller stores it, into the same LDS layout.
//
// SPL: split reduction (maps with so few tiles that most compute units would
// idle).  Work unit u is split u % a.splits of tile u / a.splits and runs a
// contiguous share of the tile's group sequence; every unit stores its fp32
// partial sums in the workspace (device-scope stores), counts itself in the
// tile's arrival counter, and the last to arrive adds the partials of all
// splits in split order -- the same sum whichever unit arrives last -- and
// runs the epilogue.  It leaves the counter zero.
template <int BN, int TH, int WM, int DD, int SS, int KSP, bool WPK, bool SPL>
__global__ __launch_bounds__(WM * 64) __attribute__((amdgpu_waves_per_eu(WM / 4, WM / 4))) void conv_bf16_g32(ConvArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)
  using WT = WTile<BN, 3, 16>;
  static_assert(SS == 1 || (SS == 2 && DD == 1), "stride 2 runs undilated");
  static_assert(!SPL || KSP == 1, "split units on the one-wave-per-row-group schedule");
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
  // (+ 64 slots: the sink of the loads past the end of a buffer, below)
  static_assert((2 * ZSLOTS + 2 * KSP * WSLOTS + (KSP == 1 ? 0 : 64) + 64) * 16 + 2 * BN * 4 <= 160 * 1024,
                "LDS budget");
  // channel-half split: the second half's sums pass through an idle halo buffer
  static_assert(KSP == 1 || (WM / 2) * CW * RW * 16 * 64 * 4 <= ZSLOTS * 16, "partial sums");
  // s_waitcnt immediate that waits for vmcnt <= n and nothing else (gfx9
  // encoding: vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8)
  constexpr auto vm_imm = [](int n) { return ((n >> 4) << 14) | 0x0F70 | (n & 15); };
  static_assert(ZIT + WIT <= 63, "vmcnt range");

  __shared__ uint4 zl[2 * ZSLOTS];
  // Weight buffers.  With KSP = 1 the two sub-stage buffers are separate
  // arrays, selected at compile time: the compiler's wait-count tracking
  // then knows that reading one does not depend on a direct-to-LDS load into
  // the other still in flight (with one array it drains every load before
  // each sub-stage's first weight read).
  __shared__ uint4 wl[KSP == 1 ? WSLOTS : 2 * KSP * WSLOTS];
  __shared__ uint4 wl_b1[KSP == 1 ? WSLOTS : 64];
  auto wbuf = [&](int b) -> uint4* { return KSP == 1 ? (b ? wl_b1 : wl) : wl + b * WSLOTS; };
  __shared__ float bias_lds[2][BN];
  __shared__ uint4 sink[64];  // destination of the load instructions past a buffer's end

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
  int* const sched = g32_sched + a.sched_slot * kSchedInts;
  auto claim = [&](int x) {  // next claim number on XCD x's counter
    return __hip_atomic_fetch_add(sched + x, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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
  const unsigned char* __restrict__ wpk = static_cast<const unsigned char*>(WPK ? a.wpk : a.w);
  const int64_t w_bytes = int64_t(a.cout) * a.kt * 9 * a.cin * 2;
  const unsigned short* __restrict__ bs = static_cast<const unsigned short*>(a.b);
  unsigned short* __restrict__ os = static_cast<unsigned short*>(a.out);

  struct Tile {
    int o, nb, nn, x0, y0, n0, nact;
    int k0, k1, k2, k3;
    int z0, z1, z2, z3;
    int t, sp, g0, g1;  // tile, split, and the split's groups [g0, g1) (SPL only)
  };
  auto act_frame = [&](KArgs k, int j) {  // the j-th output frame with an active tap
    int o = k->act_lo[0] + j;
#pragma unroll
    for (int i = 0; i + 1 < kMaxFrameIv; ++i)
      if (i + 1 < k->nact_iv && j >= k->act_n[i]) {
        j -= k->act_n[i];
        o = k->act_lo[i + 1] + j;
      }
    return o;
  };
  auto decode = [&](int t) {
    const KArgs k = kargs();
    Tile c;
    c.t = t;
    c.sp = 0;
    if constexpr (SPL) {
      c.sp = t % k->splits;
      c.t = t = t / k->splits;
    }
    c.o = act_frame(k, t % k->ta_n);
    t /= k->ta_n;
    c.nb = t % k->nblk_n;
    t /= k->nblk_n;
    const int tile_x = t % k->tiles_x;
    t /= k->tiles_x;
    const int tile_y = t % k->tiles_y;
    c.nn = t / k->tiles_y;
    c.x0 = tile_x * TW;
    c.y0 = tile_y * TH;
    c.n0 = c.nb * BN;
    c.nact = 0;
    c.k0 = c.k1 = c.k2 = c.k3 = 0;
    c.z0 = c.z1 = c.z2 = c.z3 = 0;
#pragma unroll
    for (int q = 0; q < kMaxTapsBf16; ++q) {
      const int z = c.o * k->st + k->delta[q];
      if (q < k->kt && z >= 0 && z < k->tz) {
        if (c.nact == 0) { c.k0 = q; c.z0 = z; }
        else if (c.nact == 1) { c.k1 = q; c.z1 = z; }
        else if (c.nact == 2) { c.k2 = q; c.z2 = z; }
        else { c.k3 = q; c.z3 = z; }
        ++c.nact;
      }
    }
    c.g0 = c.g1 = 0;
    if constexpr (SPL) {
      const int g = c.nact * (k->cin / 32);
      c.g0 = c.sp * g / k->splits;
      c.g1 = (c.sp + 1) * g / k->splits;
    }
    return c;
  };
  auto pick = [](int i, int v0, int v1, int v2, int v3) { return i == 0 ? v0 : i == 1 ? v1 : i == 2 ? v2 : v3; };
  auto uniform = [](const void* p) { return uniform_ptr(p); };
  // gather offsets of this thread's weight slots (in-place weights)
  int woff[WIT];
#pragma unroll
  for (int it = 0; it < WIT; ++it) woff[it] = WPK ? (it * NT + tid) * 16 : w_gather_offset<BN, 3, 16>(it * NT + tid, a.kt, a.cin);

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
    int t, ti, gz, gi;  // (gi: the group's index in its tile's sequence, SPL only)
  };
  auto halo_src = [&](const Tile& c, int ti, int gz) {
    const int z = pick(ti, c.z0, c.z1, c.z2, c.z3);
    return static_cast<const unsigned short*>(uniform((z < a.tc ? cs + (int64_t(c.nn) * a.tc + z) * frame_el
                                                                : xs + (int64_t(c.nn) * a.tx + (z - a.tc)) * frame_el) +
                                                     gz * 32));
  };
  // the weights of sub-stage cc (16 channels) of active tap ti: the packed
  // tile, or the stage's first piece in W and the bytes of W from there on
  struct WSrc {
    const unsigned char* p;
    int rec;
  };
  auto wsrc = [&](const Tile& c, int ti, int cc) {
    const int k = pick(ti, c.k0, c.k1, c.k2, c.k3);
    WSrc r;
    if constexpr (WPK) {
      r.p = static_cast<const unsigned char*>(uniform(wpk + ((int64_t(c.nb) * nch + cc) * a.kt + k) * (WSLOTS * 16)));
      r.rec = WSLOTS * 16;
    } else {
      const int64_t off = ((int64_t(c.nb) * BN * a.kt + k) * 9 * a.cin + cc * 16) * 2;
      r.p = static_cast<const unsigned char*>(uniform(wpk + off));
      r.rec = __builtin_amdgcn_readfirstlane(int(w_bytes - off));
    }
    return r;
  };
  const WSrc wnone{wpk, 0};
  // Every wave issues every load instruction of a stage (ZIT halo, WIT
  // weight), so each wait below is one count for all waves and the loop has
  // no per-wave branches: a wave whose 64 slots of the last instruction lie
  // past the buffer aims it at the sink, with offsets out of range (slot ids
  // past ZCH / WCH), which the range check turns into zeros.
  auto issue_z = [&](const unsigned short* fp, int zb, int it) {
    const bool in = ZSLOTS % NT == 0 || it * NT + wave * 64 < ZSLOTS;  // wave-uniform
    const __amdgpu_buffer_rsrc_t r =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<unsigned short*>(fp), 0, frame_bytes, 0x00020000);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        r, (__attribute__((address_space(3))) void*)(in ? zl + zb * ZSLOTS + it * NT + wave * 64 : sink), 16,
        zoff[it], 0, 0, 0);
  };
  auto issue_w = [&](const WSrc& wp, int wb, int it) {
    const bool in = WSLOTS % NT == 0 || it * NT + wave * 64 < WSLOTS;
    const __amdgpu_buffer_rsrc_t r =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<unsigned char*>(wp.p), 0, wp.rec, 0x00020000);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        r, (__attribute__((address_space(3))) void*)(in ? wbuf(wb) + it * NT + wave * 64 : sink), 16, woff[it],
        0, 0, 0);
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
    unsigned char* eb = wave < 4 ? reinterpret_cast<unsigned char*>(wbuf(widle)) + wave * 32 * EROW
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
  Grp nx{ctile, 0, 0, 0};
  Tile nt{};
  bool nx_ok = ctile >= 0;
  // (a split unit's groups start at g0: group-major, gz = g0 / nact)
  auto nx_start = [&]() {
    if constexpr (SPL) {
      nx.gi = nt.g0;
      nx.gz = nt.g0 / nt.nact;
      nx.ti = nt.g0 - nx.gz * nt.nact;
    }
  };
  if (nx_ok) {
    nt = decode(ctile);
    halo_offsets(nt);
    nx_start();
  }
  auto nx_advance = [&]() {
    if constexpr (SPL) {
      if (++nx.ti == nt.nact) {
        nx.ti = 0;
        ++nx.gz;
      }
      if (++nx.gi == nt.g1) {
        nx.t = nx.t == ctile ? tnext : tnn;
        if (nx.t < 0) {
          nx_ok = false;
          return;
        }
        nt = decode(nx.t);
        halo_offsets(nt);
        nx_start();
      }
      return;
    }
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

  // (each inline-asm wait is followed by the same wait as a builtin, which
  // the compiler's wait-count tracking sees: it then knows that the older
  // loads -- the weight sub-stage -- have landed, and does not drain the
  // halo loads still in flight before it reads that sub-stage)
  auto wait_halo_in_flight = [&]() {  // all but this wave's halo loads of the last group
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(ZIT) : "memory");
    __builtin_amdgcn_s_waitcnt(vm_imm(ZIT));
    asm volatile("" ::: "memory");
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

  // Split reduction (SPL): this thread's share of a unit's fp32 partial sums
  // (float4 runs interleaved across the workgroup's threads, so that each
  // store instruction writes one contiguous block).  The units of a tile may
  // run on different XCDs, whose L2 caches are not coherent with each
  // other: the partials are written and read with device-scope (sc1)
  // accesses, which go to the device's coherence point, and the arrival
  // count is a device-scope atomic.  Returns (uniformly) whether this unit
  // arrived last; acc then holds the tile's sum over all splits, added in
  // split order.
  __shared__ int last_lds;
  auto reduce_splits = [&](const Tile& c) {
    if constexpr (!SPL) {
      return true;
    } else {
      constexpr int NACC = CW * RW * 16;
      constexpr int kSC1 = 16;  // cache-policy bits of a buffer access: device scope
      constexpr int part_bytes = (NACC / 4) * NT * 16;
      const KArgs k = kargs();
      const int splits = k->splits;
      int* const arrivals = static_cast<int*>(k->ws);
      const unsigned char* const tile_parts =
          static_cast<const unsigned char*>(k->ws) + k->ws_part + int64_t(c.t) * splits * part_bytes;
      const __amdgpu_buffer_rsrc_t pr =
          __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(uniform(tile_parts)), 0,
                                            __builtin_amdgcn_readfirstlane(splits * part_bytes), 0x00020000);
      const int mine = __builtin_amdgcn_readfirstlane(c.sp * part_bytes);
#pragma unroll
      for (int q = 0; q < CW; ++q)
#pragma unroll
        for (int r = 0; r < RW; ++r)
#pragma unroll
          for (int v4 = 0; v4 < 4; ++v4) {
            const int e4 = (q * RW + r) * 4 + v4;
            const u32x4_t v = {__float_as_uint(acc[q][r][v4 * 4]), __float_as_uint(acc[q][r][v4 * 4 + 1]),
                               __float_as_uint(acc[q][r][v4 * 4 + 2]), __float_as_uint(acc[q][r][v4 * 4 + 3])};
            __builtin_amdgcn_raw_buffer_store_b128(v, pr, tid * 16, mine + e4 * NT * 16, kSC1);
          }
      vm_drain();  // the partials are at the coherence point
      barrier();
      if (tid == 0) {
        const int before = __hip_atomic_fetch_add(arrivals + c.t, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const bool last = before == splits - 1;
        if (last) __hip_atomic_store(arrivals + c.t, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        last_lds = last;
      }
      barrier();
      const bool last = __builtin_amdgcn_readfirstlane(last_lds) != 0;
      if (last) {
        zero_acc();
        // per 16-float accumulator run, the loads of up to four units (16
        // float4) are issued together, then added in split order
#pragma unroll
        for (int q = 0; q < CW; ++q)
#pragma unroll
          for (int r = 0; r < RW; ++r) {
            const int run = (q * RW + r) * 4 * NT * 16;
            for (int sp0 = 0; sp0 < splits; sp0 += 4) {
              u32x4_t pv[4][4];
#pragma unroll
              for (int j = 0; j < 4; ++j)
                if (sp0 + j < splits) {
                  const int so = __builtin_amdgcn_readfirstlane((sp0 + j) * part_bytes + run);
#pragma unroll
                  for (int v = 0; v < 4; ++v)
                    pv[j][v] = __builtin_amdgcn_raw_buffer_load_b128(pr, tid * 16, so + v * NT * 16, kSC1);
                }
#pragma unroll
              for (int j = 0; j < 4; ++j)
                if (sp0 + j < splits) {
#pragma unroll
                  for (int v = 0; v < 4; ++v)
#pragma unroll
                    for (int e = 0; e < 4; ++e) acc[q][r][v * 4 + e] += __uint_as_float(pv[j][v][e]);
                }
            }
          }
        vm_drain();
      }
      return last;
    }
  };

  if constexpr (KSP == 2) {
    // prologue: the first group's halo and both weight halves (group buffer 0)
    int wcur = 0;  // weight group buffer of the current group: halves 2*wcur, 2*wcur+1
    if (nx_ok) {
      const unsigned short* fp = halo_src(nt, nx.ti, nx.gz);
      const WSrc w0p = wsrc(nt, nx.ti, nx.gz * 2);
      const WSrc w1p = wsrc(nt, nx.ti, nx.gz * 2 + 1);
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
            const WSrc wn0 = more ? wsrc(nt, nx.ti, nx.gz * 2) : wnone;
            const WSrc wn1 = more ? wsrc(nt, nx.ti, nx.gz * 2 + 1) : wnone;
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
          if (gi == 0 && tid < BN) {
            unsigned bv = bval;  // (used here, not right after the load, as below)
            asm volatile("" : "+v"(bv));
            bias_lds[par][tid] = bf16_to_f32(static_cast<unsigned short>(bv));
          }
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
      const WSrc wp = wsrc(nt, nx.ti, nx.gz * 2);
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
        // (a split unit runs groups [g0, g1) of its tile)
        const int gbeg = SPL ? ct.g0 : 0, gend = SPL ? ct.g1 : ngt;
        for (int gi = gbeg; gi < gend; ++gi) {
          // group-major order: the active taps of one 32-channel group run back
          // to back, so a source frame's group is reused by the output frames of
          // the neighbouring tiles within a few groups, while it is still in L2
          const int gz = gi / ct.nact, ti = gi - gz * ct.nact;
          const uint4* zb = zl + hpar * ZSLOTS;
          unsigned short bval = 0;
          if (gi == gbeg) bval = bias_value(ct);
          const bool more = nx_ok;
          // sub-stage 0: load W[1] <- (this group, second half), H[next] <- next group
          {
            const WSrc wp1 = wsrc(ct, ti, gz * 2 + 1);
            const unsigned short* fpn = more ? halo_src(nt, nx.ti, nx.gz) : xs;
            const int hn = __builtin_amdgcn_readfirstlane(hpar ^ 1);
            compute(zb, wbuf(0), rows_in, std::integral_constant<int, 0>{}, std::integral_constant<int, WIT + ZIT>{},
                    std::integral_constant<int, NSTEP>{}, [&](int k) {
                      if (k < WIT) issue_w(wp1, 1, k);
                      else if (more) issue_z(fpn, hn, k - WIT);
                    });
          }
          if (more) wait_halo_in_flight();
          else vm_drain();
          if (gi == gbeg && tid < BN) {
            // (the empty asm keeps the use of the bias load -- and so the
            // compiler's wait for it -- here, after the sub-stage, where the
            // load has long landed, instead of right after it is issued)
            unsigned bv = bval;
            asm volatile("" : "+v"(bv));
            bias_lds[par][tid] = bf16_to_f32(static_cast<unsigned short>(bv));
          }
          barrier();
          // sub-stage 1: load W[0] <- next group, first half.  In the first
          // group, thread 0 also claims a tile (the atomic's latency hides
          // behind the sub-stage; the claim is published at its barrier).
          const int cx = (xcd + steal) & 7;
          int v = 0;
          if (gi == gbeg && claims && tid == 0) v = claim(cx);
          {
            const WSrc wpn = more ? wsrc(nt, nx.ti, nx.gz * 2) : wnone;
            compute(zb, wbuf(1), rows_in, std::integral_constant<int, 1>{}, std::integral_constant<int, WIT>{},
                    std::integral_constant<int, (NSTEP + 1) / 2>{}, [&](int k) {
                      if (more) issue_w(wpn, 0, k);
                    });
          }
          asm volatile("" ::: "memory");  // the claim is read only after the sub-stage
          if (gi == gbeg && claims && tid == 0) {
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
          if (gi == gbeg && claims) tnn = __builtin_amdgcn_readfirstlane(claim_lds);
          if (more) nx_advance();
          hpar ^= 1;
        }
        // (the output stores may stay in flight across this barrier)
        if (!SPL || reduce_splits(ct)) epilogue(ct, par, hpar ^ 1, 1);
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

  // Cache-out: source frames co_lo .. tz - 1 of every batch item go to
  // cache_out[n][0 .. tz - co_lo) in chunks of U 16-byte pieces per thread,
  // claimed from the launch's copy counter once a workgroup's tiles have run
  // out, so the copy runs on the compute units the last tiles leave idle.
  // The claim of the next chunk is in flight while a chunk is copied; the
  // buffer range check drops the pieces past the end of a frame.
  {
    const KArgs k = kargs();
    const int co_lo = k->co_lo, tz = k->tz;
    if (co_lo < tz) {
      constexpr int U = 16;
      constexpr int CHUNK = NT * 16 * U;
      const int L = tz - co_lo;
      const int cpf = int((int64_t(frame_bytes) + CHUNK - 1) / CHUNK);
      const int nchunks = k->n * L * cpf;
      const unsigned char* const xb = static_cast<const unsigned char*>(k->x);
      const unsigned char* const cb = static_cast<const unsigned char*>(k->cache);
      unsigned char* const db = static_cast<unsigned char*>(k->cache_out);
      const int tx = k->tx, tc = k->tc;
      __shared__ int co_claim[2];
      if (tid == 0) co_claim[0] = __hip_atomic_fetch_add(sched + 9, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      barrier();
      int cpar = 0;
      int c = co_claim[0];
#pragma unroll 1
      while (c < nchunks) {
        int nxt = 0;
        if (tid == 0) nxt = __hip_atomic_fetch_add(sched + 9, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const int f = c / cpf, part = c - f * cpf;
        const int nn = f / L, j = f - nn * L, zf = co_lo + j;
        const int64_t off = int64_t(part) * CHUNK;
        const unsigned char* src = (zf < tc ? cb + (int64_t(nn) * tc + zf) * frame_bytes
                                            : xb + (int64_t(nn) * tx + (zf - tc)) * frame_bytes) + off;
        unsigned char* dst = db + int64_t(f) * frame_bytes + off;
        const int64_t left = frame_bytes - off;
        const int rec = __builtin_amdgcn_readfirstlane(left < CHUNK ? int(left) : CHUNK);
        const __amdgpu_buffer_rsrc_t rs =
            __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(uniform(src)), 0, rec, 0x00020000);
        const __amdgpu_buffer_rsrc_t rd =
            __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(uniform(dst)), 0, rec, 0x00020000);
        u32x4_t v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = __builtin_amdgcn_raw_buffer_load_b128(rs, (u * NT + tid) * 16, 0, 0);
#pragma unroll
        for (int u = 0; u < U; ++u) __builtin_amdgcn_raw_buffer_store_b128(v[u], rd, (u * NT + tid) * 16, 0, 0);
        cpar ^= 1;
        if (tid == 0) co_claim[cpar] = nxt;
        barrier();
        c = co_claim[cpar];
      }
    }
  }

  // The last workgroup to finish clears the counters for the next launch
  // that uses them (its claims and every other workgroup's are done: each
  // workgroup counts itself after its last claim).
  if (tid == 0) {
    const int done = __hip_atomic_fetch_add(sched + 8, 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    if (done == int(gridDim.x) - 1)
      for (int x = 0; x < 10; ++x) __hip_atomic_store(sched + x, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
#endif
}

template <int BN, int TH, int WM, int DD, int SS, int KSP, bool WPK, bool SPL>
const void* g32_kernel() {
  return reinterpret_cast<const void*>(&conv_bf16_g32<BN, TH, WM, DD, SS, KSP, WPK, SPL>);
}

// (SPL: the split instantiation, for a.splits > 1: its work units are the
// tiles' splits, a.nat of them)
template <int BN, int TH, int WM, int DD = 1, int SS = 1, int KSP = 1, bool SPL = false>
hipError_t launch_g32(const ConvArgs& a, int64_t tiles, int cus, hipStream_t s) {
  if (a.wpk) return launch_persistent<&g32_kernel<BN, TH, WM, DD, SS, KSP, true, SPL>>(a, tiles, cus, WM * 64, s);
  return launch_persistent<&g32_kernel<BN, TH, WM, DD, SS, KSP, false, SPL>>(a, tiles, cus, WM * 64, s);
}

// The split units of a.nat tiles: a.splits per tile.
template <int BN, int TH, int WM>
hipError_t launch_g32_split(const ConvArgs& a, int cus, hipStream_t s) {
  ConvArgs b = a;
  b.nat = a.nat * a.splits;
  return launch_g32<BN, TH, WM, 1, 1, 1, true>(b, std::max(b.nat, 1), cus, s);
}

}  // namespace

namespace cc3d {

hipError_t launch_g32_family(int kernel_id, const ConvArgs& a, int64_t tiles, int cus, hipStream_t s) {
  if (a.splits > 1) {
    if (kernel_id == CC3D_K_BF16_S3_N96_G32W8) return launch_g32_split<96, 16, 8>(a, cus, s);
    if (kernel_id == CC3D_K_BF16_S3_N64_G32W8) return launch_g32_split<64, 24, 8>(a, cus, s);
    return hipErrorInvalidValue;
  }
  switch (kernel_id) {
    case CC3D_K_BF16_S3_N96_G32W8: return launch_g32<96, 16, 8>(a, tiles, cus, s);
    case CC3D_K_BF16_S3_N64_G32W8: return launch_g32<64, 24, 8>(a, tiles, cus, s);
    case CC3D_K_BF16_S3D2_N64_G32W8: return launch_g32<64, 16, 8, 2>(a, tiles, cus, s);
    case CC3D_K_BF16_S3S2_N96_G32W4: return launch_g32<96, 4, 4, 1, 2>(a, tiles, cus, s);
    case CC3D_K_BF16_S3S2_N64_G32W8: return launch_g32<64, 4, 8, 1, 2, 2>(a, tiles, cus, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace cc3d
