// conv_bf16_mfma: the implicit-GEMM kernel of the smaller 3x3 maps (two
// workgroups per compute unit), of other C_out, and of the 1x1 / (k_t,1,1)
// convs; and the packer of the stage-ordered weight image that it and the
// group-staged kernel read.
#include "cc3d_device.h"

namespace {
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

// WPK: the stage weights come from the packed image (a.wpk), one contiguous
// run per stage; otherwise each slot's 16-byte piece is gathered from W as
// the caller stores it, into the same LDS layout.  SPLIT: the instantiation
// that runs split units (a.splits > 1; the others carry no reduction code).
template <int BN, int TH, int WM, int WN, int KS, int CB, int NBUF, int OCC, bool WPK, bool SPLIT>
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
  constexpr int LPS = ZIT + WIT;               // load instructions of every wave per stage
  static_assert((NW == 4 || NW == 8) && TH % WM == 0 && BN % (32 * WN) == 0, "wave tiling");
  static_assert(PZ == 2 || PZ == 4 || PZ == 8, "stage channels");
  constexpr int WG_PER_CU = OCC * 4 / NW > 0 ? OCC * 4 / NW : 1;  // OCC is waves per SIMD
  static_assert(NBUF >= 2 && (NBUF * STAGE * 16 + 2 * BN * 4 + 1024) * WG_PER_CU <= 160 * 1024, "LDS budget");
  static_assert(LPS * (NBUF - 2) <= 63, "vmcnt range");

  __shared__ uint4 lds[NBUF * STAGE];
  __shared__ float bias_lds[2][BN];
  __shared__ uint4 sink[64];  // destination of the load instructions past a buffer's end

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
  const unsigned char* __restrict__ wpk = static_cast<const unsigned char*>(WPK ? a.wpk : a.w);
  const int64_t w_bytes = int64_t(a.cout) * a.kt * KS * KS * a.cin * 2;
  const unsigned short* __restrict__ bs = static_cast<const unsigned short*>(a.b);
  unsigned short* __restrict__ os = static_cast<unsigned short*>(a.out);

  // A work unit: split `sp` of tile `t` -- one output frame o of batch item
  // nn, a TH x 32 patch at (y0, x0), output channels [n0, n0 + BN); its
  // active taps k[0..nact) read source frames z[i] = o + delta_k[i] of
  // Z = [cache; x].  The tile's stages (active tap major, channel chunk
  // minor: nact * nch of them) are divided evenly among the splits; this
  // unit runs stages [s0, s1).
  struct Tile {
    int o, nb, nn, x0, y0, n0, nact;
    int k0, k1, k2, k3;  // active taps, in order
    int z0, z1, z2, z3;  // their source frames
    int t, sp, s0, s1;
  };
  const int splits = SPLIT ? a.splits : 1;
  auto decode = [&](int u) {
    // (through the opaque argument pointer: see kargs(); the split
    // instantiations read `a` -- with the pointer their register allocation
    // reserves a private-memory slot, which makes the runtime set up scratch)
    const ConvArgs* k = &a;
    if constexpr (!SPLIT) k = reinterpret_cast<const ConvArgs*>(kargs());
    Tile c;
    c.t = u / splits;
    c.sp = u - c.t * splits;
    int t = c.t;
    c.o = t % k->to;
    t /= k->to;
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
    const int nst = c.nact * (k->cin / CB);
    c.s0 = c.sp * nst / splits;
    c.s1 = (c.sp + 1) * nst / splits;
    return c;
  };
  auto pick = [](int i, int v0, int v1, int v2, int v3) { return i == 0 ? v0 : i == 1 ? v1 : i == 2 ? v2 : v3; };
  auto uniform = [](const void* p) { return uniform_ptr(p); };
  // gather offsets of this thread's weight slots (in-place weights)
  int woff[WIT];
#pragma unroll
  for (int it = 0; it < WIT; ++it) woff[it] = WPK ? (it * NT + tid) * 16 : w_gather_offset<BN, KS, CB>(it * NT + tid, a.kt, a.cin);

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
    const unsigned char* wp;   // weight tile (packed), or the stage's first piece in W
    int wrec;                  // bytes the weight buffer range covers
    int buf;                   // LDS buffer
  };
  auto prep_stage = [&](const Tile& c, int cc, int ti, int buf) {
    const int z = pick(ti, c.z0, c.z1, c.z2, c.z3), k = pick(ti, c.k0, c.k1, c.k2, c.k3);
    StageLoad l;
    l.fp = static_cast<const unsigned short*>(uniform((z < a.tc ? cs + (int64_t(c.nn) * a.tc + z) * frame_el
                                                                 : xs + (int64_t(c.nn) * a.tx + (z - a.tc)) * frame_el) +
                                                      cc * CB));
    if constexpr (WPK) {
      l.wp = static_cast<const unsigned char*>(uniform(wpk + ((int64_t(c.nb) * nch + cc) * a.kt + k) * (WSLOTS * 16)));
      l.wrec = WSLOTS * 16;
    } else {
      const int64_t off = ((int64_t(c.nb) * BN * a.kt + k) * (KS * KS) * a.cin + cc * CB) * 2;
      l.wp = static_cast<const unsigned char*>(uniform(wpk + off));
      l.wrec = __builtin_amdgcn_readfirstlane(int(w_bytes - off));
    }
    l.buf = __builtin_amdgcn_readfirstlane(buf);
    return l;
  };
  constexpr int NLOAD = ZIT + WIT;  // load instructions of one stage, per thread
  // slots are filled 64 at a time (one wave instruction).  Every wave
  // issues every instruction, so the waits are one count for all waves: a
  // wave whose 64-slot block lies past the tile aims it at the sink, with
  // offsets out of range (slot ids past ZCH / WCH), which the range check
  // turns into zeros.
  auto issue_piece = [&](const StageLoad& l, int j) {
    uint4* zb = lds + l.buf * STAGE;
    if (j < ZIT) {
      const bool in = ZSLOTS % NT == 0 || j * NT + wave * 64 < ZSLOTS;  // wave-uniform
      const __amdgpu_buffer_rsrc_t zr =
          __builtin_amdgcn_make_buffer_rsrc(const_cast<unsigned short*>(l.fp), 0, frame_bytes, 0x00020000);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          zr, (__attribute__((address_space(3))) void*)(in ? zb + j * NT + wave * 64 : sink), 16, zoff[j], 0, 0, 0);
    } else {
      const int it = j - ZIT;
      const bool in = WSLOTS % NT == 0 || it * NT + wave * 64 < WSLOTS;
      const __amdgpu_buffer_rsrc_t wr =
          __builtin_amdgcn_make_buffer_rsrc(const_cast<unsigned char*>(l.wp), 0, l.wrec, 0x00020000);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          wr, (__attribute__((address_space(3))) void*)(in ? zb + ZSLOTS + it * NT + wave * 64 : sink), 16,
          woff[it], 0, 0, 0);
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
  // flattened (unit, stage) sequence, crossing unit boundaries, so a unit's
  // first stages load while the previous unit finishes and writes its
  // outputs.  Stage position p uses LDS buffer p % NBUF.  lst is the stage
  // of the unit's tile (tap lti = lst / nch, chunk lcc = lst % nch).
  int ltile = ctile, lcc = 0, lti = 0, lst = 0;
  Tile lt = decode(ltile);
  auto lt_set = [&]() {
    lst = lt.s0;
    lti = lst / nch;
    lcc = lst - lti * nch;
  };
  auto lt_advance_tile = [&]() {
    for (;;) {
      ltile = next_tile(ltile);
      if (ltile < 0) return;
      lt = decode(ltile);
      if (lt.s1 > lt.s0) break;
    }
    lt_set();
    halo_offsets(lt);
  };
  if (lt.s1 > lt.s0) {
    lt_set();
    halo_offsets(lt);
  } else {
    lt_advance_tile();
  }
  auto advance_load = [&]() {
    if (++lst == lt.s1) {
      lt_advance_tile();
    } else if (++lcc == nch) {
      lcc = 0;
      ++lti;
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
  constexpr auto vm_imm = [](int n) { return ((n >> 4) << 14) | 0x0F70 | (n & 15); };
  auto wait_newer_stages = [&]() {
    constexpr int N = LPS * (NBUF - 2);
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
    __builtin_amdgcn_s_waitcnt(vm_imm(N));  // (the same wait, seen by the compiler's own tracking)
  };

  // Workgroup barrier with explicit waits only: the caller has waited for
  // the loads that must have landed; this waits for the wave's own LDS
  // accesses.  (__syncthreads() would also drain every load in flight,
  // including the NBUF - 2 stages meant to stay in flight across it.)
  auto barrier = [&]() {
    if constexpr (NBUF == 2) {
      __syncthreads();  // (nothing may stay in flight: the same waits, measured slightly faster)
    } else {
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
    }
  };

  int issued = 0;
#pragma unroll
  for (int i = 0; i < NBUF - 1; ++i)
    if (issue(i)) ++issued;
  if (NBUF > 2 && issued == NBUF - 1) wait_newer_stages();
  else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();

  // Split reduction: this thread's share of a unit's fp32 partial sums
  // (NACC floats, stored as float4 runs interleaved across the workgroup's
  // threads so that each store instruction writes one contiguous block).
  // The units of a tile may run on different XCDs, whose L2 caches are not
  // coherent with each other: the partials are written and read with
  // device-scope (sc1) accesses, which go to the device's coherence point,
  // and the arrival count is a device-scope atomic, so no cache-wide
  // write-back or invalidation is needed.
  constexpr int NACC = CW * RW * 16;
  constexpr int kSC1 = 16;  // cache-policy bits of a buffer access: device scope
  int* const arrivals = static_cast<int*>(a.ws);
  __shared__ int last_lds;
  // Store this unit's partials, count its arrival; returns (uniformly)
  // whether it arrived last, in which case acc then holds the tile's sum
  // over all splits, in split order.
  auto reduce_splits = [&](const Tile& c) {
    const int part_bytes = (NACC / 4) * NT * 16;  // one unit's partials
    const unsigned char* tile_parts =
        static_cast<const unsigned char*>(a.ws) + a.ws_part + int64_t(c.t) * splits * part_bytes;
    const __amdgpu_buffer_rsrc_t pr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<void*>(uniform(tile_parts)), 0, __builtin_amdgcn_readfirstlane(splits * part_bytes), 0x00020000);
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
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the partials are at the coherence point
    __builtin_amdgcn_s_waitcnt(0xF70);
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
      // The partials are read at the coherence point, so each load is a
      // long round trip: per 16-float accumulator run, the loads of four
      // units (16 float4) are issued together, then added in split order.
#pragma unroll
      for (int q = 0; q < CW; ++q)
#pragma unroll
        for (int r = 0; r < RW; ++r) {
          const int run = (q * RW + r) * 4 * NT * 16;
          for (int sp0 = 0; sp0 < splits; sp0 += 4) {
            u32x4_t p[4][4];
#pragma unroll
            for (int j = 0; j < 4; ++j)
              if (sp0 + j < splits) {
                const int so = __builtin_amdgcn_readfirstlane((sp0 + j) * part_bytes + run);
#pragma unroll
                for (int v = 0; v < 4; ++v)
                  p[j][v] = __builtin_amdgcn_raw_buffer_load_b128(pr, tid * 16, so + v * NT * 16, kSC1);
              }
#pragma unroll
            for (int j = 0; j < 4; ++j)
              if (sp0 + j < splits) {
#pragma unroll
                for (int v = 0; v < 4; ++v)
#pragma unroll
                  for (int e = 0; e < 4; ++e) acc[q][r][v * 4 + e] += __uint_as_float(p[j][v][e]);
              }
          }
        }
    }
    return last;
  };

  int pos = 0, par = 0;
  Tile ct = decode(ctile);
  for (;;) {
    zero_acc();
    if (ct.s1 == ct.s0) {
      // no stage (no active tap, or fewer stages than splits).  The load
      // cursor has already issued stages pos .. pos+NBUF-2 of the next units
      // into their buffers; the one buffer they leave free, (pos+NBUF-1) %
      // NBUF, stages the outputs (its next loads go out only after the
      // barrier that closes this unit).
      if (tid < BN) bias_lds[par][tid] = bf16_to_f32(bias_value(ct));
      __syncthreads();
      if (!SPLIT || reduce_splits(ct)) epilogue(ct, par, (pos + NBUF - 1) % NBUF);
      __syncthreads();
    } else {
      for (int st = ct.s0; st < ct.s1; ++st, ++pos) {
        unsigned short bval = 0;
        if (st == ct.s0) bval = bias_value(ct);  // issued before this stage's loads
        const bool more = ltile >= 0;
        const StageLoad nl = prep_stage(lt, lcc, lti, (pos + NBUF - 1) % NBUF);
        compute(pos % NBUF, more, nl);
        if (more) advance_load();  // after the pieces: they read this tile's halo offsets
        if (st == ct.s0 && tid < BN) bias_lds[par][tid] = bf16_to_f32(bval);
        // wait until stage pos+1 has landed (the NBUF-2 newer stages may stay
        // in flight); the barrier then publishes everyone's loads and the
        // bias, and retires this stage's LDS reads
        if (NBUF > 2 && more) wait_newer_stages();
        else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        barrier();
      }
      // the buffer of the last stage is idle until the next stage's loads are
      // issued: stage the outputs through it, then make sure every wave is
      // done with it before those loads go out
      if (!SPLIT || reduce_splits(ct)) epilogue(ct, par, (pos - 1) % NBUF);
      barrier();  // (the output stores may stay in flight)
    }
    par ^= 1;
    ctile = next_tile(ctile);
    if (ctile < 0) break;
    ct = decode(ctile);
  }
#endif
}

template <int BN, int TH, int WM, int WN, int KS, int CB, int NBUF, int OCC, bool WPK, bool SPLIT>
const void* mfma_kernel() {
  return reinterpret_cast<const void*>(&conv_bf16_mfma<BN, TH, WM, WN, KS, CB, NBUF, OCC, WPK, SPLIT>);
}

// Persistent launch with min(tiles, workgroups that fit) workgroups.
template <int BN, int TH, int WM, int WN, int KS, int CB, int NBUF, int OCC>
hipError_t launch_mfma(const ConvArgs& a, int64_t tiles, int cus, hipStream_t s) {
  constexpr int NT = WM * WN * 64;
  if (a.splits > 1) {  // (split calls run from the packed image only)
    if (!a.wpk) return hipErrorInvalidValue;
    return launch_persistent<&mfma_kernel<BN, TH, WM, WN, KS, CB, NBUF, OCC, true, true>>(a, tiles, cus, NT, s);
  }
  if (a.wpk) return launch_persistent<&mfma_kernel<BN, TH, WM, WN, KS, CB, NBUF, OCC, true, false>>(a, tiles, cus, NT, s);
  return launch_persistent<&mfma_kernel<BN, TH, WM, WN, KS, CB, NBUF, OCC, false, false>>(a, tiles, cus, NT, s);
}

template <int BN, int KS, int CB>
hipError_t pack_bf16(const ConvArgs& a, void* dst, hipStream_t s) {
  using T = WTile<BN, KS, CB>;
  const unsigned short* w = static_cast<const unsigned short*>(a.w);
  uint4* wpk = static_cast<uint4*>(dst);
  int cout = a.cout, kt = a.kt, cin = a.cin, nblk = a.nblk_n;
  int64_t total = int64_t(kt) * (cin / CB) * nblk * T::WSLOTS;
  const unsigned pgrid = unsigned(std::min<int64_t>((total + 255) / 256, 4096));
  void* pargs[] = {&w, &wpk, &cout, &kt, &cin, &nblk, &total};
  return hipLaunchKernel(reinterpret_cast<const void*>(&pack_weights<BN, KS, CB>), dim3(pgrid), dim3(256), pargs, 0, s);
}

}  // namespace

namespace cc3d {

hipError_t launch_mfma_family(int kernel_id, int cin_chunk, const ConvArgs& a, int64_t tiles, int cus,
                              hipStream_t s) {
  switch (kernel_id) {
    case CC3D_K_BF16_S3_N96_X2: return launch_mfma<96, 8, 4, 1, 3, 16, 2, 2>(a, tiles, cus, s);
    case CC3D_K_BF16_S3_N32: return launch_mfma<32, 8, 4, 1, 3, 16, 3, 2>(a, tiles, cus, s);
    case CC3D_K_BF16_S1_N192:
      if (cin_chunk == 64) return launch_mfma<192, 8, 2, 2, 1, 64, 2, 1>(a, tiles, cus, s);
      return launch_mfma<192, 8, 2, 2, 1, 32, 3, 1>(a, tiles, cus, s);
    case CC3D_K_BF16_S1_N32:
      if (cin_chunk == 64) return launch_mfma<32, 8, 4, 1, 1, 64, 3, 1>(a, tiles, cus, s);
      if (cin_chunk == 32) return launch_mfma<32, 8, 4, 1, 1, 32, 3, 2>(a, tiles, cus, s);
      return launch_mfma<32, 8, 4, 1, 1, 16, 3, 2>(a, tiles, cus, s);
  }
  return hipErrorInvalidValue;
}

hipError_t pack_stage_weights(int block_n, int ks, int cin_chunk, const ConvArgs& a, void* dst, hipStream_t s) {
  if (ks == 3 && cin_chunk == 16) {
    if (block_n == 96) return pack_bf16<96, 3, 16>(a, dst, s);
    if (block_n == 64) return pack_bf16<64, 3, 16>(a, dst, s);
    if (block_n == 32) return pack_bf16<32, 3, 16>(a, dst, s);
  }
  if (ks == 1 && block_n == 192) {
    if (cin_chunk == 64) return pack_bf16<192, 1, 64>(a, dst, s);
    if (cin_chunk == 32) return pack_bf16<192, 1, 32>(a, dst, s);
  }
  if (ks == 1 && block_n == 32) {
    if (cin_chunk == 64) return pack_bf16<32, 1, 64>(a, dst, s);
    if (cin_chunk == 32) return pack_bf16<32, 1, 32>(a, dst, s);
    if (cin_chunk == 16) return pack_bf16<32, 1, 16>(a, dst, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace cc3d
