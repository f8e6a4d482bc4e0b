// conv_bf16_s1rd: the 1x1 / (k_t,1,1) convs (temporal-only: no spatial
// neighbourhood, so the K reduction is a plain GEMM over active taps x C_in
// per output pixel; lowering section of "Cache-Aware Conv3D Lowering Across
// Embedded World-Model Decoders").
//
// Tile: 256 consecutive pixels of one output frame (the frame is flattened:
// without a spatial halo, rows do not matter) x 192 output channels.  Four
// waves, each 64 pixels x all 192 channels (4 x 12 MFMA blocks of 16x16,
// fp32 accumulators).  A stage is one active tap x 64 input channels.
//
// Operand paths.  The pixel operand of a 16x16x32 MFMA lane is 8 consecutive
// input channels of one pixel -- 16 contiguous bytes of the channels-last
// frame -- and the four lanes of a pixel hold 32 consecutive channels, so
// each wave loads its own pixels from memory straight into registers, with
// no LDS round trip and no barrier on them; the register file is the
// pipeline buffer (D stages in flight, 32 VGPRs each).  One load instruction
// covers 16 pixels x 64 contiguous bytes: half a cache line per pixel (the
// 32x32x16 operand, 32 pixels x 32 bytes, costs the address unit twice the
// cache-line lookups per byte, and that path is what bounds this kernel).  The weights (shared
// by the four waves) stream into LDS with direct-to-LDS loads from the
// stage-ordered packed image (or gathered from W as stored), one 24 KB stage
// tile per LDS buffer.
#include "cc3d_device.h"

namespace {

typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));

template <bool WPK, int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void conv_bf16_s1rd(ConvArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)  // the host pass only needs the launch stub
  constexpr int BN = 192, CB = 64, NT = 256, TP = 256;
  constexpr int CW = BN / 16;             // 16-channel MFMA blocks (all of them, per wave)
  constexpr int RB = 4;                   // 16-pixel MFMA blocks per wave
  constexpr int KK = CB / 32;             // MFMA k-steps per stage
  using WT = WTile<BN, 1, CB>;            // slot q*PLANE + co: W[co][q*8 .. q*8+8) of the stage
  constexpr int WIT = WT::WSLOTS / NT;    // weight slots per thread per stage
  constexpr int XL = RB * KK;             // pixel loads per lane per stage
  constexpr int LPS = XL + WIT;           // vector-memory instructions per wave per stage
  static_assert(WT::WSLOTS % NT == 0 && WT::WCH == WT::WSLOTS, "whole weight tile per stage");
  static_assert(D >= 2 && D <= 4, "stage depth");
  constexpr int OOB = int(0x80000000u);

  __shared__ uint4 wl0[WT::WSLOTS];
  __shared__ uint4 wl1[WT::WSLOTS];
  __shared__ uint4 wl2[D > 2 ? WT::WSLOTS : 1];
  __shared__ uint4 wl3[D > 3 ? WT::WSLOTS : 1];
  __shared__ float bias_lds[2][BN];
  // (separate arrays, indexed statically, so that the compiler sees that a
  // direct-to-LDS load into one buffer does not alias reads of another)
  auto wbuf = [&](auto J) -> uint4* {
    constexpr int j = decltype(J)::value;
    if constexpr (j == 0) return wl0;
    else if constexpr (j == 1) return wl1;
    else if constexpr (j == 2) return wl2;
    else return wl3;
  };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, l16 = lane & 15;  // MFMA lane: k (or row) quarter, column

  // Persistent schedule: workgroup b runs on XCD b % 8; each XCD owns one
  // contiguous range of tiles.  Tile order: output frame fastest, then the
  // channel block, then the pixel block, then the batch item, so the four
  // channel blocks of one pixel block -- which read the same pixels -- and
  // the output frames that share source frames run together in one L2.
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int nblk_here = (int(gridDim.x) >> 3) + (xcd < int(gridDim.x & 7) ? 1 : 0);
  const int tq = a.ntiles >> 3, tr = a.ntiles & 7;
  const int t_begin = xcd * tq + min(xcd, tr);
  const int t_end = t_begin + tq + (xcd < tr ? 1 : 0);
  const int first = t_begin + slot;
  if (first >= t_end) return;  // uniform over the workgroup
  auto next_tile = [&](int t) { return t + nblk_here < t_end ? t + nblk_here : -1; };

  const int P = a.h * a.wd;               // pixels per frame (= output pixels: 1x1, stride 1)
  const int nch = a.cin / CB;
  const int64_t frame_el = int64_t(P) * a.cin;
  const int frame_bytes = int(frame_el * 2);
  const unsigned short* __restrict__ xs = static_cast<const unsigned short*>(a.x);
  const unsigned short* __restrict__ cs = static_cast<const unsigned short*>(a.cache);
  const unsigned char* __restrict__ wsrc = static_cast<const unsigned char*>(WPK ? a.wpk : a.w);
  const int64_t w_bytes = int64_t(a.cout) * a.kt * a.cin * 2;
  const unsigned short* __restrict__ bs = static_cast<const unsigned short*>(a.b);
  unsigned short* __restrict__ os = static_cast<unsigned short*>(a.out);

  // Tile t: output frame o of batch item nn, pixels [p0, p0 + 256), output
  // channels [n0, n0 + 192); its active taps read source frames z_i of
  // Z = [cache; x]; nst = active taps x channel chunks stages, tap major.
  struct Tile {
    int o, nn, p0, n0, nact, nst;
    int k0, k1, k2, k3;
    int z0, z1, z2, z3;
  };
  auto decode = [&](int t) {
    Tile c;
    c.o = t % a.to;
    t /= a.to;
    c.n0 = (t % a.nblk_n) * BN;
    t /= a.nblk_n;
    c.p0 = (t % a.tiles_x) * TP;
    c.nn = t / a.tiles_x;
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
    c.nst = c.nact * nch;
    return c;
  };
  auto pick = [](int i, int v0, int v1, int v2, int v3) { return i == 0 ? v0 : i == 1 ? v1 : i == 2 ? v2 : v3; };

  // weight slot offsets of this thread (slot it*256 + tid of a stage tile)
  int woff[WIT];
#pragma unroll
  for (int it = 0; it < WIT; ++it)
    woff[it] = WPK ? (it * NT + tid) * 16 : w_gather_offset<BN, 1, CB>(it * NT + tid, a.kt, a.cin);

  // ---- load cursor: the flattened (tile, stage) sequence, D - 1 stages
  // ahead of the compute cursor ----
  int ltile = first, lst = 0;
  Tile lt = decode(ltile);
  int xoff[RB];  // byte offset in the frame of this lane's pixel rows (past the frame: zeros)
  auto set_xoff = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int px = lt.p0 + wave * 64 + rb * 16 + l16;
      xoff[rb] = px < P ? (px * a.cin + g * 8) * 2 : OOB;
    }
  };
  auto skip_empty = [&]() __attribute__((always_inline)) {  // move the load cursor to a tile with stages
    while (ltile >= 0 && lt.nst == 0) {
      ltile = next_tile(ltile);
      if (ltile >= 0) lt = decode(ltile);
    }
    lst = 0;
    if (ltile >= 0) set_xoff();
  };
  skip_empty();

  struct StageSrc {
    __amdgpu_buffer_rsrc_t xr, wr;
    int xch;  // byte offset of the stage's first channel
  };
  // The sources of the load cursor's stage; past the last stage, sources
  // with no bytes in range (their loads return zeros and touch no memory),
  // so that every step issues the same LPS loads and the waits below can be
  // fixed counts.
  auto prep = [&]() __attribute__((always_inline)) {
    if (ltile < 0) {
      StageSrc s;
      s.xr = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(uniform_ptr(xs)), 0, 0, 0x00020000);
      s.wr = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(uniform_ptr(wsrc)), 0, 0, 0x00020000);
      s.xch = 0;
      return s;
    }
    const int ti = lst / nch, cc = lst - (lst / nch) * nch;
    const int z = pick(ti, lt.z0, lt.z1, lt.z2, lt.z3), k = pick(ti, lt.k0, lt.k1, lt.k2, lt.k3);
    const unsigned short* fp = z < a.tc ? cs + (int64_t(lt.nn) * a.tc + z) * frame_el
                                        : xs + (int64_t(lt.nn) * a.tx + (z - a.tc)) * frame_el;
    StageSrc s;
    s.xr = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(uniform_ptr(fp)), 0, frame_bytes, 0x00020000);
    s.xch = __builtin_amdgcn_readfirstlane(cc * CB * 2);
    const int nb = lt.n0 / BN;
    if constexpr (WPK) {
      const unsigned char* wp = wsrc + ((int64_t(nb) * nch + cc) * a.kt + k) * (WT::WSLOTS * 16);
      s.wr = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(uniform_ptr(wp)), 0, WT::WSLOTS * 16, 0x00020000);
    } else {
      const int64_t off = ((int64_t(nb) * BN * a.kt + k) * a.cin + cc * CB) * 2;
      s.wr = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(uniform_ptr(wsrc + off)), 0,
                                               __builtin_amdgcn_readfirstlane(int(w_bytes - off)), 0x00020000);
    }
    return s;
  };
  auto advance_load = [&]() __attribute__((always_inline)) {
    if (ltile < 0) return;
    if (++lst == lt.nst) {
      ltile = next_tile(ltile);
      if (ltile >= 0) lt = decode(ltile);
      skip_empty();
    }
  };

  // pixel operand ring: xr[j][rb][kk] = channels kk*32 + g*8 .. +8 of the
  // stage, for 16-pixel block rb of this wave
  u32x4_t xr[D][RB][KK];
  // piece p (0 .. LPS-1) of a stage's loads into buffer J: weight slots
  // first, then pixel loads
  auto issue_piece = [&](auto J, const StageSrc& s, int p) __attribute__((always_inline)) {
    constexpr int j = decltype(J)::value;
    if (p < WIT) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(s.wr, (__attribute__((address_space(3))) void*)(wbuf(J) + p * NT + wave * 64),
                                               16, woff[p], 0, 0, 0);
    } else {
      const int q = p - WIT, rb = q / KK, kk = q % KK;
      xr[j][rb][kk] = __builtin_amdgcn_raw_buffer_load_b128(s.xr, xoff[rb], s.xch + kk * 64, 0);
    }
  };

  f32x4_t acc[CW][RB];
  auto zero_acc = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int c = 0; c < CW; ++c)
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[c][rb][v] = 0.f;
  };

  // One stage: KK k-steps x CW channel blocks = NG groups of RB MFMAs.  The
  // weight fragment of a group (one ds_read of 16 bytes per lane) is read
  // from LDS two groups ahead, so its latency hides behind two groups of
  // MFMAs while only three fragments are live.  The next loads (`nxt`, into
  // buffer (J + D - 1) % D) are spread over the groups.
  auto compute = [&](auto J, const StageSrc& nxt) __attribute__((always_inline)) {
    constexpr int j = decltype(J)::value;
    constexpr int jn = (j + D - 1) % D;
    constexpr int NG = KK * CW;
    const uint4* wb = wbuf(J);
    auto read_w = [&](int i) __attribute__((always_inline)) {
      const int kk = i / CW, c = i % CW;
      return __builtin_bit_cast(bf16x8_t, wb[(kk * 4 + g) * WT::PLANE + c * 16 + l16]);
    };
    bf16x8_t wf[3];
    wf[0] = read_w(0);
    wf[1] = read_w(1);
#pragma unroll
    for (int i = 0; i < NG; ++i) {
      if (i + 2 < NG) wf[(i + 2) % 3] = read_w(i + 2);
      __builtin_amdgcn_sched_barrier(0);
      const int kk = i / CW, c = i % CW;
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
        acc[c][rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[i % 3], __builtin_bit_cast(bf16x8_t, xr[j][rb][kk]),
                                                             acc[c][rb], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int p = 0; p < LPS; ++p)
        if (p * NG / LPS == i) issue_piece(std::integral_constant<int, jn>{}, nxt, p);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Epilogue: + bias once (fp32), round to nearest even, bf16 stores.  The
  // accumulators are read out of their AGPRs one element per store (inline
  // v_accvgpr_read), so that the compiler does not copy all 192 of them to
  // VGPRs at once while the next stages' pixels occupy 96 VGPRs.  The
  // lane holding pixel l16 of a 16-pixel block has channels g*4 .. g*4+3 of
  // each 16-channel block: 4 consecutive channels, one 8-byte store each.  Stores to pixels past the frame fall outside the
  // buffer's range and are dropped, so every wave issues exactly ST stores.
  auto epilogue = [&](const Tile& c, int par) __attribute__((always_inline)) {
    unsigned short* ob = os + ((int64_t(c.nn) * a.to + c.o) * P) * a.cout + c.n0;
    const __amdgpu_buffer_rsrc_t orc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<void*>(uniform_ptr(ob)), 0, __builtin_amdgcn_readfirstlane(int((int64_t(P) * a.cout - c.n0) * 2)),
        0x00020000);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int px = c.p0 + wave * 64 + rb * 16 + l16;
      const int ooff = px < P ? (px * a.cout + g * 4) * 2 : OOB;
#pragma unroll
      for (int q = 0; q < CW; ++q) {
        const int cl = q * 16;  // + g*4 in ooff
        const float4 bv = *reinterpret_cast<const float4*>(&bias_lds[par][cl + g * 4]);
        float f[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)  // (read from the accumulator registers one at a time: see above)
          asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(f[e]) : "a"(acc[q][rb][e]));
        const unsigned lo = pack_bf16x2(f[0] + bv.x, f[1] + bv.y);
        const unsigned hi = pack_bf16x2(f[2] + bv.z, f[3] + bv.w);
        const u32x2_t v = {lo, hi};
        __builtin_amdgcn_raw_buffer_store_b64(v, orc, ooff, cl * 2, 0);
        // (one store at a time: converting all 96 pairs first would need
        // 192 more VGPRs while the next stages' pixels are in flight)
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };
  auto load_bias = [&](const Tile& c, int par) __attribute__((always_inline)) {
    if (tid < BN) bias_lds[par][tid] = a.has_bias ? bf16_to_f32(bs[c.n0 + tid]) : 0.f;
  };

  constexpr auto vm_imm = [](int n) { return ((n >> 4) << 14) | 0x0F70 | (n & 15); };
  // Wait until at most N of this wave's vector-memory instructions are in
  // flight, then a workgroup barrier that also retires the LDS reads.
#define CC3D_S1_WAIT_BARRIER(N)                                  \
  do {                                                           \
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");     \
    __builtin_amdgcn_s_waitcnt(vm_imm(N));                       \
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");           \
    __builtin_amdgcn_s_barrier();                                \
    asm volatile("" ::: "memory");                               \
  } while (0)

  // ---- prologue: positions 0 .. D-2 ----
  static_for_while<0, D - 1>([&](auto J) __attribute__((always_inline)) {
    const StageSrc s = prep();
#pragma unroll
    for (int p = 0; p < LPS; ++p) issue_piece(J, s, p);
    advance_load();
    return true;
  });
  CC3D_S1_WAIT_BARRIER(LPS * (D - 2));

  // ---- compute: tiles in turn; a tile's stages in groups of D (D divides
  // the channel chunks per tap, so every tile's stage count is a multiple of
  // D, and stage s of any tile sits in buffer s % D) ----
  int par = 0;
  for (int ctile = first; ctile >= 0; ctile = next_tile(ctile), par ^= 1) {
    const Tile ct = decode(ctile);
    load_bias(ct, par);  // read by this tile's epilogue, after at least one barrier
    if (ct.nst == 0) {   // no active tap: the output is the bias alone
      __syncthreads();
      zero_acc();
      epilogue(ct, par);
      continue;
    }
    zero_acc();
    for (int cst = 0; cst < ct.nst; cst += D) {
      static_for_while<0, D>([&](auto J) __attribute__((always_inline)) {
        // compute the stage in buffer J and issue the one D - 1 stages
        // ahead; then wait for the next stage (the D - 2 after it stay in
        // flight; an epilogue's stores, issued after them, are waited for)
        const StageSrc nxt = prep();
        compute(J, nxt);
        advance_load();
        CC3D_S1_WAIT_BARRIER(LPS * (D - 2));
        return true;
      });
    }
    epilogue(ct, par);
  }
  // (no direct-to-LDS load may be in flight when the workgroup ends)
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#undef CC3D_S1_WAIT_BARRIER
#endif
}

template <bool WPK, int D>
const void* s1rd_kernel() {
  return reinterpret_cast<const void*>(&conv_bf16_s1rd<WPK, D>);
}

}  // namespace

namespace cc3d {

// The stage depth D must divide the 64-channel chunks per tap (C_in / 64):
// 3 where it does, else 4, else 2.
hipError_t launch_s1rd(const ConvArgs& a, int64_t tiles, int cus, hipStream_t s) {
  if (a.cin % 64 != 0 || a.cout % 192 != 0 || a.kh != 1 || a.kw != 1) return hipErrorInvalidValue;
  const int nch = a.cin / 64;
  if (nch % 3 == 0) {
    if (a.wpk) return launch_persistent<&s1rd_kernel<true, 3>>(a, tiles, cus, 256, s);
    return launch_persistent<&s1rd_kernel<false, 3>>(a, tiles, cus, 256, s);
  }
  if (nch % 4 == 0) {
    if (a.wpk) return launch_persistent<&s1rd_kernel<true, 4>>(a, tiles, cus, 256, s);
    return launch_persistent<&s1rd_kernel<false, 4>>(a, tiles, cus, 256, s);
  }
  if (nch % 2 == 0) {
    if (a.wpk) return launch_persistent<&s1rd_kernel<true, 2>>(a, tiles, cus, 256, s);
    return launch_persistent<&s1rd_kernel<false, 2>>(a, tiles, cus, 256, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace cc3d
