// conv_bf16_gen (any spatial kernel size, stride, dilation and padding),
// conv_f32_direct (the fp32 path) and copy_tail_frames (the cache-out).
#include "cc3d_device.h"

namespace {
// bf16 kernel for any spatial kernel size, stride, dilation and padding
// (k_t <= 4, C_in % 16 == 0): an implicit GEMM over stages (active temporal
// tap, spatial tap, 32-channel chunk).  A stage gathers, for every output
// pixel of the tile, the 16-byte channel pieces of the input pixel that tap
// reads, straight into LDS (the buffer range check writes zeros for the
// padding and for channels past C_in), and the 32 x 32 weight block from W
// as the caller stores it ([C_out][k_t][k_h][k_w][C_in]).  No
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
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(a.w), 0, w_bytes, 0x00020000);
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

}  // namespace

namespace cc3d {

// One workgroup per tile.
hipError_t launch_gen_family(int kernel_id, const ConvArgs& a, int64_t tiles, hipStream_t s) {
  if (kernel_id == CC3D_K_BF16_GEN_N64) return launch_conv(reinterpret_cast<const void*>(&conv_bf16_gen<64>), a, tiles, s);
  if (kernel_id == CC3D_K_BF16_GEN_N96) return launch_conv(reinterpret_cast<const void*>(&conv_bf16_gen<96>), a, tiles, s);
  return hipErrorInvalidValue;
}

hipError_t launch_f32_direct(const ConvArgs& a, int64_t tiles, hipStream_t s) {
  return launch_conv(reinterpret_cast<const void*>(&conv_f32_direct), a, tiles, s);
}

hipError_t launch_copy_tail(const void* x, const void* cache, void* dst, int64_t frame_bytes, int n, int tx, int tc,
                            int frames, bool vec16, hipStream_t s) {
  const int64_t units = vec16 ? frame_bytes / 16 : frame_bytes;
  const int total = n * frames;
  const unsigned gx = unsigned(std::max<int64_t>(1, std::min<int64_t>((units + 1023) / 1024, 2048)));
  const unsigned gy = unsigned(std::min(total, 65535));
  const unsigned char* xp = static_cast<const unsigned char*>(x);
  const unsigned char* cp = static_cast<const unsigned char*>(cache);
  unsigned char* dp = static_cast<unsigned char*>(dst);
  int64_t fb = frame_bytes;
  int v16 = vec16 ? 1 : 0, L = frames;
  void* args[] = {&xp, &cp, &dp, &fb, &n, &tx, &tc, &L, &v16};
  return hipLaunchKernel(reinterpret_cast<const void*>(&copy_tail_frames), dim3(gx, gy), dim3(256), args, 0, s);
}

}  // namespace cc3d
