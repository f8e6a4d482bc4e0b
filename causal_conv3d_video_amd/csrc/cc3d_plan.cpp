// Host-side planner for the cached causal Conv3D: contract check, the
// temporal tap intervals of the lowering (cache-augmented source Z = [C; X],
// p_l = p_base - |C|, delta_k = k*d_t - p_l, equal-length output and source
// intervals; "Cache-Aware Conv3D Lowering Across Embedded World-Model
// Decoders", lowering section), and the kernel tile choice.  No device calls.
#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <new>
#include <string>

#include "cc3d_internal.h"

namespace cc3d {
std::atomic<uint64_t> g_fast_path{0}, g_unsupported{0}, g_invalid{0}, g_device_error{0};
}

namespace {

int64_t floordiv(int64_t num, int64_t den) {
  int64_t q = num / den;
  if ((num % den != 0) && (num < 0)) q -= 1;
  return q;
}
int64_t ceildiv(int64_t num, int64_t den) { return -floordiv(-num, den); }

cc3d_status_t refuse(cc3d_status_t s) {
  if (s == CC3D_ERR_UNSUPPORTED) cc3d::g_unsupported.fetch_add(1, std::memory_order_relaxed);
  if (s == CC3D_ERR_INVALID_ARG) cc3d::g_invalid.fetch_add(1, std::memory_order_relaxed);
  return s;
}

struct Variant {
  cc3d_kernel_id id;
  int tile_h, tile_w, block_n, cin_chunk;
  const char* name;
};

// bf16 kernel variants.  The patch width is 32 output columns (one MFMA
// operand block of pixels); rows and channel tiles trade accumulator
// registers against LDS and L2 traffic per MFMA.  variant_for() gives the
// named variant's geometry for a call, or nothing when it cannot run it.
// The halo-staged kernels' spatial envelope: 3x3 "same" or 1x1, stride and
// dilation 1.
bool same_spatial(const cc3d_desc_t& d) {
  return d.k_h == d.k_w && (d.k_h == 1 || d.k_h == 3) && d.s_h == 1 && d.s_w == 1 && d.d_h == 1 && d.d_w == 1 &&
         d.p_h == (d.k_h - 1) / 2 && d.p_w == (d.k_w - 1) / 2;
}

// Compute units of the target (MI355X); the split heuristic sizes work for
// them (the kernels themselves run on any count).
constexpr int kComputeUnits = 256;

// The few-output-channel kernel streams halo rows through patches of 4 to
// 16 output rows by 128 columns.
constexpr int kFewRowsMin = 4, kFewRowsMax = 16;
const char* const kFewNames[] = {"bf16_s3_few_p4x128",  "bf16_s3_few_p5x128",  "bf16_s3_few_p6x128",
                                 "bf16_s3_few_p7x128",  "bf16_s3_few_p8x128",  "bf16_s3_few_p9x128",
                                 "bf16_s3_few_p10x128", "bf16_s3_few_p11x128", "bf16_s3_few_p12x128",
                                 "bf16_s3_few_p13x128", "bf16_s3_few_p14x128", "bf16_s3_few_p15x128",
                                 "bf16_s3_few_p16x128"};
static_assert(sizeof kFewNames / sizeof kFewNames[0] == kFewRowsMax - kFewRowsMin + 1, "few-kernel names");

// Patch height of the few-output-channel kernel: each compute unit (256 on
// the target) runs ceil(patches / 256) patches of rows + 2 halo rows per
// frame; take the height with the fewest halo rows per unit, the tallest on
// ties (less halo re-read in total).
int few_rows(const cc3d_desc_t& d) {
  const int64_t strips = int64_t(d.n) * ((d.w + 127) / 128);
  int best = kFewRowsMax;
  int64_t best_cost = -1;
  for (int r = kFewRowsMax; r >= kFewRowsMin; --r) {
    const int64_t rounds = (strips * ((d.h + r - 1) / r) + 255) / 256;
    const int64_t cost = rounds * (r + 2);
    if (best_cost < 0 || cost < best_cost) {
      best = r;
      best_cost = cost;
    }
  }
  return best;
}

// 3x3 taps at spatial dilation 2 with the padding that keeps the map size
// (2), unit spatial stride: the dilated group-staged kernel's envelope.
bool dilated_same(const cc3d_desc_t& d) {
  return d.k_h == 3 && d.k_w == 3 && d.s_h == 1 && d.s_w == 1 && d.d_h == 2 && d.d_w == 2 && d.p_h == 2 &&
         d.p_w == 2;
}

// 3x3 taps at spatial stride 2 with padding 1, no spatial dilation (the
// encoder's downsampling conv): the strided group-staged kernel's envelope.
bool strided_3x3(const cc3d_desc_t& d) {
  return d.k_h == 3 && d.k_w == 3 && d.s_h == 2 && d.s_w == 2 && d.d_h == 1 && d.d_w == 1 && d.p_h == 1 &&
         d.p_w == 1;
}

// Fingerprint of a packed weight image: plans whose fingerprints (and
// packed_weight_bytes) are equal read the same image, whatever their frame
// counts, cache depth and map size.  FNV-1a over the fields that shape it.
uint64_t layout_fingerprint(int32_t kind, int32_t block_n, int32_t ks, int32_t cin_chunk, const cc3d_desc_t& d) {
  const int32_t f[] = {kind, block_n, ks, cin_chunk, d.c_out, d.c_in, d.k_t, d.k_h, d.k_w};
  uint64_t h = 1469598103934665603ull;
  for (int32_t v : f)
    for (int i = 0; i < 4; ++i) {
      h ^= uint64_t((uint32_t(v) >> (8 * i)) & 0xFF);
      h *= 1099511628211ull;
    }
  return h;
}

bool variant_for(const cc3d_desc_t& d, const char* name, Variant* v) {
  const std::string n(name);
  if (n == "bf16_gen_n64_p8x32") {  // any spatial parameters
    *v = {CC3D_K_BF16_GEN_N64, 8, 32, 64, 32, "bf16_gen_n64_p8x32"};
    return true;
  }
  if (n == "bf16_gen_n96_p8x32") {  // any spatial parameters, C_out % 96 == 0
    *v = {CC3D_K_BF16_GEN_N96, 8, 32, 96, 32, "bf16_gen_n96_p8x32"};
    return d.c_out % 96 == 0;
  }
  if (n == "bf16_s3d2_n64_p16x32_g32") {  // 3x3 "same" at spatial dilation 2
    *v = {CC3D_K_BF16_S3D2_N64_G32W8, 16, 32, 64, 16, "bf16_s3d2_n64_p16x32_g32"};
    return dilated_same(d) && d.c_out % 64 == 0 && d.c_in % 32 == 0;
  }
  if (n == "bf16_s3s2_n96_p4x32_g32") {  // 3x3 at spatial stride 2, padding 1
    *v = {CC3D_K_BF16_S3S2_N96_G32W4, 4, 32, 96, 16, "bf16_s3s2_n96_p4x32_g32"};
    return strided_3x3(d) && d.c_out % 96 == 0 && d.c_in % 32 == 0;
  }
  if (n == "bf16_s3s2_n64_p4x32_g32") {  // the same with 64 output channels per tile
    *v = {CC3D_K_BF16_S3S2_N64_G32W8, 4, 32, 64, 16, "bf16_s3s2_n64_p4x32_g32"};
    return strided_3x3(d) && d.c_out % 64 == 0 && d.c_in % 32 == 0;
  }
  if (!same_spatial(d)) return false;
  const bool s3 = d.k_h == 3;
  const int cb = d.c_in % 64 == 0 ? 64 : d.c_in % 32 == 0 ? 32 : 16;
  if (n == "bf16_s3_n64_p24x32_g32") {
    *v = {CC3D_K_BF16_S3_N64_G32W8, 24, 32, 64, 16, "bf16_s3_n64_p24x32_g32"};
    return s3 && d.c_out % 64 == 0 && d.c_in % 32 == 0;
  }
  if (n == "bf16_s3_n96_p16x32_g32") {
    *v = {CC3D_K_BF16_S3_N96_G32W8, 16, 32, 96, 16, "bf16_s3_n96_p16x32_g32"};
    return s3 && d.c_out % 96 == 0 && d.c_in % 32 == 0;
  }
  if (n == "bf16_s3_n96_p8x32_x2") {
    *v = {CC3D_K_BF16_S3_N96_X2, 8, 32, 96, 16, "bf16_s3_n96_p8x32_x2"};
    return s3 && d.c_out % 96 == 0;
  }
  for (int r = kFewRowsMin; r <= kFewRowsMax; ++r)
    if (n == kFewNames[r - kFewRowsMin]) {
      *v = {CC3D_K_BF16_S3_FEW, r, 128, d.c_out, 32, kFewNames[r - kFewRowsMin]};
      return s3 && d.k_t == 3 && d.d_t == 1 && d.s_t == 1 && d.c_out <= 5 && d.c_in % 32 == 0 && d.c_in <= 96;
    }
  if (n == "bf16_s3_n32_p8x32") {
    *v = {CC3D_K_BF16_S3_N32, 8, 32, 32, 16, "bf16_s3_n32_p8x32"};
    return s3;
  }
  // the 192-channel tile stages at least 32 input channels (its stage buffer
  // must also hold the epilogue's output staging)
  if (n == "bf16_s1_n192_p8x32") {
    *v = {CC3D_K_BF16_S1_N192, 8, 32, 192, cb, "bf16_s1_n192_p8x32"};
    return !s3 && d.c_out % 192 == 0 && cb >= 32;
  }
  // the register-direct 1x1 kernel: its stage depth (2, 3 or 4) must divide
  // the 64-channel chunks per tap
  if (n == "bf16_s1_n192_p256_rd") {
    *v = {CC3D_K_BF16_S1_N192_RD, 1, 256, 192, 64, "bf16_s1_n192_p256_rd"};
    return !s3 && d.c_out % 192 == 0 && d.c_in % 64 == 0 && ((d.c_in / 64) % 2 == 0 || (d.c_in / 64) % 3 == 0);
  }
  if (n == "bf16_s1_n32_p8x32") {
    *v = {CC3D_K_BF16_S1_N32, 8, 32, 32, cb, "bf16_s1_n32_p8x32"};
    return !s3;
  }
  return false;
}

// Default choice.  Large 3x3 maps take the group-staged kernel: the halo
// staged by 32 channels, one workgroup per compute unit (its 64-wide tile
// from 1.5 rounds of 256 tiles: 384->384 at 120x208 with 2 frames, 420
// tiles, 347 vs 383 us on the two-workgroup kernel; 960 tiles at 180x320,
// 8% faster).  Where C_out is a multiple of 64 its
// 24x32-pixel x 64-channel tile (three rows per wave) reads 15% fewer LDS
// bytes per MFMA than the 16x32 x 96 one and runs 1-3% faster.  Small maps
// keep two smaller workgroups per compute unit so that every unit gets
// tiles.  causal_conv3d_plan_autotune times the alternatives.
const char* default_variant(const cc3d_desc_t& d) {
  if (!same_spatial(d)) {
    if (dilated_same(d) && d.c_out % 64 == 0 && d.c_in % 32 == 0) return "bf16_s3d2_n64_p16x32_g32";
    // (the 96-wide tile has 3 MFMAs per spatial tap and wave, the 64-wide one 2)
    if (strided_3x3(d) && d.c_out % 96 == 0 && d.c_in % 32 == 0) return "bf16_s3s2_n96_p4x32_g32";
    if (strided_3x3(d) && d.c_out % 64 == 0 && d.c_in % 32 == 0) return "bf16_s3s2_n64_p4x32_g32";
    return d.c_out % 96 == 0 ? "bf16_gen_n96_p8x32" : "bf16_gen_n64_p8x32";
  }
  if (d.k_h == 3) {
    if (d.c_out % 64 == 0 && d.c_in % 32 == 0) {
      const int64_t tiles64 =
          int64_t(d.n) * ((d.h + 23) / 24) * ((d.w + 31) / 32) * (d.c_out / 64) * std::max(1, d.t_x);
      if (tiles64 >= 384) return "bf16_s3_n64_p24x32_g32";
    }
    if (d.c_out % 96 == 0) {
      const int64_t big_tiles = int64_t(d.n) * ((d.h + 15) / 16) * ((d.w + 31) / 32) * (d.c_out / 96) *
                                std::max(1, d.t_x);
      if (d.c_in % 32 == 0 && big_tiles >= 768) return "bf16_s3_n96_p16x32_g32";
      // maps so small that the 96-wide tiles leave three quarters of the
      // compute units idle take 32-wide tiles (three times as many; 384->384
      // at 30x52: 32 vs 58 us, 48->384: 15 vs 21 us)
      const int64_t x2_tiles = int64_t(d.n) * ((d.h + 7) / 8) * ((d.w + 31) / 32) * (d.c_out / 96) *
                               std::max(1, d.t_x);
      if (x2_tiles < 64) return "bf16_s3_n32_p8x32";
      // where the 24-row tiles pad the map no more than the 8-row ones and
      // fill at most half the compute units, the group-staged tile in split
      // units (packed calls with a workspace; 384->384 at 90x160, 1 frame +
      // 2 cached: 109 vs 111 us back to back, 118 vs 128 us launched alone)
      if (d.c_out % 64 == 0 && d.c_in % 32 == 0 && (d.h + 23) / 24 * 24 == (d.h + 7) / 8 * 8) {
        const int64_t tiles64 =
            int64_t(d.n) * ((d.h + 23) / 24) * ((d.w + 31) / 32) * (d.c_out / 64) * std::max(1, d.t_x);
        if (tiles64 * 2 <= kComputeUnits) return "bf16_s3_n64_p24x32_g32";
      }
      return "bf16_s3_n96_p8x32_x2";
    }
    if (d.c_out <= 5 && d.k_t == 3 && d.d_t == 1 && d.s_t == 1 && d.c_in % 32 == 0 && d.c_in <= 96)
      return kFewNames[few_rows(d) - kFewRowsMin];
    return "bf16_s3_n32_p8x32";
  }
  const int cb = d.c_in % 64 == 0 ? 64 : d.c_in % 32 == 0 ? 32 : 16;
  // 1x1: the register-direct kernel where it applies (384->768 (3,1,1):
  // 281 vs 309 us at 180x320, 36 vs 39 us at 90x160; both kernels are bound
  // by the vector-memory address path, not by the matrix cores)
  // (maps with fewer than 64 of its tiles take the 32-wide tiles, as above:
  // 384->768 at 30x52, 20 vs 31 us)
  const int nch = d.c_in / 64;
  const int64_t rd_tiles = int64_t(d.n) * std::max(1, d.t_x) * ((int64_t(d.h) * d.w + 255) / 256) * (d.c_out / 192);
  if (d.c_out % 192 == 0 && cb == 64 && (nch % 2 == 0 || nch % 3 == 0) && rd_tiles >= 64)
    return "bf16_s1_n192_p256_rd";
  if (d.c_out % 192 == 0 && cb >= 32 && rd_tiles >= 64) return "bf16_s1_n192_p8x32";
  return "bf16_s1_n32_p8x32";
}

}  // namespace

namespace {

cc3d_status_t plan_impl(const cc3d_desc_t* desc, const char* kernel, cc3d_plan_t* out) {
  if (out) *out = nullptr;
  if (!desc || !out) return refuse(CC3D_ERR_INVALID_ARG);
  const cc3d_desc_t d = *desc;
  if (d.dtype != CC3D_F32 && d.dtype != CC3D_BF16) return refuse(CC3D_ERR_INVALID_ARG);
  if (d.n < 1 || d.c_in < 1 || d.c_out < 1 || d.h < 1 || d.w < 1 || d.t_x < 1 || d.t_cache < 0 ||
      d.k_t < 1 || d.k_h < 1 || d.k_w < 1 || d.s_t < 1 || d.s_h < 1 || d.s_w < 1 || d.d_t < 1 ||
      d.d_h < 1 || d.d_w < 1 || d.p_h < 0 || d.p_w < 0 || d.p_base < 0 || d.groups < 1 ||
      (d.has_bias != 0 && d.has_bias != 1))
    return refuse(CC3D_ERR_INVALID_ARG);
  // One group, as in the lowering's contract.  Temporal stride > 1 (the
  // encoder's downsampling convs, outside that contract) is supported: output
  // frame o reads source frame o*s_t + delta_k.
  if (d.groups != 1 || d.k_t > CC3D_MAX_KT) return refuse(CC3D_ERR_UNSUPPORTED);

  cc3d_plan_info_t in;
  std::memset(&in, 0, sizeof in);
  in.t_z = d.t_cache + d.t_x;
  in.p_l = d.p_base - d.t_cache;
  const int64_t t_out = floordiv(int64_t(in.t_z) + in.p_l - int64_t(d.d_t) * (d.k_t - 1) - 1, d.s_t) + 1;
  const int64_t h_out = floordiv(int64_t(d.h) + 2 * d.p_h - int64_t(d.d_h) * (d.k_h - 1) - 1, d.s_h) + 1;
  const int64_t w_out = floordiv(int64_t(d.w) + 2 * d.p_w - int64_t(d.d_w) * (d.k_w - 1) - 1, d.s_w) + 1;
  if (t_out < 1 || h_out < 1 || w_out < 1) return refuse(CC3D_ERR_INVALID_ARG);
  in.t_out = int32_t(t_out);
  in.h_out = int32_t(h_out);
  in.w_out = int32_t(w_out);
  in.t_cache_out = std::min(d.p_base, in.t_z);

  // Per-tap intervals: 0 <= o < T_o and 0 <= o*s_t + delta_k < |Z|.  With
  // unit stride the source frames are the interval [o_lo, o_hi) + delta_k,
  // of the same length; with s_t > 1 they are every s_t-th frame of
  // [src_lo, src_hi).
  int64_t active_pairs = 0;
  int64_t read_frames = 0;  // frames of Z read by at least one active tap
  for (int k = 0; k < d.k_t; ++k) {
    cc3d_tap_t& tp = in.taps[k];
    tp.delta = k * d.d_t - in.p_l;
    tp.o_lo = int32_t(std::max<int64_t>(0, ceildiv(-int64_t(tp.delta), d.s_t)));
    tp.o_hi = int32_t(std::min<int64_t>(in.t_out, ceildiv(int64_t(in.t_z) - tp.delta, d.s_t)));
    tp.active = tp.o_hi > tp.o_lo;
    if (!tp.active) tp.o_hi = tp.o_lo;
    tp.src_lo = tp.o_lo * d.s_t + tp.delta;
    tp.src_hi = tp.active ? (tp.o_hi - 1) * d.s_t + tp.delta + 1 : tp.src_lo;
    if (tp.active) {
      in.n_active_taps += 1;
      active_pairs += tp.o_hi - tp.o_lo;
    }
  }
  for (int32_t z = 0; z < in.t_z; ++z) {
    bool read = false;
    for (int k = 0; k < d.k_t; ++k) {
      const cc3d_tap_t& tp = in.taps[k];
      read = read || (tp.active && z >= tp.src_lo && z < tp.src_hi && (z - tp.src_lo) % d.s_t == 0);
    }
    read_frames += read;
  }

  const int elem = d.dtype == CC3D_BF16 ? 2 : 4;
  const double spatial = double(h_out) * w_out;
  const double mac_per_px = double(d.c_out) * d.c_in * d.k_h * d.k_w;
  in.flops_nominal = 2.0 * d.n * double(t_out) * spatial * mac_per_px * d.k_t;
  in.flops_active = 2.0 * d.n * double(active_pairs) * spatial * mac_per_px;
  const double frame_in = double(d.h) * d.w * d.c_in * elem;
  in.bytes_conv = d.n * double(read_frames) * frame_in +
                  double(d.c_out) * d.k_t * d.k_h * d.k_w * d.c_in * elem +
                  (d.has_bias ? double(d.c_out) * elem : 0.0) +
                  double(d.n) * t_out * spatial * d.c_out * elem;
  in.bytes_cache_out = 2.0 * d.n * in.t_cache_out * frame_in;

  auto* p = new (std::nothrow) cc3d_plan;
  if (!p) return CC3D_ERR_NO_MEMORY;
  p->d = d;
  p->elem = elem;
  const int64_t frame_el_in = int64_t(d.h) * d.w * d.c_in;
  p->x_bytes = int64_t(d.n) * d.t_x * frame_el_in * elem;
  p->cache_bytes = int64_t(d.n) * d.t_cache * frame_el_in * elem;
  p->w_bytes = int64_t(d.c_out) * d.k_t * d.k_h * d.k_w * d.c_in * elem;
  p->b_bytes = d.has_bias ? int64_t(d.c_out) * elem : 0;
  p->out_bytes = int64_t(d.n) * t_out * h_out * w_out * d.c_out * elem;
  p->cache_out_bytes = int64_t(d.n) * in.t_cache_out * frame_el_in * elem;

  if (d.dtype == CC3D_BF16) {
    // buffer-load offsets are 32-bit byte offsets within one frame / the weights
    const int64_t frame_bytes =
        std::max(int64_t(d.h) * d.w * std::max(d.c_in, d.c_out), h_out * w_out * d.c_out) * 2;
    const int64_t w_bytes = int64_t(d.c_out) * d.k_t * d.k_h * d.k_w * d.c_in * 2;
    if (d.c_in % 16 != 0 || d.k_t > 4 || frame_bytes >= (int64_t(1) << 31) || w_bytes >= (int64_t(1) << 31)) {
      delete p;
      return refuse(CC3D_ERR_UNSUPPORTED);
    }
    Variant v{};
    if (!variant_for(d, kernel ? kernel : default_variant(d), &v)) {
      delete p;
      return refuse(CC3D_ERR_UNSUPPORTED);
    }
    in.kernel_id = v.id;
    p->tile_h = v.tile_h;
    p->tile_w = v.tile_w;
    p->cin_chunk = v.cin_chunk;
    p->tiles_y = int32_t((h_out + v.tile_h - 1) / v.tile_h);
    p->tiles_x = int32_t((w_out + v.tile_w - 1) / v.tile_w);
    if (v.id == CC3D_K_BF16_S1_N192_RD) {  // tiles of the flattened frame
      p->tiles_y = 1;
      p->tiles_x = int32_t((h_out * w_out + v.tile_w - 1) / v.tile_w);
    }
    p->nblk_n = (d.c_out + v.block_n - 1) / v.block_n;
    in.block_m = v.tile_h * v.tile_w;
    in.block_n = v.block_n;
    // the few-channel kernel's patches run through every output frame
    in.tiles = int64_t(d.n) * (v.id == CC3D_K_BF16_S3_FEW ? 1 : t_out) * p->tiles_y * p->tiles_x * p->nblk_n;
    // Packed weight image: for the halo-staged kernels one stage tile of
    // 16-byte slots per (channel block, channel chunk, tap), in that order;
    // the few-channel and gather kernels read W's own layout, so theirs is a
    // copy of W.
    const int64_t ks = d.k_h;
    const int64_t slots = (int64_t(v.block_n) * ks * ks * (v.cin_chunk / 8) + 63) / 64 * 64;
    p->pack_kind = 1;
    in.packed_weight_bytes = int64_t(d.k_t) * (d.c_in / v.cin_chunk) * p->nblk_n * slots * 16;
    if (v.id == CC3D_K_BF16_S3_FEW || v.id == CC3D_K_BF16_GEN_N64 || v.id == CC3D_K_BF16_GEN_N96) {
      p->pack_kind = 2;
      in.packed_weight_bytes = w_bytes;
    }
    if (v.id == CC3D_K_BF16_S3_FEW) in.bytes_cache_out /= 2;  // written from the staged rows, not re-read
    in.weight_layout = layout_fingerprint(p->pack_kind, v.block_n, int32_t(ks), v.cin_chunk, d);
    // Split reduction (the two-workgroup and 1x1 kernels of conv_bf16_mfma;
    // causal_conv3d_forward_packed):
    // when a call's tiles would leave three quarters or more of the chip's
    // workgroup slots idle, each tile's K stages are divided among up to 16
    // units (at least 4 stages each) so that the slots fill.  Each unit
    // writes a tile of fp32 partials (block_m * block_n floats) to the
    // workspace, after an int per tile of arrival counters.  Fewer than 4
    // splits are not taken: the partial-sum traffic and the last arriver's
    // reduction then cost more than the idle slots.  (Measured on the
    // two-workgroup kernel: 384->384 at 30x52, 32 tiles, 16 splits, 109 ->
    // 89 us; at 90x160, 240 tiles, 2 splits gained nothing, and 48->384 at
    // 30x52, 32 tiles of 9 stages, 2 splits lost time.)
    in.splits = 1;
    if (v.id == CC3D_K_BF16_S3_N96_X2 || v.id == CC3D_K_BF16_S3_N32 || v.id == CC3D_K_BF16_S1_N192 ||
        v.id == CC3D_K_BF16_S1_N32) {
      const int wg_per_cu = (v.id == CC3D_K_BF16_S1_N192 || v.cin_chunk == 64) ? 1 : 2;
      const int64_t slots = int64_t(kComputeUnits) * wg_per_cu;
      const int64_t stages = int64_t(in.n_active_taps) * (d.c_in / v.cin_chunk);
      if (in.tiles * 4 <= slots) {
        const int64_t s = std::min<int64_t>({slots / std::max<int64_t>(in.tiles, 1), stages / 4, 16});
        in.splits = s >= 4 ? int32_t(s) : 1;
      }
      if (in.splits > 1)
        in.workspace_bytes = (in.tiles * 4 + 255) / 256 * 256 +
                             in.tiles * in.splits * int64_t(in.block_m) * in.block_n * 4;
    }
    // The group-staged kernel (one workgroup per compute unit) splits each
    // tile's group sequence when its tiles would leave half the compute units
    // or more idle: up to 4 splits, as many as fill the units, each with at
    // least one 32-channel group of every tile.
    if (v.id == CC3D_K_BF16_S3_N64_G32W8 || v.id == CC3D_K_BF16_S3_N96_G32W8) {
      if (in.tiles * 2 <= kComputeUnits) {
        const int64_t s = std::min<int64_t>({kComputeUnits / std::max<int64_t>(in.tiles, 1), d.c_in / 32, 4});
        in.splits = s >= 2 ? int32_t(s) : 1;
      }
      if (in.splits > 1)
        in.workspace_bytes = (in.tiles * 4 + 255) / 256 * 256 +
                             in.tiles * in.splits * int64_t(in.block_m) * in.block_n * 4;
    }
    std::snprintf(in.kernel_name, sizeof in.kernel_name, "%s", v.name);
  } else {
    if (kernel && std::strcmp(kernel, "f32_direct") != 0) {
      delete p;
      return refuse(CC3D_ERR_UNSUPPORTED);
    }
    const int64_t frame_el = int64_t(h_out) * w_out * d.c_out;
    if (frame_el >= (int64_t(1) << 31) || int64_t(d.h) * d.w * d.c_in >= (int64_t(1) << 31)) {
      delete p;
      return refuse(CC3D_ERR_UNSUPPORTED);
    }
    in.kernel_id = CC3D_K_F32_DIRECT;
    in.block_m = 256;
    in.block_n = 1;
    in.splits = 1;
    const int64_t total = int64_t(d.n) * t_out * h_out * w_out * d.c_out;
    in.tiles = (total + 255) / 256;
    std::snprintf(in.kernel_name, sizeof in.kernel_name, "%s", "f32_direct");
  }
  if (in.tiles >= (int64_t(1) << 31)) {
    delete p;
    return refuse(CC3D_ERR_UNSUPPORTED);
  }
  p->info = in;
  *out = p;
  return CC3D_OK;
}

}  // namespace

namespace {

// With CC3D_LOG=1 in the environment every plan built is printed to stderr:
// the descriptor, the tap intervals, the kernel and its work.
bool log_plans() {
  static const bool on = [] {
    const char* v = std::getenv("CC3D_LOG");
    return v && v[0] == '1';
  }();
  return on;
}

void dump_plan(const cc3d_plan* p) {
  const cc3d_desc_t& d = p->d;
  const cc3d_plan_info_t& i = p->info;
  std::fprintf(stderr,
               "cc3d plan: N=%d C_in=%d C_out=%d H=%d W=%d T_x=%d T_cache=%d k=(%d,%d,%d) s=(%d,%d,%d) "
               "d=(%d,%d,%d) p=(%d,%d) p_base=%d bias=%d %s\n"
               "  |Z|=%d p_l=%d T_o=%d H_o=%d W_o=%d cache_out=%d active taps=%d\n",
               d.n, d.c_in, d.c_out, d.h, d.w, d.t_x, d.t_cache, d.k_t, d.k_h, d.k_w, d.s_t, d.s_h, d.s_w, d.d_t,
               d.d_h, d.d_w, d.p_h, d.p_w, d.p_base, d.has_bias, d.dtype == CC3D_BF16 ? "bf16" : "fp32", i.t_z,
               i.p_l, i.t_out, i.h_out, i.w_out, i.t_cache_out, i.n_active_taps);
  for (int k = 0; k < d.k_t; ++k)
    std::fprintf(stderr, "  tap %d: delta=%d out=[%d,%d) src=[%d,%d)%s\n", k, i.taps[k].delta, i.taps[k].o_lo,
                 i.taps[k].o_hi, i.taps[k].src_lo, i.taps[k].src_hi, i.taps[k].active ? "" : " inactive");
  std::fprintf(stderr,
               "  kernel %s: tile %d px x %d ch, %lld tiles, splits %d, packed weights %lld B, workspace %lld B, "
               "%.3f GFLOP active (%.3f nominal)\n",
               i.kernel_name, i.block_m, i.block_n, static_cast<long long>(i.tiles), i.splits,
               static_cast<long long>(i.packed_weight_bytes), static_cast<long long>(i.workspace_bytes),
               i.flops_active * 1e-9, i.flops_nominal * 1e-9);
}

cc3d_status_t plan_logged(const cc3d_desc_t* desc, const char* kernel, cc3d_plan_t* out) {
  const cc3d_status_t s = plan_impl(desc, kernel, out);
  if (log_plans()) {
    if (s == CC3D_OK) dump_plan(*out);
    else std::fprintf(stderr, "cc3d plan refused%s%s: %s\n", kernel ? " for " : "", kernel ? kernel : "",
                      causal_conv3d_status_string(s));
  }
  return s;
}

}  // namespace

extern "C" cc3d_status_t causal_conv3d_plan(const cc3d_desc_t* desc, cc3d_plan_t* out) {
  return plan_logged(desc, nullptr, out);
}

extern "C" cc3d_status_t causal_conv3d_plan_variant(const cc3d_desc_t* desc, const char* kernel_name,
                                                    cc3d_plan_t* out) {
  if (out) *out = nullptr;
  if (!kernel_name) return refuse(CC3D_ERR_INVALID_ARG);
  return plan_logged(desc, kernel_name, out);
}

extern "C" cc3d_status_t causal_conv3d_plan_info(cc3d_plan_t plan, cc3d_plan_info_t* info) {
  if (!plan || !info) return refuse(CC3D_ERR_INVALID_ARG);
  *info = plan->info;
  return CC3D_OK;
}

extern "C" void causal_conv3d_plan_destroy(cc3d_plan_t plan) { delete plan; }

extern "C" const char* causal_conv3d_status_string(cc3d_status_t s) {
  switch (s) {
    case CC3D_OK: return "ok";
    case CC3D_ERR_INVALID_ARG: return "invalid argument";
    case CC3D_ERR_UNSUPPORTED: return "unsupported by the cached causal Conv3D kernels";
    case CC3D_ERR_DEVICE: return "HIP runtime rejected a launch";
    case CC3D_ERR_NO_MEMORY: return "out of host memory";
  }
  return "unknown status";
}

extern "C" void causal_conv3d_counters(cc3d_counters_t* out, int reset) {
  using namespace cc3d;
  if (out) {
    out->fast_path = g_fast_path.load();
    out->unsupported = g_unsupported.load();
    out->invalid = g_invalid.load();
    out->device_error = g_device_error.load();
  }
  if (reset) {
    g_fast_path = 0;
    g_unsupported = 0;
    g_invalid = 0;
    g_device_error = 0;
  }
}
