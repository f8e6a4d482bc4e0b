// Launcher of the cached causal Conv3D on gfx950 (MI355X): argument checks,
// the kernel argument block of a plan, and the C entry points that run,
// pack and tune.
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
// fp32 and rounded to nearest even at the end; the planner picks one per
// plan, see cc3d_plan.cpp):
//   * conv_bf16_g32 (cc3d_k_g32.hip): large 3x3 maps, also at spatial
//     dilation 2 ("same") and at spatial stride 2.  One persistent workgroup
//     per compute unit with a dynamic per-XCD tile schedule; the halo of one
//     (active tap, 32-channel group) is staged once into LDS and serves 9
//     spatial taps x 2 sub-stages of 16 channels.  Workgroups whose tiles
//     have run out copy the cache-out.
//   * conv_bf16_mfma (cc3d_k_mfma.hip): smaller 3x3 maps (two workgroups per
//     compute unit), other C_out, and the 1x1 / (k_t,1,1) convs.
//   * conv_bf16_few (cc3d_few.inc): C_out <= 5 (the RGB head).  Walks
//     time per patch, streaming whole halo rows; stores the cache-out from
//     the rows it stages.
//   * conv_bf16_gen, conv_f32_direct, copy_tail_frames (cc3d_k_misc.hip):
//     any other spatial parameters, the fp32 path, the cache-out of the
//     other kernels.
// The halo-staged kernels read their weights from a packed, stage-ordered
// image when the caller supplies one (causal_conv3d_pack_weights), and
// gather them from W in place otherwise; nothing is kept between calls.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdint>
#include <cstring>
#include <utility>

#include "cc3d_device.h"

namespace cc3d {

// Counter-table slots: eager launches take [0, kSchedEager) in turn,
// launches recorded during stream capture [kSchedEager, kSchedSlots).
int next_sched_slot(bool capturing) {
  static std::atomic<uint32_t> eager{0}, captured{0};
  if (capturing) return kSchedEager + int(captured.fetch_add(1, std::memory_order_relaxed) % (kSchedSlots - kSchedEager));
  return int(eager.fetch_add(1, std::memory_order_relaxed) % kSchedEager);
}

}  // namespace cc3d

namespace {

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

cc3d_status_t device_error() {
  cc3d::g_device_error.fetch_add(1, std::memory_order_relaxed);
  return CC3D_ERR_DEVICE;
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

bool is_g32(int32_t id) {
  return id == CC3D_K_BF16_S3_N96_G32W8 || id == CC3D_K_BF16_S3_N64_G32W8 || id == CC3D_K_BF16_S3D2_N64_G32W8 ||
         id == CC3D_K_BF16_S3S2_N96_G32W4 || id == CC3D_K_BF16_S3S2_N64_G32W8;
}

bool is_mfma(int32_t id) {
  return id == CC3D_K_BF16_S3_N96_X2 || id == CC3D_K_BF16_S3_N32 || id == CC3D_K_BF16_S1_N192 ||
         id == CC3D_K_BF16_S1_N32;
}

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

// The argument block of a plan's convolution (pointers filled by the caller).
void plan_args(const cc3d_plan* plan, ConvArgs& a) {
  const cc3d_desc_t& d = plan->d;
  const cc3d_plan_info_t& in = plan->info;
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
  a.nblk_n = plan->nblk_n;
  a.ntiles = int(in.tiles);
  a.has_bias = d.has_bias;
  a.co_lo = in.t_z;
  a.splits = 1;
}

// Pixel output of the head: 8-bit codes instead of bf16 (see ConvArgs).
struct PixelOut {
  float scale, offset;
};

// One convolution of `plan`.  Exactly one of w (weights as stored) and wpk
// (the packed image) is given; ws (ws_bytes >= plan_info.workspace_bytes)
// enables the plan's split reduction.
cc3d_status_t run_plan(cc3d_plan_t plan, const void* x, const void* cache_in, const void* w, const void* wpk,
                       const void* b, void* out, void* cache_out, void* stream, const PixelOut* px = nullptr,
                       void* ws = nullptr, int64_t ws_bytes = 0) {
  if (!plan) return invalid();
  const cc3d_desc_t& d = plan->d;
  const cc3d_plan_info_t& in = plan->info;
  if (px && in.kernel_id != CC3D_K_BF16_S3_FEW) {
    cc3d::g_unsupported.fetch_add(1, std::memory_order_relaxed);
    return CC3D_ERR_UNSUPPORTED;
  }
  const int64_t out_bytes = px ? plan->out_bytes / plan->elem : plan->out_bytes;
  const bool bf16 = d.dtype == CC3D_BF16;
  if (d.t_cache == 0) cache_in = nullptr;
  if (!d.has_bias) b = nullptr;
  if (!x || !out || (!w && !wpk) || (d.t_cache > 0 && !cache_in) || (d.has_bias && !b)) return invalid();
  const uintptr_t al = bf16 ? 16 : 4;
  if (!aligned(x, al) || !aligned(cache_in, al) || !aligned(w, al) || !aligned(wpk, 16) || (!px && !aligned(out, al)) ||
      !aligned(cache_out, al) || !aligned(b, uintptr_t(plan->elem)))
    return invalid();
  const void* wsrc = w ? w : wpk;
  const int64_t wsrc_bytes = w ? plan->w_bytes : in.packed_weight_bytes;
  if (overlaps(out, out_bytes, x, plan->x_bytes) || overlaps(out, out_bytes, cache_in, plan->cache_bytes) ||
      overlaps(out, out_bytes, wsrc, wsrc_bytes) || overlaps(out, out_bytes, b, plan->b_bytes) ||
      overlaps(out, out_bytes, cache_out, plan->cache_out_bytes) ||
      overlaps(cache_out, plan->cache_out_bytes, x, plan->x_bytes) ||
      overlaps(cache_out, plan->cache_out_bytes, cache_in, plan->cache_bytes) ||
      overlaps(cache_out, plan->cache_out_bytes, wsrc, wsrc_bytes) ||
      overlaps(cache_out, plan->cache_out_bytes, b, plan->b_bytes))
    return invalid();
  const bool split = ws && in.splits > 1;
  if (split && (ws_bytes < in.workspace_bytes || !aligned(ws, 256) || overlaps(ws, ws_bytes, out, out_bytes) ||
                overlaps(ws, ws_bytes, cache_out, plan->cache_out_bytes) || overlaps(ws, ws_bytes, x, plan->x_bytes) ||
                overlaps(ws, ws_bytes, cache_in, plan->cache_bytes) || overlaps(ws, ws_bytes, wsrc, wsrc_bytes) ||
                overlaps(ws, ws_bytes, b, plan->b_bytes)))
    return invalid();

  ConvArgs a{};
  plan_args(plan, a);
  a.x = x;
  a.cache = cache_in;
  a.b = b;
  a.out = out;
  // the halo-staged kernels read the packed image; the others read W's own
  // layout, which is what their packed image is
  if (plan->pack_kind == 1) {
    a.w = w;
    a.wpk = w ? nullptr : wpk;
  } else {
    a.w = wsrc;
    a.wpk = nullptr;
  }
  // the few-output-channel and group-staged kernels write the cache-out themselves
  const bool fused_co = (in.kernel_id == CC3D_K_BF16_S3_FEW || is_g32(in.kernel_id)) && cache_out && in.t_cache_out > 0;
  a.cache_out = fused_co ? cache_out : nullptr;
  a.co_lo = fused_co ? a.tz - in.t_cache_out : a.tz;
  a.splits = split ? in.splits : 1;
  a.ntiles = int(in.tiles * a.splits);
  if (split) {
    a.ws = ws;
    a.ws_part = (in.tiles * 4 + 255) / 256 * 256;
  }
  if (px) {
    a.out_u8 = 1;
    a.px_scale = px->scale;
    a.px_offset = px->offset;
  }
  if (is_g32(in.kernel_id) && !frame_intervals(plan, a)) return invalid();

  hipStream_t s = static_cast<hipStream_t>(stream);
  int cus = 256;
  if (bf16) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return device_error();
    cus = device_cus(dev);
  }
  if (is_g32(in.kernel_id)) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(s, &cs) != hipSuccess) return device_error();
    a.sched_slot = cc3d::next_sched_slot(cs == hipStreamCaptureStatusActive);
  }

  hipError_t e = hipSuccess;
  if (in.kernel_id == CC3D_K_F32_DIRECT) e = cc3d::launch_f32_direct(a, in.tiles, s);
  else if (is_g32(in.kernel_id)) e = cc3d::launch_g32_family(in.kernel_id, a, std::max<int64_t>(a.nat, 1), cus, s);
  else if (is_mfma(in.kernel_id)) e = cc3d::launch_mfma_family(in.kernel_id, plan->cin_chunk, a, a.ntiles, cus, s);
  else if (in.kernel_id == CC3D_K_BF16_S1_N192_RD) e = cc3d::launch_s1rd(a, in.tiles, cus, s);
  else if (in.kernel_id == CC3D_K_BF16_S3_FEW) {
    switch (d.c_out) {
      case 1: e = cc3d::launch_few_cout<1>(a, in.tiles, cus, s); break;
      case 2: e = cc3d::launch_few_cout<2>(a, in.tiles, cus, s); break;
      case 3: e = cc3d::launch_few_cout<3>(a, in.tiles, cus, s); break;
      case 4: e = cc3d::launch_few_cout<4>(a, in.tiles, cus, s); break;
      default: e = cc3d::launch_few_cout<5>(a, in.tiles, cus, s); break;
    }
  }
  else if (in.kernel_id == CC3D_K_BF16_GEN_N64 || in.kernel_id == CC3D_K_BF16_GEN_N96)
    e = cc3d::launch_gen_family(in.kernel_id, a, in.tiles, s);
  else return invalid();
  if (e == hipSuccess && cache_out && in.t_cache_out > 0 && !fused_co) {
    const int64_t frame_bytes = int64_t(d.h) * d.w * d.c_in * plan->elem;
    const bool vec16 = (frame_bytes % 16 == 0) && aligned(x, 16) && aligned(cache_in, 16) && aligned(cache_out, 16);
    e = cc3d::launch_copy_tail(x, cache_in, cache_out, frame_bytes, d.n, d.t_x, d.t_cache, in.t_cache_out, vec16, s);
  }
  if (e != hipSuccess) return device_error();
  cc3d::g_fast_path.fetch_add(1, std::memory_order_relaxed);
  return CC3D_OK;
}

}  // namespace

extern "C" cc3d_status_t causal_conv3d_forward(cc3d_plan_t plan, const void* x, const void* cache_in,
                                               const void* w, const void* b, void* out, void* cache_out,
                                               void* stream) {
  if (!w) return invalid();
  return run_plan(plan, x, cache_in, w, nullptr, b, out, cache_out, stream);
}

extern "C" cc3d_status_t causal_conv3d_pack_weights(cc3d_plan_t plan, const void* w, void* w_packed, void* stream) {
  if (!plan || !w || !w_packed || plan->d.dtype != CC3D_BF16) return invalid();
  if (!aligned(w, 16) || !aligned(w_packed, 16) ||
      overlaps(w, plan->w_bytes, w_packed, plan->info.packed_weight_bytes))
    return invalid();
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (plan->pack_kind == 1) {
    ConvArgs a{};
    plan_args(plan, a);
    a.w = w;
    e = cc3d::pack_stage_weights(plan->info.block_n, plan->d.k_h, plan->cin_chunk, a, w_packed, s);
  } else {
    e = hipMemcpyAsync(w_packed, w, size_t(plan->w_bytes), hipMemcpyDeviceToDevice, s);
  }
  return e == hipSuccess ? CC3D_OK : device_error();
}

extern "C" cc3d_status_t causal_conv3d_forward_packed(cc3d_plan_t plan, const void* x, const void* cache_in,
                                                      const void* w_packed, const void* b, void* out,
                                                      void* cache_out, void* workspace, int64_t workspace_bytes,
                                                      void* stream) {
  if (!plan || !w_packed || plan->d.dtype != CC3D_BF16) return invalid();
  if (workspace_bytes < 0 || (workspace_bytes > 0 && !workspace)) return invalid();
  if (plan->info.workspace_bytes > 0 && (!workspace || workspace_bytes < plan->info.workspace_bytes)) return invalid();
  return run_plan(plan, x, cache_in, nullptr, w_packed, b, out, cache_out, stream, nullptr, workspace,
                  workspace_bytes);
}

extern "C" cc3d_status_t causal_conv3d_forward_u8(cc3d_plan_t plan, const void* x, const void* cache_in,
                                                  const void* w, const void* b, void* out, void* cache_out,
                                                  float scale, float offset, void* stream) {
  if (!(scale == scale) || !(offset == offset) || !w) return invalid();  // NaN
  const PixelOut px{scale, offset};
  return run_plan(plan, x, cache_in, w, nullptr, b, out, cache_out, stream, &px);
}

// Per-signature variant choice: every bf16 variant that can run the call is
// timed on the caller's buffers, with its weights packed into a temporary
// buffer, and the fastest is kept.
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
                                            "bf16_s1_n192_p256_rd",
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
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipEvent_t e0 = nullptr, e1 = nullptr;
  if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) {
    if (e0) (void)hipEventDestroy(e0);
    return device_error();
  }
  void* wpk = nullptr;
  void* ws = nullptr;
  int64_t wpk_bytes = 0, ws_bytes = 0;
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
    cc3d_status_t rs = CC3D_OK;
    // temporary packed image and split workspace (zero-filled), grown as needed
    if (p->info.packed_weight_bytes > wpk_bytes) {
      if (wpk) (void)hipFree(wpk);
      wpk = nullptr;
      wpk_bytes = 0;
      if (hipStreamSynchronize(s) != hipSuccess || hipMalloc(&wpk, size_t(p->info.packed_weight_bytes)) != hipSuccess) {
        wpk = nullptr;
        rs = device_error();
      } else {
        wpk_bytes = p->info.packed_weight_bytes;
      }
    }
    if (rs == CC3D_OK && p->info.workspace_bytes > ws_bytes) {
      if (ws) (void)hipFree(ws);
      ws = nullptr;
      ws_bytes = 0;
      if (hipStreamSynchronize(s) != hipSuccess || hipMalloc(&ws, size_t(p->info.workspace_bytes)) != hipSuccess ||
          hipMemsetAsync(ws, 0, size_t(p->info.workspace_bytes), s) != hipSuccess) {
        rs = device_error();
      } else {
        ws_bytes = p->info.workspace_bytes;
      }
    }
    // pack, one untimed run, then time the convolution alone
    if (rs == CC3D_OK) rs = causal_conv3d_pack_weights(p, w, wpk, stream);
    if (rs == CC3D_OK) rs = causal_conv3d_forward_packed(p, x, cache_in, wpk, b, out, nullptr, ws, ws_bytes, stream);
    if (rs == CC3D_OK && hipEventRecord(e0, s) != hipSuccess) rs = device_error();
    for (int i = 0; i < launches && rs == CC3D_OK; ++i)
      rs = causal_conv3d_forward_packed(p, x, cache_in, wpk, b, out, nullptr, ws, ws_bytes, stream);
    float ms = 0.f;
    if (rs == CC3D_OK && (hipEventRecord(e1, s) != hipSuccess || hipEventSynchronize(e1) != hipSuccess ||
                          hipEventElapsedTime(&ms, e0, e1) != hipSuccess))
      rs = device_error();
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
  (void)hipStreamSynchronize(s);
  if (wpk) (void)hipFree(wpk);
  if (ws) (void)hipFree(ws);
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
