/*
 * cc3d.h -- cached causal Conv3D for AMD Instinct MI355X (gfx950).  C ABI.
 *
 * The operation is the cached causal 3-D convolution of world-model video
 * VAE decoders, as stated in "Cache-Aware Conv3D Lowering Across Embedded
 * World-Model Decoders", lowering section (the paper's Sec. 4, the paragraphs
 * that define the cache-augmented source, the per-tap source time, the
 * effective left padding and the output/source intervals):
 *
 *   Z = [C; X]  -- the temporal cache C (trailing frames of the previous
 *                  chunk) joined ahead of the current input X along time;
 *   p_l = p_base - |C|            effective causal left pad;
 *   delta_k = k*d_t - p_l         offset of temporal tap k (unit stride);
 *   tap k of output frame o reads source frame o + delta_k; frames outside
 *   [0, |Z|) contribute zero, so tap k is evaluated only for o in
 *   [o_lo, o_hi) = [max(0, -delta_k), min(T_o, |Z| - delta_k)), whose source
 *   interval [o_lo + delta_k, o_hi + delta_k) has the same length;
 *   y[o] = b + sum over active taps k of Conv2D(Z[o + delta_k], W[:, :, k])
 *   with PyTorch's cross-correlation convention and the original spatial
 *   stride, zero padding and dilation; the bias is added exactly once.
 *   T_o = |Z| + p_l - d_t*(k_t - 1)  (T_o = |X| when p_base = d_t*(k_t - 1)).
 * Temporal stride s_t > 1 (the encoder's downsampling convs, which the paper
 * leaves outside its unit-stride contract) generalises this: tap k of output
 * frame o reads source frame o*s_t + delta_k, tap k is evaluated for o in
 * [ceil(-delta_k / s_t), min(T_o, ceil((|Z| - delta_k) / s_t))), and
 * T_o = floor((|Z| + p_l - d_t*(k_t - 1) - 1) / s_t) + 1.  Chunked calls
 * carrying the last p_base frames equal one call over the whole sequence
 * when every chunk's length is a multiple of s_t.
 *
 * All active temporal taps, all spatial taps and all input channels form one
 * K reduction accumulated in registers by one kernel (no per-tap Conv2D, no
 * materialised [C; X], no per-tap weight copies).  The carried cache (the
 * last min(p_base, |Z|) frames of Z) is written by a second small kernel.
 *
 * Layouts (dense, channels last; element type given by the descriptor):
 *   x          [N][T_x][H][W][C_in]
 *   cache_in   [N][T_cache][H][W][C_in]
 *   w          [C_out][k_t][k_h][k_w][C_in]   (PyTorch OIDHW weight in
 *                                              channels_last_3d memory format)
 *   b          [C_out]
 *   out        [N][T_o][H_o][W_o][C_out]
 *   cache_out  [N][min(p_base, T_cache + T_x)][H][W][C_in]
 *
 * Ownership: every tensor is caller-owned device memory, and so is the packed
 * weight image of causal_conv3d_pack_weights.  A plan is host metadata only
 * (no device memory, no device call when it is built); it keeps no weight
 * copy.  The library's only device state is a static table of tile counters
 * for the group-staged kernel's dynamic schedule (each launch takes a slot
 * and leaves it zero when it completes).
 * Threading: plans are immutable; any thread may use a plan, and calls of
 * one plan may run at the same time on different streams (at most 1024
 * launches of the group-staged kernel in flight per process).  A launch
 * recorded during stream capture keeps its counter slot for every replay of
 * the graph: two graph launches that share a slot (one in 1024 captured
 * launches) must not run at the same time; they never share one with an
 * eager call.  Counters are atomic.
 * Errors: every check is synchronous and happens before any launch; a launch
 * failure reported by the runtime returns CC3D_ERR_DEVICE; faults during
 * execution surface at the caller's next synchronisation.  The library never
 * falls back to another implementation: an unsupported call returns
 * CC3D_ERR_UNSUPPORTED and the caller decides what to do.
 */
#ifndef CC3D_H
#define CC3D_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  CC3D_OK = 0,
  CC3D_ERR_INVALID_ARG = 1,  /* NULL/misaligned/overlapping buffer, bad size, empty output */
  CC3D_ERR_UNSUPPORTED = 2,  /* outside the supported contract (see causal_conv3d_plan) */
  CC3D_ERR_DEVICE = 3,       /* the HIP runtime rejected a launch */
  CC3D_ERR_NO_MEMORY = 4     /* host allocation failed */
} cc3d_status_t;

typedef enum {
  CC3D_F32 = 0,   /* fp32 storage, fp32 arithmetic */
  CC3D_BF16 = 1   /* bf16 storage, fp32 accumulation, RNE-rounded bf16 output */
} cc3d_dtype_t;

#define CC3D_MAX_KT 8

/* Convolution descriptor: the shape of one call. */
typedef struct cc3d_desc {
  int32_t n, c_in, c_out, h, w;
  int32_t t_x;      /* |X|, frames of the current input, >= 1 */
  int32_t t_cache;  /* |C|, cached frames ahead of X, >= 0 */
  int32_t k_t, k_h, k_w;
  int32_t s_t, s_h, s_w;
  int32_t d_t, d_h, d_w;
  int32_t p_h, p_w;  /* symmetric spatial zero padding */
  int32_t p_base;    /* base causal left pad (d_t*(k_t-1) keeps T_o = |X|) */
  int32_t groups;
  int32_t has_bias;
  int32_t dtype;     /* cc3d_dtype_t */
} cc3d_desc_t;

/* One temporal tap of the plan. */
typedef struct cc3d_tap {
  int32_t delta;          /* k*d_t - p_l */
  int32_t o_lo, o_hi;     /* output frames that read this tap: [o_lo, o_hi) */
  int32_t src_lo, src_hi; /* frames of Z they read: [o_lo+delta, o_hi+delta) at
                             unit stride; every s_t-th frame of [src_lo, src_hi) */
  int32_t active;         /* o_hi > o_lo */
} cc3d_tap_t;

typedef struct cc3d_plan_info {
  int32_t t_z;            /* |Z| = |C| + |X| */
  int32_t p_l;            /* p_base - |C| (negative: leading cache frames unused) */
  int32_t t_out, h_out, w_out;
  int32_t t_cache_out;    /* frames written to cache_out: min(p_base, |Z|) */
  int32_t n_active_taps;
  cc3d_tap_t taps[CC3D_MAX_KT];
  double flops_nominal;   /* 2*N*T_o*H_o*W_o*C_out*C_in*k_t*k_h*k_w */
  double flops_active;    /* the same counted over active (o, k) pairs only */
  double bytes_conv;      /* algorithmic HBM bytes of the conv kernel: each
                             read source frame once, W, b, the output */
  double bytes_cache_out; /* HBM bytes the cache-out adds: the carried
                             frames read and written (by the group-staged
                             kernel once its tiles run out, or by a copy
                             kernel); written only on the few-output-channel
                             kernel, which stores it from the rows it stages */
  int32_t kernel_id;      /* which kernel variant forward launches */
  int32_t block_m, block_n; /* output pixels x output channels per tile */
  int64_t tiles;          /* output tiles of the conv kernel (bf16: processed by
                             min(tiles, compute units) persistent workgroups) */
  int64_t packed_weight_bytes; /* size of the packed weight image (bf16) */
  uint64_t weight_layout;      /* fingerprint of that image: plans with equal
                                  weight_layout and packed_weight_bytes read
                                  the same image (e.g. the chunk plans of one
                                  streaming signature) */
  int64_t workspace_bytes;     /* device scratch causal_conv3d_forward_packed
                                  needs (split reductions); 0: none */
  int32_t splits;              /* K-splits per tile of forward_packed (1: none) */
  char kernel_name[64];
} cc3d_plan_info_t;

typedef struct cc3d_plan* cc3d_plan_t;

typedef struct cc3d_counters {
  uint64_t fast_path;     /* forward calls that launched */
  uint64_t unsupported;   /* plans refused as unsupported */
  uint64_t invalid;       /* plans or forwards refused as invalid */
  uint64_t device_error;  /* launches the runtime rejected */
} cc3d_counters_t;

/*
 * Validate a call's shape and build its plan (host only; no device call).
 *   desc  shape of the call; it is copied.
 *   out   receives the plan; set to NULL on error.
 * Contract (the paper's lowering covers 5-D tensors with unit temporal
 * stride and one group; every call it observed has k_t = 3; temporal stride
 * > 1 is supported here as well):
 *   CC3D_ERR_UNSUPPORTED when groups != 1, k_t > CC3D_MAX_KT, or, for
 *   bf16: k_t > 4, C_in not a multiple of 16, or one frame (input or
 *   output) or the weights reaching 2^31 bytes.  Any spatial kernel size,
 *   stride, dilation and padding runs: 3x3 "same" and 1x1 convs with unit
 *   spatial stride and dilation on the halo-staged kernels, the others on
 *   the gather kernel ("bf16_gen_n96_p8x32" where C_out % 96 == 0, else
 *   "bf16_gen_n64_p8x32"), but for 3x3 "same" convs at spatial dilation 2,
 *   which have a halo-staged kernel of their own.
 *   CC3D_ERR_INVALID_ARG for a NULL pointer, a size < 1 (t_cache < 0), an
 *   unknown dtype, or an empty output (T_o, H_o or W_o < 1).
 * Logging: with CC3D_LOG=1 in the environment (read once per process) every
 * plan built by this call or by causal_conv3d_plan_variant is printed to
 * stderr -- the descriptor, |Z|, p_l, T_o, each temporal tap's delta, output
 * interval and source interval, and the kernel with its tile, tile count,
 * splits and buffer sizes -- and every refused plan with its status.
 */
cc3d_status_t causal_conv3d_plan(const cc3d_desc_t* desc, cc3d_plan_t* out);

/*
 * As causal_conv3d_plan, but run the call with the named kernel variant
 * instead of the default choice (for tests that pin a variant and for
 * tuning; the name is the one plan_info reports).  Variants:
 *   "bf16_s3_n64_p24x32_g32"  3x3, C_out % 64 == 0, C_in % 32 == 0
 *                              (default for large maps)
 *   "bf16_s3_n96_p16x32_g32"  3x3, C_out % 96 == 0, C_in % 32 == 0
 *                              (default for large maps where C_out % 64 != 0)
 *                              (both: on maps whose tiles leave half the
 *                              compute units idle, forward_packed splits each
 *                              tile's channel groups, plan_info.splits)
 *   "bf16_s3_n96_p8x32_x2"    3x3, C_out % 96 == 0
 *   "bf16_s3_n32_p8x32"       3x3, any C_out
 *   "bf16_s3_few_p<R>x128"    3x3, k_t = 3, d_t = 1, s_t = 1, C_out <= 5,
 *                              C_in in {32, 64, 96}; patches of R output rows
 *                              (4 <= R <= 16) by 128 columns (default for the
 *                              RGB head, with R chosen for the map size)
 *   "bf16_s1_n192_p8x32"      1x1, C_out % 192 == 0, C_in % 32 == 0
 *   "bf16_s1_n192_p256_rd"    1x1, C_out % 192 == 0, C_in % 64 == 0 with
 *                              C_in / 64 even or a multiple of 3; tiles of 256
 *                              consecutive pixels, pixels loaded straight into
 *                              registers
 *   "bf16_s1_n32_p8x32"       1x1, any C_out
 *   (the variants above need unit spatial stride and dilation and "same"
 *   padding)
 *   "bf16_gen_n64_p8x32"      any spatial parameters (default outside that
 *                              envelope): input pixels gathered per spatial
 *                              tap, W read as it is
 *   "bf16_gen_n96_p8x32"      the same, 96 output channels per tile,
 *                              C_out % 96 == 0 (the default there)
 *   "bf16_s3d2_n64_p16x32_g32" 3x3 at spatial dilation 2, padding 2, unit
 *                              spatial stride, C_out % 64 == 0, C_in % 32 == 0
 *                              (the default there): the halo-staged kernel
 *   "bf16_s3s2_n96_p4x32_g32" 3x3 at spatial stride 2, padding 1, spatial
 *                              dilation 1, C_out % 96 == 0, C_in % 32 == 0
 *                              (the default there): the halo-staged kernel
 *                              on 4x32-output-pixel tiles
 *   "bf16_s3s2_n64_p4x32_g32" the same with C_out % 64 == 0 (the default
 *                              there where C_out % 96 != 0)
 *   "f32_direct"              fp32
 * Every variant computes the same operation; bf16 results of different
 * variants may differ in the last bit (fp32 accumulation order).
 * Returns CC3D_ERR_INVALID_ARG for a NULL name, CC3D_ERR_UNSUPPORTED for an
 * unknown name or a variant that cannot run this call, and otherwise what
 * causal_conv3d_plan returns.
 */
cc3d_status_t causal_conv3d_plan_variant(const cc3d_desc_t* desc, const char* kernel_name, cc3d_plan_t* out);

/*
 * Per-signature tuning (the pages time every runtime signature of a decoder;
 * the variant that suits one shape need not suit another).  Plans desc on
 * every bf16 variant that can run it, runs each once on the caller's
 * buffers through causal_conv3d_forward_packed, with its weights packed
 * into a temporary device buffer and a temporary split workspace (which it
 * allocates and frees), times `launches` further convolutions of it with
 * HIP events on `stream`, and returns in *out the plan of the fastest with
 * its average time in *best_ms (may be NULL).  fp32 descriptors get
 * causal_conv3d_plan's plan without timing.
 *   x, cache_in, w, b, out  as for causal_conv3d_forward (out is
 *                           overwritten; cache_out is not written)
 *   launches                timed convolutions per variant, >= 1
 * Blocking: it waits for its own launches (a tuning-time call, not for the
 * decode loop).  Every launch counts in the fast-path counter.  Returns what causal_conv3d_plan returns for a refused
 * descriptor, CC3D_ERR_INVALID_ARG for a NULL out or launches < 1 or a
 * buffer the forward call rejects, and CC3D_ERR_DEVICE when a launch or an
 * event fails; *out is NULL on error.
 */
cc3d_status_t causal_conv3d_plan_autotune(const cc3d_desc_t* desc, const void* x, const void* cache_in,
                                          const void* w, const void* b, void* out, int launches, void* stream,
                                          cc3d_plan_t* out_plan, float* best_ms);

/* Intervals, sizes, work and launch geometry of a plan (host only). */
cc3d_status_t causal_conv3d_plan_info(cc3d_plan_t plan, cc3d_plan_info_t* info);

/* Release a plan (host memory only); NULL is ignored.  Launches already
 * issued do not depend on the plan. */
void causal_conv3d_plan_destroy(cc3d_plan_t plan);

/*
 * Run the cached causal Conv3D of `plan` asynchronously on `stream`.
 *   x          device pointer, [N][T_x][H][W][C_in]; required.
 *   cache_in   device pointer, [N][T_cache][H][W][C_in]; required when
 *              T_cache > 0, ignored when T_cache = 0.
 *   w          device pointer, [C_out][k_t][k_h][k_w][C_in]; required.  Read
 *              in place (the kernels gather each stage's weights from it).
 *   b          device pointer, [C_out]; required iff has_bias.
 *   out        device pointer, [N][T_o][H_o][W_o][C_out]; required.
 *   cache_out  device pointer, [N][t_cache_out][H][W][C_in], or NULL when no
 *              carry is wanted.
 *   stream     a hipStream_t (NULL: the null stream).
 * Frames of Z outside every tap's source interval are never read (e.g. the
 * leading |C| - p_base cache frames when |C| > p_base).  Allocates nothing,
 * never synchronises; the call may be recorded in a graph.
 * Returns CC3D_ERR_INVALID_ARG (nothing launched) for a NULL required
 * pointer, a bf16 buffer not 16-byte aligned (fp32: 4-byte), `out`
 * overlapping any other buffer, or `cache_out` overlapping x, cache_in, w or
 * b (in a streaming loop ping-pong two cache buffers).  Returns
 * CC3D_ERR_DEVICE if the runtime rejects a launch.
 */
cc3d_status_t causal_conv3d_forward(cc3d_plan_t plan, const void* x, const void* cache_in,
                                    const void* w, const void* b, void* out, void* cache_out,
                                    void* stream);

/*
 * Weights that do not change between calls (a decoder at inference) can be
 * packed once into the kernels' stage order, so that every stage's weights
 * stream into LDS as whole cache lines (the paper keeps the weights
 * unchanged and slices them per tap; here the one image serves every tap).
 * causal_conv3d_pack_weights writes plan_info.packed_weight_bytes bytes of
 * that image from w into the caller-owned device buffer w_packed (16-byte
 * aligned) on `stream`.  Every plan with the same weight_layout reads the
 * same image, so the chunk plans of one streaming signature share one.
 * causal_conv3d_forward_packed then runs the convolution from it; its other
 * arguments are those of causal_conv3d_forward, plus a caller-owned
 * workspace of at least plan_info.workspace_bytes (NULL and 0 when that is
 * 0; zero-filled before its first use; calls that share a workspace must
 * not overlap).  Both are asynchronous on `stream`, allocate nothing and may
 * be recorded in a graph.  They return CC3D_ERR_INVALID_ARG for an fp32
 * plan, a NULL required pointer, a misaligned buffer, w_packed overlapping w
 * (pack) or out / cache_out (forward), or a workspace smaller than
 * workspace_bytes; the other rules are causal_conv3d_forward's.  The image
 * is read asynchronously: do not rewrite it while a call may still read it.
 */
cc3d_status_t causal_conv3d_pack_weights(cc3d_plan_t plan, const void* w, void* w_packed, void* stream);
cc3d_status_t causal_conv3d_forward_packed(cc3d_plan_t plan, const void* x, const void* cache_in,
                                           const void* w_packed, const void* b, void* out, void* cache_out,
                                           void* workspace, int64_t workspace_bytes, void* stream);

/*
 * For callers that cannot allocate device memory (code under graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): the convolution of
 * causal_conv3d_forward_packed with the split workspace in a static device
 * array of the library (CC3D_NOALLOC_SCRATCH_BYTES, one per device the
 * library runs on, held until the process ends) instead of a caller
 * buffer; the array used is the current device's, which must be the
 * device of `stream` and of the buffers.  It allocates nothing; before a split call it zeroes the array's
 * arrival counters with a small kernel on `stream`.  Every call on a device
 * shares that device's array: calls that overlap on one device (other
 * streams, other threads) race and must not be issued.  Arguments and
 * errors are those of causal_conv3d_forward_packed, plus
 * CC3D_ERR_UNSUPPORTED for a plan whose workspace_bytes exceeds
 * CC3D_NOALLOC_SCRATCH_BYTES and CC3D_ERR_DEVICE when the array's address
 * cannot be obtained.  Plans without a split need no array and run as
 * causal_conv3d_forward_packed.
 */
#define CC3D_NOALLOC_SCRATCH_BYTES (64u << 20)
cc3d_status_t causal_conv3d_forward_packed_noalloc(cc3d_plan_t plan, const void* x, const void* cache_in,
                                                   const void* w_packed, const void* b, void* out, void* cache_out,
                                                   void* stream);

/*
 * The RGB head with its pixel quantisation fused in (FastVideo pull request
 * "[perf] Quantize frames to uint8 on-device before the post-decode D->H
 * copy": the decoded frames are scaled by 255, clamped to [0, 255] and cast
 * to uint8 on the device, so the copy to the host is of bytes).  Runs the
 * plan's convolution and writes out as 8-bit codes, one byte per channel in
 * the layout of out ([N][T_o][H_o][W_o][C_out]):
 *   code = trunc(clamp(fma(y, scale, offset) * 255, 0, 255))
 * decided in fp32 from the unrounded fp32 sum y (bias included).  scale =
 * offset = 0.5 maps a head output in [-1, 1] to [0, 1] first (that mapping is
 * not on the pages; it is the usual video-decoder convention).  A NaN sum
 * gives code 0.  w is read in place, as by causal_conv3d_forward; cache_out
 * is written as by causal_conv3d_forward.
 * out needs no alignment.  Returns CC3D_ERR_UNSUPPORTED unless the plan runs
 * on the few-output-channel kernel ("bf16_s3_few_p<R>x128"),
 * CC3D_ERR_INVALID_ARG for a NaN scale or offset and as
 * causal_conv3d_forward otherwise.
 */
cc3d_status_t causal_conv3d_forward_u8(cc3d_plan_t plan, const void* x, const void* cache_in, const void* w,
                                       const void* b, void* out, void* cache_out, float scale, float offset,
                                       void* stream);

/* Static description of a status code. */
const char* causal_conv3d_status_string(cc3d_status_t status);

/* Snapshot the route counters into *out (may be NULL); reset them if reset != 0. */
void causal_conv3d_counters(cc3d_counters_t* out, int reset);

#ifdef __cplusplus
}
#endif

#endif /* CC3D_H */
