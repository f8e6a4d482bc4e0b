// Host driver for the sanitizer build of the planner (AddressSanitizer and
// UndefinedBehaviorSanitizer; test infrastructure).  Plans every descriptor
// of an exhaustive grid of small shapes on the default choice and on every
// named variant, reads the plan info, checks the interval invariants that
// the lowering section's equal-length output and source intervals imply, and
// destroys the plans; then the refused and invalid paths.  Exit status 0 when
// every check held; a sanitizer report aborts the run.
#include <cstdio>
#include <cstring>
#include <initializer_list>

#include "cc3d.h"

static const char* const kNames[] = {
    "bf16_s3_n64_p24x32_g32", "bf16_s3_n96_p16x32_g32", "bf16_s3_n96_p8x32_x2", "bf16_s3_n32_p8x32",
    "bf16_s3_few_p4x128", "bf16_s3_few_p16x128", "bf16_s1_n192_p8x32", "bf16_s1_n192_p256_rd", "bf16_s1_n32_p8x32",
    "bf16_gen_n64_p8x32", "bf16_gen_n96_p8x32", "bf16_s3d2_n64_p16x32_g32", "bf16_s3s2_n96_p4x32_g32", "bf16_s3s2_n64_p4x32_g32",
    "f32_direct", "no_such_kernel"};

static int failures = 0;
#define CHECK(c)                                                            \
  do {                                                                      \
    if (!(c)) {                                                             \
      std::fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
      ++failures;                                                           \
    }                                                                       \
  } while (0)

static void check_plan(cc3d_plan_t p, const cc3d_desc_t& d) {
  cc3d_plan_info_t in;
  CHECK(causal_conv3d_plan_info(p, &in) == CC3D_OK);
  CHECK(in.t_z == d.t_cache + d.t_x);
  CHECK(in.t_cache_out == (d.p_base < in.t_z ? d.p_base : in.t_z));
  for (int k = 0; k < d.k_t; ++k) {
    const cc3d_tap_t& t = in.taps[k];
    CHECK(t.o_lo <= t.o_hi && t.active == (t.o_hi > t.o_lo));
    if (t.active) {
      CHECK(t.o_lo >= 0 && t.o_hi <= in.t_out);
      CHECK(t.src_lo >= 0 && t.src_hi <= in.t_z);
      CHECK(t.src_hi - t.src_lo == (t.o_hi - t.o_lo - 1) * d.s_t + 1);
    }
  }
  CHECK(std::strlen(in.kernel_name) > 0 && std::strlen(in.kernel_name) < sizeof in.kernel_name);
  CHECK(in.tiles > 0 && in.splits >= 1 && in.workspace_bytes >= 0);
}

int main() {
  int planned = 0;
  for (int dtype = 0; dtype < 2; ++dtype)
    for (int kt = 1; kt <= 4; ++kt)
      for (int ks = 1; ks <= 5; ks += 2)
        for (int st = 1; st <= 2; ++st)
          for (int dt = 1; dt <= 2; ++dt)
            for (int tx = 1; tx <= 4; ++tx)
              for (int tc = 0; tc <= 4; ++tc)
                for (int cout : {3, 40, 96, 192})
                  for (int cin : {16, 32, 96}) {
                    cc3d_desc_t d{};
                    d.n = 1 + (tx & 1);
                    d.c_in = cin;
                    d.c_out = cout;
                    d.h = 5 + tc;
                    d.w = 33 + tx;
                    d.t_x = tx;
                    d.t_cache = tc;
                    d.k_t = kt;
                    d.k_h = d.k_w = ks;
                    d.s_t = st;
                    d.s_h = d.s_w = 1 + (tc == 3);
                    d.d_t = dt;
                    d.d_h = d.d_w = 1 + (tc == 4);
                    d.p_h = d.p_w = (ks - 1) / 2 * d.d_h;
                    d.p_base = dt * (kt - 1) + (tx == 4);
                    d.groups = 1;
                    d.has_bias = tx != 2;
                    d.dtype = dtype;
                    cc3d_plan_t p = nullptr;
                    const cc3d_status_t s = causal_conv3d_plan(&d, &p);
                    CHECK((s == CC3D_OK) == (p != nullptr));
                    if (s == CC3D_OK) {
                      check_plan(p, d);
                      ++planned;
                    }
                    causal_conv3d_plan_destroy(p);
                    for (const char* name : kNames) {
                      cc3d_plan_t q = nullptr;
                      const cc3d_status_t sv = causal_conv3d_plan_variant(&d, name, &q);
                      CHECK(sv == CC3D_OK || sv == CC3D_ERR_UNSUPPORTED || sv == CC3D_ERR_INVALID_ARG);
                      if (sv == CC3D_OK) check_plan(q, d);
                      causal_conv3d_plan_destroy(q);
                    }
                  }
  // refused and invalid descriptors, NULL arguments
  cc3d_desc_t d{};
  d.n = d.c_in = d.c_out = d.h = d.w = d.t_x = 1;
  d.k_t = d.k_h = d.k_w = d.s_t = d.s_h = d.s_w = d.d_t = d.d_h = d.d_w = 1;
  d.groups = 2;
  cc3d_plan_t p = nullptr;
  CHECK(causal_conv3d_plan(&d, &p) == CC3D_ERR_UNSUPPORTED && p == nullptr);
  d.groups = 1;
  d.t_x = 0;
  CHECK(causal_conv3d_plan(&d, &p) == CC3D_ERR_INVALID_ARG && p == nullptr);
  CHECK(causal_conv3d_plan(nullptr, &p) == CC3D_ERR_INVALID_ARG);
  CHECK(causal_conv3d_plan(&d, nullptr) == CC3D_ERR_INVALID_ARG);
  CHECK(causal_conv3d_plan_variant(&d, nullptr, &p) == CC3D_ERR_INVALID_ARG);
  CHECK(causal_conv3d_plan_info(nullptr, nullptr) == CC3D_ERR_INVALID_ARG);
  causal_conv3d_plan_destroy(nullptr);
  for (int s = -1; s < 6; ++s) CHECK(causal_conv3d_status_string(static_cast<cc3d_status_t>(s)) != nullptr);
  cc3d_counters_t c;
  causal_conv3d_counters(&c, 1);
  causal_conv3d_counters(nullptr, 0);
  std::printf("planned %d descriptors, %d failed checks\n", planned, failures);
  return failures == 0 && planned > 0 ? 0 : 1;
}
