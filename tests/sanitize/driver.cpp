// Runs the library's host code under the sanitizers (see stubs.cpp): host
// parameters for every mode, context construction and teardown, the layout
// and parameter getters, and the argument validation of every entry point
// with valid and invalid arguments.  Exits non-zero on an unexpected status;
// a sanitizer finding aborts the process.
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "tq.h"

static int failures = 0;
#define EXPECT(cond)                                                   \
  do {                                                                 \
    if (!(cond)) {                                                     \
      std::fprintf(stderr, "line %d: expected %s\n", __LINE__, #cond); \
      ++failures;                                                      \
    }                                                                  \
  } while (0)

static void host_params(int d, int bits, int mode, bool ok) {
  const int m = (mode == TQ_MODE_MSE) ? 0 : d;
  const int w = mode == TQ_MODE_PROD ? bits - 1 : mode == TQ_MODE_FRAC ? (bits + 1) / 2 - 1 : bits;
  const int n = w >= 1 && w <= 4 ? (1 << w) * 2 : 2;
  std::vector<double> Pi((size_t)d * d > 0 ? (size_t)d * d : 1), S((size_t)(m ? m : 1) * (d > 0 ? d : 1)),
      c(n), t(n);
  const int st = tq_host_params(d, bits, 7, mode, Pi.data(), S.data(), c.data(), t.data());
  EXPECT((st == TQ_OK) == ok);
}

static void context_round_trip(int d, int bits, int mode) {
  tq_ctx *ctx = nullptr;
  int st;
  switch (mode) {
    case TQ_MODE_PROD: st = tq_init(d, bits, 3, &ctx); break;
    case TQ_MODE_MSE: st = tq_init_mse(d, bits, 3, &ctx); break;
    case TQ_MODE_POLAR: st = tq_init_polar(d, bits, 3, &ctx); break;
    default: st = tq_init_frac(d, bits, 3, &ctx); break;
  }
  EXPECT(st == TQ_OK && ctx);
  if (!ctx) return;
  tq_layout_t lay;
  EXPECT(tq_layout(ctx, &lay) == TQ_OK && lay.d == d && lay.mode == mode);
  const int nl = mode == TQ_MODE_POLAR ? 8 : 2;
  std::vector<double> Pi((size_t)d * d), S((size_t)d * d), c((size_t)nl * 16), t((size_t)nl * 16);
  EXPECT(tq_get_params(ctx, Pi.data(), S.data(), c.data(), t.data()) == TQ_OK);
  const bool sketch = mode == TQ_MODE_PROD || mode == TQ_MODE_FRAC;
  // host buffers stand in for device memory (the launchers are stubs)
  const int n = 5;
  std::vector<float> x((size_t)n * d, 1.f), norms(64), rnorms(64), logits(4096), out((size_t)4 * d);
  std::vector<unsigned char> codes((size_t)64 * lay.code_bytes + 16), signs((size_t)64 * (lay.sign_bytes + 1) + 16);
  auto al = [](void *p) { return (void *)(((uintptr_t)p + 15) & ~(uintptr_t)15); };
  float *xa = (float *)al(x.data());
  unsigned char *ca = (unsigned char *)al(codes.data()), *sa = (unsigned char *)al(signs.data());
  EXPECT(tq_quantize(ctx, xa, TQ_F32, n, d, 1, ca, sketch ? sa : nullptr, norms.data(),
                     sketch ? rnorms.data() : nullptr, nullptr) == TQ_OK);
  EXPECT(tq_quantize(ctx, xa, TQ_F32, n, d - 1, 1, ca, sketch ? sa : nullptr, norms.data(),
                     sketch ? rnorms.data() : nullptr, nullptr) == TQ_EINVAL);
  EXPECT(tq_quantize(ctx, xa, 7, n, d, 1, ca, nullptr, norms.data(), nullptr, nullptr) == TQ_EINVAL);
  EXPECT(tq_quantize(ctx, xa, TQ_F32, n, d, 0, ca, nullptr, norms.data(), nullptr, nullptr) == TQ_EINVAL);
  size_t ws = 0;
  const int sst = tq_workspace_size(ctx, TQ_OP_SCORES, 1, 4, 0, &ws);
  EXPECT((sst == TQ_OK) == sketch);
  std::vector<unsigned char> wsb(ws + 16);
  void *wa = al(wsb.data());
  const int st2 = tq_scores(ctx, xa, 1, 4, 5, 5, ca, sa, norms.data(), rnorms.data(), logits.data(), wa, ws, nullptr);
  EXPECT((st2 == TQ_OK) == sketch);
  EXPECT(tq_scores(ctx, xa, 1, 4, 6, 5, ca, sa, norms.data(), rnorms.data(), logits.data(), wa, ws, nullptr) ==
         TQ_EINVAL);                                   // ldk < T
  EXPECT(tq_scores(ctx, xa, 1, 0, 5, 5, ca, sa, norms.data(), rnorms.data(), logits.data(), wa, ws, nullptr) ==
         TQ_EINVAL);                                   // qpg < 1
  if (sketch) {
    EXPECT(tq_scores(ctx, xa, 1, 4, 5, 5, ca, sa, norms.data(), rnorms.data(), logits.data(), wa, ws ? ws - 1 : 0,
                     nullptr) == TQ_EINVAL);           // workspace too small
    EXPECT(tq_prep_queries(ctx, xa, 1, 4, wa, ws, nullptr) == TQ_OK);
    EXPECT(tq_dequant(ctx, ca, sa, norms.data(), rnorms.data(), 3, out.data(), nullptr) == TQ_OK);
    EXPECT(tq_dequant(ctx, ca, nullptr, norms.data(), rnorms.data(), 3, out.data(), nullptr) == TQ_EINVAL);
  }
  const int kst = tq_workspace_size(ctx, TQ_OP_TOPK, 2, 10, 5, &ws);
  EXPECT((kst == TQ_OK) == (mode == TQ_MODE_PROD));
  EXPECT(tq_workspace_size(ctx, TQ_OP_TOPK, 2, 10, TQ_MAX_TOPK + 1, &ws) == TQ_EINVAL);
  tq_free(ctx);
}

int main() {
  for (int mode : {TQ_MODE_PROD, TQ_MODE_MSE})
    for (int d : {8, 64, 96, 128, 200, 256, 264, 520})
      for (int bits = 0; bits <= 5; ++bits) {
        const bool ok = mode == TQ_MODE_PROD ? (bits >= 2 && bits <= 4) : (bits >= 1 && bits <= 4);
        host_params(d, bits, mode, ok);
      }
  for (int d : {0, 7, 1032, 1020}) host_params(d, 3, TQ_MODE_PROD, false);
  for (int hb : {4, 5, 6, 7}) {
    host_params(128, hb, TQ_MODE_FRAC, hb == 5 || hb == 7);
    host_params(256, hb, TQ_MODE_FRAC, hb == 5 || hb == 7);
    host_params(192, hb, TQ_MODE_FRAC, false);
  }
  host_params(128, 3, TQ_MODE_POLAR, false);           // polar codebooks come from tq_polar_codebook
  for (int d : {32, 64, 128, 256})
    for (int b = 1; b <= 4; ++b) {
      std::vector<double> c(8 * 16), t(8 * 16);          // log2(d) levels x 2^b
      EXPECT(tq_polar_codebook(d, b, c.data(), t.data()) == TQ_OK);
    }
  EXPECT(tq_polar_codebook(96, 2, nullptr, nullptr) == TQ_EINVAL);

  context_round_trip(128, 3, TQ_MODE_PROD);
  context_round_trip(200, 2, TQ_MODE_PROD);
  context_round_trip(264, 4, TQ_MODE_PROD);
  context_round_trip(64, 4, TQ_MODE_MSE);
  context_round_trip(128, 2, TQ_MODE_POLAR);
  context_round_trip(128, 5, TQ_MODE_FRAC);
  context_round_trip(256, 7, TQ_MODE_FRAC);

  tq_ctx *h = nullptr;
  EXPECT(tq_init(7, 3, 0, &h) == TQ_EINVAL && h == nullptr);
  EXPECT(tq_init(128, 3, 0, nullptr) == TQ_EINVAL);
  EXPECT(tq_quantize(nullptr, nullptr, 0, 1, 128, 1, nullptr, nullptr, nullptr, nullptr, nullptr) == TQ_EINVAL);
  EXPECT(tq_softmax(nullptr, -1, 4, 1.f, nullptr, nullptr) == TQ_EINVAL);
  EXPECT(tq_topk(nullptr, nullptr, 1, 1, nullptr, nullptr, nullptr, nullptr, 1, nullptr, nullptr, nullptr, 0,
                 nullptr) == TQ_EINVAL);
  tq_free(nullptr);
  std::printf("host checks: %d failures\n", failures);
  return failures ? 1 : 0;
}
