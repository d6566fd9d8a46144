// Drives every validation branch of the C ABI (include/kvpop.h) in a build of
// abi.cpp with AddressSanitizer and UBSan and the host-only stand-ins of
// abi_stubs.cpp.  Host arrays the ABI reads (cu_seqlens_host) are heap
// allocations of exactly the documented length, so a read past them is
// reported.  Device pointers are never dereferenced by the ABI layer; the
// valid calls reach the stand-in launchers.  Prints "all N cases passed".
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "kvpop.h"
#include "stub_control.h"

static int g_cases = 0, g_fail = 0;

static void expect(const char *what, kvpop_status got, kvpop_status want) {
  ++g_cases;
  const char *msg = kvpop_last_error();
  bool ok = got == want;
  if (want != KVPOP_OK && (msg == nullptr || msg[0] == '\0')) ok = false;  // a failure says why
  if (want == KVPOP_OK && msg != nullptr && msg[0] != '\0') ok = false;    // success clears it
  if (!ok) {
    ++g_fail;
    std::printf("FAIL %s: status %d, expected %d (%s)\n", what, got, want, msg ? msg : "(null)");
  }
}

static void expect_size(const char *what, size_t got, size_t want) {
  ++g_cases;
  if (got != want) {
    ++g_fail;
    std::printf("FAIL %s: size %zu, expected %zu\n", what, got, want);
  }
}

alignas(256) static unsigned char g_dev[1 << 16];  // stands in for device memory; never read by the ABI
static void *P(size_t off = 0) { return g_dev + off; }
static float *F(size_t off = 0) { return reinterpret_cast<float *>(g_dev + off); }
static int32_t *I(size_t off = 0) { return reinterpret_cast<int32_t *>(g_dev + off); }

// cu_seqlens_host of exactly n_docs + 1 entries on the heap
struct Cu {
  int32_t *host = nullptr;
  explicit Cu(const std::vector<int32_t> &v) {
    host = static_cast<int32_t *>(std::malloc(v.size() * sizeof(int32_t)));
    std::memcpy(host, v.data(), v.size() * sizeof(int32_t));
  }
  ~Cu() { std::free(host); }
};

static kvpop_shape shape(int B = 1, int S = 64, int Hq = 4, int Hkv = 2, int D = 64, int dtype = KVPOP_BF16) {
  kvpop_shape s;
  std::memset(&s, 0, sizeof(s));
  s.batch = B;
  s.seqlen = S;
  s.n_q_heads = Hq;
  s.n_kv_heads = Hkv;
  s.head_dim = D;
  s.dtype = dtype;
  s.softmax_scale = 0.f;
  return s;
}

static kvpop_status fwd(const kvpop_shape *s, void *q = P(), void *k = P(), void *v = P(), void *o = P(),
                        float *lse = F()) {
  return kvpop_attn_fwd_lse(s, q, k, v, o, lse, nullptr);
}
static kvpop_status tgt(const kvpop_shape *s, int window = 4, int agg = KVPOP_AGG_SUM, float eps = 0.f,
                        void *ws = P(), size_t ws_bytes = kStubWorkspace, const void *q = P(), float *lse = F()) {
  return kvpop_future_target(s, q, P(), lse, window, agg, 0, eps, F(), ws, ws_bytes, nullptr);
}
static kvpop_status bud(const kvpop_shape *s, int sinks = 4, int window = 8, int topk = 16, void *ws = P(),
                        size_t ws_bytes = kStubWorkspace, int32_t *rank = I(), int32_t *cut = I()) {
  return kvpop_budget_mask_fwd(s, P(), P(), P(), F(), sinks, window, topk, P(), F(), rank, cut, ws, ws_bytes,
                               nullptr);
}

static void shape_cases() {
  kvpop_shape s = shape();
  expect("valid forward", fwd(&s), KVPOP_OK);
  expect("null shape", fwd(nullptr), KVPOP_EINVAL);
  struct { const char *what; kvpop_shape s; kvpop_status want; } table[] = {
      {"batch 0", shape(0), KVPOP_EINVAL},
      {"seqlen 0", shape(1, 0), KVPOP_EINVAL},
      {"seqlen -5", shape(1, -5), KVPOP_EINVAL},
      {"n_q_heads 0", shape(1, 64, 0), KVPOP_EINVAL},
      {"n_kv_heads 0", shape(1, 64, 4, 0), KVPOP_EINVAL},
      {"group not whole", shape(1, 64, 3, 2), KVPOP_EINVAL},
      {"head_dim 96", shape(1, 64, 4, 2, 96), KVPOP_EUNSUPPORTED},
      {"head_dim -64", shape(1, 64, 4, 2, -64), KVPOP_EUNSUPPORTED},
      {"dtype 7", shape(1, 64, 4, 2, 64, 7), KVPOP_EUNSUPPORTED},
      {"seqlen above 2^24", shape(1, (1 << 24) + 1), KVPOP_EUNSUPPORTED},
      {"elements above the limit", shape(1 << 20, 1 << 24, 1 << 10, 1 << 10, 128), KVPOP_EUNSUPPORTED},
      {"int32 extremes", shape(INT32_MAX, INT32_MAX, INT32_MAX, INT32_MAX, 128), KVPOP_EUNSUPPORTED},
      {"fp32 forward at 128", shape(1, 64, 4, 2, 128, KVPOP_F32), KVPOP_EUNSUPPORTED},
  };
  for (auto &c : table) expect(c.what, fwd(&c.s), c.want);
}

static void packed_cases() {
  const int S = 100;
  {
    Cu cu({0, 10, 60, 100});
    kvpop_shape s = shape(1, S);
    s.cu_seqlens = I(64);
    s.cu_seqlens_host = cu.host;
    s.n_docs = 3;
    expect("valid packed forward", fwd(&s), KVPOP_OK);
    expect("valid packed target", tgt(&s), KVPOP_OK);
    expect("valid packed budget", bud(&s), KVPOP_OK);
    s.batch = 2;
    expect("packed with batch 2", fwd(&s), KVPOP_EINVAL);
    s.batch = 1;
    s.cu_seqlens = nullptr;
    expect("host offsets without device offsets", fwd(&s), KVPOP_EINVAL);
    s.cu_seqlens = I(64);
    s.cu_seqlens_host = nullptr;
    expect("device offsets without host offsets", fwd(&s), KVPOP_EINVAL);
    s.cu_seqlens_host = cu.host;
    s.n_docs = 0;
    expect("n_docs 0", fwd(&s), KVPOP_EINVAL);
    s.n_docs = 2;
    expect("n_docs short of seqlen", fwd(&s), KVPOP_EINVAL);
    s.n_docs = 3;
    s.cu_seqlens = I(66);
    expect("misaligned device offsets", fwd(&s), KVPOP_EINVAL);
  }
  struct { const char *what; std::vector<int32_t> cu; kvpop_status want; } table[] = {
      {"offsets not from 0", {1, 50, 100}, KVPOP_EINVAL},
      {"empty document", {0, 50, 50, 100}, KVPOP_EINVAL},
      {"falling offsets", {0, 60, 40, 100}, KVPOP_EINVAL},
      {"offsets past seqlen", {0, 50, 101}, KVPOP_EINVAL},
      {"offsets short of seqlen", {0, 50, 99}, KVPOP_EINVAL},
      {"one document", {0, 100}, KVPOP_OK},
  };
  for (auto &c : table) {
    Cu cu(c.cu);
    kvpop_shape s = shape(1, S);
    s.cu_seqlens = I(64);
    s.cu_seqlens_host = cu.host;
    s.n_docs = (int)c.cu.size() - 1;
    expect(c.what, fwd(&s), c.want);
  }
  // many documents: every offset is read, none beyond
  std::vector<int32_t> many(1001);
  for (int i = 0; i <= 1000; ++i) many[i] = 3 * i;
  Cu cu(many);
  kvpop_shape s = shape(1, 3000);
  s.cu_seqlens = I(64);
  s.cu_seqlens_host = cu.host;
  s.n_docs = 1000;
  expect("1000 documents", fwd(&s), KVPOP_OK);
}

static void pointer_cases() {
  kvpop_shape s = shape();
  expect("null q", fwd(&s, nullptr), KVPOP_EINVAL);
  expect("null k", fwd(&s, P(), nullptr), KVPOP_EINVAL);
  expect("null v", fwd(&s, P(), P(), nullptr), KVPOP_EINVAL);
  expect("null o (LSE only)", fwd(&s, P(), P(), P(), nullptr), KVPOP_OK);
  expect("null lse", fwd(&s, P(), P(), P(), P(), nullptr), KVPOP_EINVAL);
  expect("misaligned q", fwd(&s, P(8)), KVPOP_EINVAL);
  expect("misaligned v", fwd(&s, P(), P(), P(4)), KVPOP_EINVAL);
  expect("misaligned o", fwd(&s, P(), P(), P(), P(2)), KVPOP_EINVAL);
  expect("misaligned lse", fwd(&s, P(), P(), P(), P(), F(2)), KVPOP_EINVAL);
}

static void target_cases() {
  kvpop_shape s = shape();
  expect("valid target", tgt(&s), KVPOP_OK);
  expect("negative window", tgt(&s, -1), KVPOP_EINVAL);
  expect("agg 3", tgt(&s, 4, 3), KVPOP_EINVAL);
  expect("agg -1", tgt(&s, 4, -1), KVPOP_EINVAL);
  expect("eps negative", tgt(&s, 4, KVPOP_AGG_SUM, -1e-6f), KVPOP_EINVAL);
  expect("eps NaN", tgt(&s, 4, KVPOP_AGG_SUM, std::nanf("")), KVPOP_EINVAL);
  expect("eps inf", tgt(&s, 4, KVPOP_AGG_SUM, INFINITY), KVPOP_EINVAL);
  expect("workspace too small", tgt(&s, 4, KVPOP_AGG_SUM, 0.f, P(), kStubWorkspace - 1), KVPOP_EWORKSPACE);
  expect("workspace null", tgt(&s, 4, KVPOP_AGG_SUM, 0.f, nullptr, kStubWorkspace), KVPOP_EWORKSPACE);
  expect("workspace misaligned", tgt(&s, 4, KVPOP_AGG_SUM, 0.f, P(8)), KVPOP_EINVAL);
  expect("target null q", tgt(&s, 4, KVPOP_AGG_SUM, 0.f, P(), kStubWorkspace, nullptr), KVPOP_EINVAL);
  expect("target null lse", tgt(&s, 4, KVPOP_AGG_SUM, 0.f, P(), kStubWorkspace, P(), nullptr), KVPOP_EINVAL);
  expect("window at INT32_MAX", tgt(&s, INT32_MAX), KVPOP_OK);
}

static void noalloc_cases() {
  kvpop_shape s = shape();
  auto call = [&](const kvpop_shape *sh, int window, int agg, float eps, const void *q, float *lse) {
    return kvpop_future_target_noalloc(sh, q, P(), lse, window, agg, 0, eps, F(), nullptr);
  };
  expect("valid no-allocation target", call(&s, 4, KVPOP_AGG_SUM, 0.f, P(), F()), KVPOP_OK);
  expect("no-allocation null q", call(&s, 4, KVPOP_AGG_SUM, 0.f, nullptr, F()), KVPOP_EINVAL);
  expect("no-allocation null lse", call(&s, 4, KVPOP_AGG_SUM, 0.f, P(), nullptr), KVPOP_EINVAL);
  expect("no-allocation misaligned q", call(&s, 4, KVPOP_AGG_SUM, 0.f, P(8), F()), KVPOP_EINVAL);
  expect("no-allocation negative window", call(&s, -2, KVPOP_AGG_SUM, 0.f, P(), F()), KVPOP_EINVAL);
  expect("no-allocation agg 5", call(&s, 4, 5, 0.f, P(), F()), KVPOP_EINVAL);
  expect("no-allocation eps NaN", call(&s, 4, KVPOP_AGG_SUM, std::nanf(""), P(), F()), KVPOP_EINVAL);
  expect("no-allocation null shape", call(nullptr, 4, KVPOP_AGG_SUM, 0.f, P(), F()), KVPOP_EINVAL);
  // the stand-in sizes grow as B * heads * S * 64 bytes: 2^20 positions at 2 KV heads exceed 64 MiB
  kvpop_shape big = shape(1, 1 << 20, 4, 2, 128);
  expect("no-allocation beyond the scratch", call(&big, 4, KVPOP_AGG_SUM, 0.f, P(), F()), KVPOP_EUNSUPPORTED);
  kvpop_shape mid = shape(1, (1 << 18) + (1 << 16), 4, 2, 128);
  expect("no-allocation SUM within the scratch", call(&mid, 4, KVPOP_AGG_SUM, 0.f, P(), F()), KVPOP_OK);
  expect("no-allocation per-head beyond the scratch", call(&mid, 4, KVPOP_AGG_NONE, 0.f, P(), F()),
         KVPOP_EUNSUPPORTED);
}

static void budget_cases() {
  kvpop_shape s = shape();
  expect("valid budget", bud(&s), KVPOP_OK);
  expect("budget without rank/cutoff outputs", bud(&s, 4, 8, 16, P(), kStubWorkspace, nullptr, nullptr), KVPOP_OK);
  expect("negative sinks", bud(&s, -1), KVPOP_EINVAL);
  expect("negative window", bud(&s, 4, -1), KVPOP_EINVAL);
  expect("negative topk", bud(&s, 4, 8, -1), KVPOP_EINVAL);
  expect("budget workspace too small", bud(&s, 4, 8, 16, P(), 10), KVPOP_EWORKSPACE);
  expect("budget workspace null", bud(&s, 4, 8, 16, nullptr), KVPOP_EWORKSPACE);
  expect("misaligned rank_out", bud(&s, 4, 8, 16, P(), kStubWorkspace, I(2)), KVPOP_EINVAL);
  kvpop_shape f = shape(1, 64, 4, 2, 128, KVPOP_F32);
  expect("fp32 budget at 128", bud(&f), KVPOP_EUNSUPPORTED);
  kvpop_shape big = shape(1, 1 << 23, 4, 2, 128);
  expect("gather offsets above 2^31 bytes", bud(&big), KVPOP_EUNSUPPORTED);
  expect("budget null q", kvpop_budget_mask_fwd(&s, nullptr, P(), P(), F(), 1, 2, 3, P(), F(), nullptr, nullptr, P(),
                                                kStubWorkspace, nullptr), KVPOP_EINVAL);
  expect("budget mask alone", kvpop_budget_mask_fwd(&s, P(), P(), P(), F(), 1, 2, 3, nullptr, nullptr, I(), I(), P(),
                                                  kStubWorkspace, nullptr), KVPOP_OK);
  expect("budget null o only", kvpop_budget_mask_fwd(&s, P(), P(), P(), F(), 1, 2, 3, nullptr, F(), I(), I(), P(),
                                                     kStubWorkspace, nullptr), KVPOP_EINVAL);
  expect("budget null lse only", kvpop_budget_mask_fwd(&s, P(), P(), P(), F(), 1, 2, 3, P(), nullptr, I(), I(), P(),
                                                       kStubWorkspace, nullptr), KVPOP_EINVAL);
  expect("budget null scores", kvpop_budget_mask_fwd(&s, P(), P(), P(), nullptr, 1, 2, 3, P(), F(), nullptr, nullptr,
                                                     P(), kStubWorkspace, nullptr), KVPOP_EINVAL);
  kvpop_lists_layout lay;
  expect("lists layout", kvpop_budget_lists_layout(&s, 4, 8, 16, &lay), KVPOP_OK);
  expect("lists layout null out", kvpop_budget_lists_layout(&s, 4, 8, 16, nullptr), KVPOP_EINVAL);
  expect("lists layout negative topk", kvpop_budget_lists_layout(&s, 4, 8, -16, &lay), KVPOP_EINVAL);
  expect("lists layout null shape", kvpop_budget_lists_layout(nullptr, 4, 8, 16, &lay), KVPOP_EINVAL);
}

static void size_cases() {
  kvpop_shape s = shape();
  expect_size("fwd workspace", kvpop_workspace_size(KVPOP_CALL_FWD_LSE, &s, 0, 0, 0), 0);
  expect_size("target workspace", kvpop_workspace_size(KVPOP_CALL_FUTURE_TARGET, &s, 0, 0, 0), kStubWorkspace);
  expect_size("budget workspace", kvpop_workspace_size(KVPOP_CALL_BUDGET_MASK_FWD, &s, 1, 2, 3), kStubWorkspace);
  expect_size("unknown call", kvpop_workspace_size(99, &s, 0, 0, 0), 0);
  expect_size("negative budget", kvpop_workspace_size(KVPOP_CALL_BUDGET_MASK_FWD, &s, -1, 2, 3), 0);
  kvpop_shape bad = shape(1, 64, 3, 2);
  expect_size("invalid shape", kvpop_workspace_size(KVPOP_CALL_FUTURE_TARGET, &bad, 0, 0, 0), 0);
  expect_size("null shape", kvpop_workspace_size(KVPOP_CALL_FUTURE_TARGET, nullptr, 0, 0, 0), 0);
  expect_size("teacher workspace", kvpop_teacher_workspace_size(1, 2, 64), kStubWorkspace);
  expect_size("teacher workspace bad", kvpop_teacher_workspace_size(0, 2, 64), 0);
  expect_size("loss workspace bad", kvpop_boundary_loss_workspace_size(1, 2, (1 << 24) + 1), 0);
}

static void teacher_loss_cases() {
  const size_t W = kStubWorkspace;
  expect("valid teacher", kvpop_teacher_labels(1, 2, 64, F(), F(), 1, 4, 8, 16, I(), I(), nullptr, nullptr, P(), W,
                                               nullptr), KVPOP_OK);
  expect("teacher batch 0", kvpop_teacher_labels(0, 2, 64, F(), F(), 1, 4, 8, 16, I(), I(), nullptr, nullptr, P(), W,
                                                 nullptr), KVPOP_EINVAL);
  expect("teacher too large", kvpop_teacher_labels(1 << 16, 1 << 10, 1 << 24, F(), F(), 1, 4, 8, 16, I(), I(),
                                                   nullptr, nullptr, P(), W, nullptr), KVPOP_EUNSUPPORTED);
  expect("teacher decay step 0", kvpop_teacher_labels(1, 2, 64, F(), F(), 0, 4, 8, 16, I(), I(), nullptr, nullptr,
                                                      P(), W, nullptr), KVPOP_EINVAL);
  expect("teacher null label", kvpop_teacher_labels(1, 2, 64, F(), F(), 1, 4, 8, 16, nullptr, I(), nullptr, nullptr,
                                                    P(), W, nullptr), KVPOP_EINVAL);
  expect("teacher negative window", kvpop_teacher_labels(1, 2, 64, F(), nullptr, 1, 4, -8, 16, I(), I(), nullptr,
                                                         nullptr, P(), W, nullptr), KVPOP_EINVAL);
  expect("teacher small workspace", kvpop_teacher_labels(1, 2, 64, F(), nullptr, 1, 4, 8, 16, I(), I(), nullptr,
                                                         nullptr, P(), W - 4, nullptr), KVPOP_EWORKSPACE);
  expect("valid loss", kvpop_boundary_loss(1, 2, 64, F(), I(), I(), 4, 8, 16, 0.5f, nullptr, F(), F(), P(), W,
                                           nullptr), KVPOP_OK);
  expect("loss tau 0", kvpop_boundary_loss(1, 2, 64, F(), I(), I(), 4, 8, 16, 0.f, nullptr, F(), F(), P(), W,
                                           nullptr), KVPOP_EINVAL);
  expect("loss tau NaN", kvpop_boundary_loss(1, 2, 64, F(), I(), I(), 4, 8, 16, std::nanf(""), nullptr, F(), F(), P(),
                                             W, nullptr), KVPOP_EINVAL);
  expect("loss tau inf", kvpop_boundary_loss(1, 2, 64, F(), I(), I(), 4, 8, 16, INFINITY, nullptr, F(), F(), P(), W,
                                             nullptr), KVPOP_EINVAL);
  expect("loss null grad", kvpop_boundary_loss(1, 2, 64, F(), I(), I(), 4, 8, 16, 0.5f, nullptr, F(), nullptr, P(),
                                               W, nullptr), KVPOP_EINVAL);
  expect("loss misaligned weight", kvpop_boundary_loss(1, 2, 64, F(), I(), I(), 4, 8, 16, 0.5f, F(1) , F(), F(),
                                                       P(), W, nullptr), KVPOP_EINVAL);
}

static kvpop_decode_shape dshape(int Hq = 8, int Hkv = 2, int D = 128, int dtype = KVPOP_BF16, int s = 4, int w = 8,
                                 int k = 16) {
  kvpop_decode_shape d;
  std::memset(&d, 0, sizeof(d));
  d.batch = 1;
  d.n_q_heads = Hq;
  d.n_kv_heads = Hkv;
  d.head_dim = D;
  d.dtype = dtype;
  d.sinks = s;
  d.window = w;
  d.topk = k;
  return d;
}

static void decode_cases() {
  const size_t W = kStubWorkspace;
  kvpop_decode_shape d = dshape();
  expect_size("decode state", kvpop_decode_state_size(&d), W);
  expect("decode init", kvpop_decode_init(&d, P(), W, nullptr), KVPOP_OK);
  expect("decode step", kvpop_decode_step(&d, P(), W, 0, P(), P(), P(), F(), P(), F(), nullptr), KVPOP_OK);
  expect("decode negative position", kvpop_decode_step(&d, P(), W, -1, P(), P(), P(), F(), P(), F(), nullptr),
         KVPOP_EINVAL);
  expect("decode small state", kvpop_decode_step(&d, P(), W - 1, 0, P(), P(), P(), F(), P(), F(), nullptr),
         KVPOP_EWORKSPACE);
  expect("decode misaligned state", kvpop_decode_init(&d, P(4), W, nullptr), KVPOP_EINVAL);
  expect("decode null score", kvpop_decode_step(&d, P(), W, 0, P(), P(), P(), nullptr, P(), F(), nullptr),
         KVPOP_EINVAL);
  struct { const char *what; kvpop_decode_shape d; kvpop_status want; } table[] = {
      {"decode 16 heads per group", dshape(32, 2), KVPOP_EUNSUPPORTED},
      {"decode group not whole", dshape(6, 4), KVPOP_EINVAL},
      {"decode head_dim 96", dshape(8, 2, 96), KVPOP_EUNSUPPORTED},
      {"decode dtype 9", dshape(8, 2, 128, 9), KVPOP_EUNSUPPORTED},
      {"decode negative topk", dshape(8, 2, 128, KVPOP_BF16, 4, 8, -1), KVPOP_EINVAL},
      {"decode no slots", dshape(8, 2, 128, KVPOP_BF16, 0, 0, 0), KVPOP_EINVAL},
      {"decode 2^20 + 1 slots", dshape(8, 2, 128, KVPOP_BF16, 1, 0, 1 << 20), KVPOP_EUNSUPPORTED},
      {"decode slots overflow int32", dshape(8, 2, 128, KVPOP_BF16, INT32_MAX, INT32_MAX, INT32_MAX),
       KVPOP_EUNSUPPORTED},
  };
  for (auto &c : table) {
    expect(c.what, kvpop_decode_init(&c.d, P(), W, nullptr), c.want);
    expect_size(c.what, kvpop_decode_state_size(&c.d), 0);
  }
  expect("decode null shape", kvpop_decode_init(nullptr, P(), W, nullptr), KVPOP_EINVAL);
}

static void device_cases() {
  kvpop_shape s = shape();
  g_stub_devices = 0;
  expect("no device", fwd(&s), KVPOP_EHIP);
  expect("invalid before device", fwd(&s, nullptr), KVPOP_EINVAL);   // validation first
  g_stub_devices = 1;
  expect("device back", fwd(&s), KVPOP_OK);
}

int main() {
  shape_cases();
  packed_cases();
  pointer_cases();
  target_cases();
  noalloc_cases();
  budget_cases();
  size_cases();
  teacher_loss_cases();
  decode_cases();
  device_cases();
  for (int st = -2; st < 8; ++st) {
    ++g_cases;
    const char *m = kvpop_status_str(st);
    if (m == nullptr || m[0] == '\0') {
      ++g_fail;
      std::printf("FAIL status_str(%d)\n", st);
    }
  }
  if (g_stub_launches == 0) {
    ++g_fail;
    std::printf("FAIL no valid call reached a launcher\n");
  }
  if (g_fail) {
    std::printf("%d of %d cases failed\n", g_fail, g_cases);
    return 1;
  }
  std::printf("all %d cases passed (%d launches)\n", g_cases, g_stub_launches);
  return 0;
}
