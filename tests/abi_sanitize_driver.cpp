// Host-side exercise of the C ABI for an AddressSanitizer + UndefinedBehaviorSanitizer build of the
// library's host code (built and run by tests/test_abi_sanitizers.py on a machine without a GPU).
//
// Every call below either is host-only (layout, workspace sizes, status strings, stage timing) or is
// rejected by argument validation before anything is enqueued, so the fake device pointers are never
// dereferenced. Each check compares the returned status with the one the header specifies; the exit
// status is the number of failed checks (the sanitizers abort on their own findings).
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "pisa.h"

static int g_failed = 0;

static void expect(bool ok, const char* what) {
  if (!ok) {
    std::fprintf(stderr, "FAILED: %s (last error: %s)\n", what, pisa_last_error());
    ++g_failed;
  }
}

static pisa_shape shape(int batch = 1, int seq_len = 1024, int hq = 4, int hkv = 1, int d = 128, int c = 64,
                        int k = 16, int q_tile = 4, int dtype = PISA_BF16) {
  pisa_shape s;
  std::memset(&s, 0, sizeof s);
  s.batch = batch;
  s.seq_len = seq_len;
  s.n_q_heads = hq;
  s.n_kv_heads = hkv;
  s.head_dim = d;
  s.block = c;
  s.top_k = k;
  s.branch = 2;
  s.causal = 1;
  s.q_tile = q_tile;
  s.scale = 0.f;
  s.dtype = dtype;
  return s;
}

int main() {
  void* g = reinterpret_cast<void*>(uintptr_t(1) << 20);              // aligned fake device pointer
  void* odd = reinterpret_cast<void*>((uintptr_t(1) << 20) + 4);       // misaligned
  float* gf = static_cast<float*>(g);
  int32_t* gi = static_cast<int32_t*>(g);
  const size_t big = size_t(1) << 40;

  // ---- layout: level sizes n_0 = ceil(N / C), n_l = ceil(n_{l-1} / 2) up to one root
  const int cases[][2] = {{1024, 32}, {1000, 32}, {65536, 64}, {262144, 64}, {1, 64}, {131328, 64}};
  for (const auto& nc : cases) {
    pisa_shape s = shape(1, nc[0], 4, 1, 128, nc[1], 16, 1);
    int32_t n_levels = 0;
    int64_t off[32];
    int64_t nodes = 0;
    expect(pisa_pyramid_layout(&s, &n_levels, off, &nodes) == PISA_OK, "pyramid_layout ok");
    int64_t n = (nc[0] + nc[1] - 1) / nc[1], total = 0;
    int levels = 0;
    bool match = true;
    while (true) {
      match = match && levels < n_levels && off[levels] == total;
      total += n;
      ++levels;
      if (n == 1) break;
      n = (n + 1) / 2;
    }
    expect(match && levels == n_levels && nodes == total, "pyramid_layout levels and offsets");
  }
  {
    pisa_shape s = shape();
    int32_t nl;
    int64_t nodes;
    expect(pisa_pyramid_layout(&s, &nl, nullptr, &nodes) == PISA_OK, "pyramid_layout optional outputs");
    expect(pisa_pyramid_layout(nullptr, &nl, nullptr, &nodes) == PISA_EINVAL, "pyramid_layout null shape");
  }

  // ---- workspace sizes
  {
    pisa_shape s = shape(1, 65536, 32, 8);
    size_t b = 0;
    for (int op = PISA_OP_SELECT; op <= PISA_OP_ATTN_BWD; ++op)
      expect(pisa_workspace_size(&s, op, &b) == PISA_OK, "workspace_size op");
    expect(pisa_workspace_size(&s, 99, &b) == PISA_EINVAL, "workspace_size unknown op");
    expect(pisa_workspace_size(&s, PISA_OP_SELECT, nullptr) == PISA_EINVAL, "workspace_size null out");
  }

  // ---- invalid shapes: the status from pisa_workspace_size and from every enqueueing call
  struct Bad {
    pisa_shape s;
    pisa_status st;
  };
  Bad bad[] = {
      {shape(0), PISA_EINVAL},
      {shape(1, 0), PISA_EINVAL},
      {shape(1, 1024, 6, 4), PISA_EINVAL},
      {shape(1, 1024, 3, 1), PISA_EUNSUPPORTED},
      {shape(1, 1024, 32, 1, 128, 64, 16, 1), PISA_EUNSUPPORTED},
      {shape(1, 1024, 4, 1, 96), PISA_EUNSUPPORTED},
      {shape(1, 1024, 4, 1, 128, 16), PISA_EUNSUPPORTED},
      {shape(1, 1024, 4, 1, 128, 64, 0), PISA_EINVAL},
      {shape(1, 1024, 4, 1, 128, 64, 33), PISA_EUNSUPPORTED},
      {shape(1, 1024, 4, 1, 128, 64, 16, 3), PISA_EINVAL},
      {shape(1, 1024, 4, 1, 128, 64, 16, 8), PISA_EUNSUPPORTED},
      {shape(1, 1024, 4, 1, 128, 64, 16, 4, 7), PISA_EINVAL},
      {shape(64, 1 << 17, 64, 16), PISA_EUNSUPPORTED},
  };
  bad[0].s.branch = 2;
  {
    pisa_shape nc = shape();
    nc.causal = 0;
    size_t b = 0;
    expect(pisa_workspace_size(&nc, PISA_OP_SELECT, &b) == PISA_EUNSUPPORTED, "non-causal shape");
    expect(pisa_select(&nc, g, g, gf, gi, nullptr, g, big, nullptr) == PISA_EUNSUPPORTED, "non-causal select");
  }
  for (const Bad& x : bad) {
    size_t b = 0;
    expect(pisa_workspace_size(&x.s, PISA_OP_SELECT, &b) == x.st, "bad shape: workspace_size");
    expect(pisa_select(&x.s, g, g, gf, gi, nullptr, g, big, nullptr) == x.st, "bad shape: select");
    expect(pisa_build_pyramid(&x.s, g, nullptr, gf, nullptr, nullptr) == x.st, "bad shape: build_pyramid");
    expect(pisa_sparse_attn(&x.s, g, g, g, gi, g, nullptr, g, big, nullptr) == x.st, "bad shape: sparse_attn");
    expect(bsa_select(&x.s, g, g, gi, g, big, nullptr) == x.st, "bad shape: bsa_select");
    expect(pisa_select_noalloc(&x.s, g, g, gf, gi, nullptr, nullptr) == x.st || x.st == PISA_EINVAL,
           "bad shape: select_noalloc");
  }
  {
    pisa_shape s = shape();
    s.branch = 3;
    size_t b;
    expect(pisa_workspace_size(&s, PISA_OP_SELECT, &b) == PISA_EUNSUPPORTED, "branch 3");
    s = shape();
    s.scale = -1.f;
    expect(pisa_workspace_size(&s, PISA_OP_SELECT, &b) == PISA_EINVAL, "negative scale");
    s.scale = INFINITY;
    expect(pisa_workspace_size(&s, PISA_OP_SELECT, &b) == PISA_EINVAL, "infinite scale");
  }

  // ---- null and misaligned pointers, missing or short workspaces
  {
    pisa_shape s = shape();
    expect(pisa_select(&s, nullptr, g, gf, gi, nullptr, g, big, nullptr) == PISA_EINVAL, "select null q");
    expect(pisa_select(&s, odd, g, gf, gi, nullptr, g, big, nullptr) == PISA_EINVAL, "select misaligned q");
    expect(pisa_select(&s, g, g, gf, gi, static_cast<float*>(odd), g, big, nullptr) == PISA_EINVAL,
           "select misaligned sel_lse");
    expect(pisa_select(nullptr, g, g, gf, gi, nullptr, g, big, nullptr) == PISA_EINVAL, "select null shape");
    expect(pisa_build_pyramid(&s, g, nullptr, nullptr, nullptr, nullptr) == PISA_EINVAL, "pyramid null mean");
    expect(pisa_sparse_attn(&s, g, g, nullptr, gi, g, nullptr, g, big, nullptr) == PISA_EINVAL, "attn null v");
    expect(bsa_select(&s, g, g, nullptr, g, big, nullptr) == PISA_EINVAL, "bsa null sel");
    size_t need = 0;
    pisa_workspace_size(&s, PISA_OP_SELECT, &need);
    expect(pisa_select(&s, g, g, gf, gi, nullptr, g, need - 1, nullptr) == PISA_EWORKSPACE, "select short ws");
    expect(pisa_select(&s, g, g, gf, gi, nullptr, nullptr, need, nullptr) == PISA_EWORKSPACE, "select null ws");
    pisa_workspace_size(&s, PISA_OP_ATTN, &need);
    expect(pisa_sparse_attn(&s, g, g, g, gi, g, nullptr, g, need - 1, nullptr) == PISA_EWORKSPACE, "attn short ws");
    pisa_workspace_size(&s, PISA_OP_BSA, &need);
    expect(bsa_select(&s, g, g, gi, g, need - 1, nullptr) == PISA_EWORKSPACE, "bsa short ws");
  }

  // ---- host lengths (pyramid build and decode)
  {
    pisa_shape s = shape(2);
    const int32_t over[2] = {5, 2000}, neg[2] = {-1, 3}, full[2] = {1024, 3}, ok[2] = {1000, 3};
    expect(pisa_build_pyramid(&s, g, over, gf, gf, nullptr) == PISA_EINVAL, "lens above capacity");
    expect(pisa_build_pyramid(&s, g, neg, gf, gf, nullptr) == PISA_EINVAL, "negative lens");
    expect(pisa_decode_step(&s, full, g, g, g, g, g, gf, gf, g, nullptr, nullptr, 0, nullptr) == PISA_EINVAL,
           "decode at capacity");
    expect(pisa_decode_step(&s, nullptr, g, g, g, g, g, gf, gf, g, nullptr, nullptr, 0, nullptr) == PISA_EINVAL,
           "decode null lens");
    expect(pisa_decode_step(&s, ok, g, g, g, g, g, gf, gf, g, nullptr, nullptr, 0, nullptr) == PISA_EWORKSPACE,
           "decode without workspace");
    size_t need = 0;
    expect(pisa_workspace_size(&s, PISA_OP_DECODE, &need) == PISA_OK && need > 0, "decode workspace size");
    expect(pisa_decode_step(&s, ok, g, g, g, g, g, gf, gf, g, nullptr, g, need - 1, nullptr) == PISA_EWORKSPACE,
           "decode short workspace");
  }

  // ---- the other entry points' validation
  {
    pisa_shape s = shape();
    expect(pisa_select_noalloc_max_bytes() == size_t(64) << 20, "noalloc max bytes");
    pisa_shape big_s = shape(1, 65536, 32, 8);
    expect(pisa_select_noalloc(&big_s, g, g, gf, gi, nullptr, nullptr) == PISA_EUNSUPPORTED, "noalloc too large");
    pisa_shape f32 = shape(1, 1024, 4, 1, 128, 64, 16, 4, PISA_FP32);
    expect(pisa_sparse_attn_backward(&f32, g, g, g, gi, g, gf, g, g, g, g, g, big, nullptr) == PISA_EUNSUPPORTED,
           "backward fp32");
    size_t need = 0;
    pisa_workspace_size(&s, PISA_OP_ATTN_BWD, &need);
    expect(pisa_sparse_attn_backward(&s, g, g, g, gi, g, gf, g, g, g, g, g, need - 1, nullptr) == PISA_EWORKSPACE,
           "backward short workspace");
    expect(pisa_sparse_attn_backward(&s, g, g, g, gi, g, nullptr, g, g, g, g, g, big, nullptr) == PISA_EINVAL,
           "backward null o_lse");
    expect(pisa_flat_leaf_lse(&s, g, g, nullptr, 4, gf, gf, nullptr) == PISA_EINVAL, "flat_leaf_lse null positions");
    expect(pisa_flat_leaf_lse(&s, g, g, gi, -1, gf, gf, nullptr) == PISA_EINVAL, "flat_leaf_lse negative count");
    expect(pisa_selection_quality(&s, gf, gf, gi, 4, gi, gi, gf, nullptr, nullptr) == PISA_EINVAL,
           "quality null mass");
    expect(pisa_build_pyramid_pooled(&s, g, 7, gf, nullptr, nullptr) == PISA_EINVAL, "pooled unknown pool");
    expect(pisa_build_pyramid_pooled(&s, g, PISA_POOL_MAX, gf, gf, nullptr) == PISA_EUNSUPPORTED,
           "pooled max with variance");
    pisa_variant v{PISA_SCORE_MEAN_VAR, PISA_BUDGET_FIXED, -1};
    expect(pisa_select_variant(&s, &v, g, g, gf, nullptr, gi, nullptr) == PISA_EINVAL, "variant without variance");
    v = pisa_variant{9, PISA_BUDGET_FIXED, -1};
    expect(pisa_select_variant(&s, &v, g, g, gf, gf, gi, nullptr) == PISA_EINVAL, "variant unknown score");
    expect(pisa_select_variant(&s, nullptr, g, g, gf, gf, gi, nullptr) == PISA_EINVAL, "variant null options");
    const int64_t* gu = static_cast<const int64_t*>(g);
    size_t tneed = 0, sneed = 0;
    pisa_shape s1 = shape(1, 1024, 4, 1, 128, 64, 16, 1);
    expect(pisa_workspace_size(&s, PISA_OP_TRACE, &tneed) == PISA_OK &&
               pisa_workspace_size(&s1, PISA_OP_SELECT, &sneed) == PISA_OK && tneed == sneed && tneed > 0,
           "trace workspace is the q_tile 1 select workspace");
    expect(pisa_select_trace(&s, g, g, gf, gu, -1, gi, g, big, nullptr) == PISA_EINVAL, "trace negative count");
    expect(pisa_select_trace(&s, nullptr, nullptr, nullptr, nullptr, 0, nullptr, nullptr, 0, nullptr) == PISA_OK,
           "trace of no units");
    expect(pisa_select_trace(&s, g, g, gf, nullptr, 4, gi, g, big, nullptr) == PISA_EINVAL, "trace null units");
    expect(pisa_select_trace(&s, g, g, gf, gu, 4, nullptr, g, big, nullptr) == PISA_EINVAL, "trace null output");
    expect(pisa_select_trace(&s, g, g, gf, gu, 4, gi, g, tneed - 1, nullptr) == PISA_EWORKSPACE,
           "trace short workspace");
    expect(pisa_select_trace(nullptr, g, g, gf, gu, 4, gi, g, big, nullptr) == PISA_EINVAL, "trace null shape");
  }

  // ---- status strings, last error, stage timing
  for (int st = 0; st >= -4; --st) expect(pisa_status_string(st) != nullptr, "status string");
  expect(pisa_status_string(-99) != nullptr && pisa_status_string(12345) != nullptr, "unknown status string");
  expect(pisa_last_error() != nullptr, "last error");
  expect(pisa_stage_timing(0) == PISA_OK, "stage timing off");
  char names[4][32];
  double tot[4];
  int32_t cnt[4];
  expect(pisa_stage_times(names, tot, cnt, 4) >= 0, "stage times");
  expect(pisa_stage_times(names, tot, cnt, -1) < 0, "stage times negative cap");

  std::printf("abi sanitize driver: %d failed checks\n", g_failed);
  return g_failed;
}
