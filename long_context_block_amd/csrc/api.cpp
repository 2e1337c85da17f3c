// C ABI of libpisa.so: argument validation, workspace layout and launch sequencing.
// Validation completes before anything is enqueued; the kernels live in the .hip files.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <algorithm>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "pisa.h"
#include "internal.hpp"

namespace {

thread_local std::string g_last_error;

pisa_status fail(pisa_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

pisa_status ok() {
  g_last_error.clear();
  return PISA_OK;
}

// ---- optional stage timing (per calling thread)
struct StageEvent {
  std::string name;
  hipEvent_t a, b;
};
struct StageTimer {
  bool on = false;
  std::vector<StageEvent> pending;
  std::vector<hipEvent_t> pool;
  std::map<std::string, std::pair<double, int>> totals;
  hipEvent_t get() {
    if (!pool.empty()) {
      hipEvent_t e = pool.back();
      pool.pop_back();
      return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
  }
};
thread_local StageTimer g_timer;

// Records events around one launcher when stage timing is on.
struct Stage {
  hipStream_t s;
  const char* name;
  hipEvent_t a = nullptr;
  // an event that cannot be recorded drops this stage's interval (the timer is advisory)
  Stage(hipStream_t st, const char* n) : s(st), name(n) {
    if (g_timer.on) {
      a = g_timer.get();
      if (a && hipEventRecord(a, s) != hipSuccess) {
        g_timer.pool.push_back(a);
        a = nullptr;
      }
    }
  }
  ~Stage() {
    if (a) {
      hipEvent_t b = g_timer.get();
      if (b && hipEventRecord(b, s) == hipSuccess) {
        g_timer.pending.push_back({name, a, b});
      } else {
        g_timer.pool.push_back(a);
        if (b) g_timer.pool.push_back(b);
      }
    }
  }
};

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

#define PISA_CHECK_PTR(p, name)                                                     \
  do {                                                                              \
    if (!(p)) return fail(PISA_EINVAL, "%s: null pointer", name);                   \
    if (!aligned16(p)) return fail(PISA_EINVAL, "%s: not 16-byte aligned", name);   \
  } while (0)

#define PISA_CHECK_OPT_PTR(p, name)                                                  \
  do {                                                                              \
    if ((p) && !aligned16(p)) return fail(PISA_EINVAL, "%s: not 16-byte aligned", name); \
  } while (0)

struct Plan {
  pisa::SelDims sd;
  long long U;       // units B*Hkv*N
  long long BH;
  int n1_buckets;    // buckets per KV head and chunk for the selection regroup (level-1 nodes, at least 1)
  int nch;           // position chunks per KV head
  size_t elem;       // bytes per Q/K/V element
};

pisa_status make_levels(long long n_tokens, int C, pisa::Levels* lv) {
  std::memset(lv, 0, sizeof(*lv));
  long long n = (n_tokens + C - 1) / C;
  if (n < 1) n = 1;
  int l = 0;
  long long off = 0;
  while (true) {
    if (l >= pisa::kMaxLevels) return fail(PISA_EUNSUPPORTED, "pyramid deeper than %d levels", pisa::kMaxLevels);
    if (n > 0x7fffffffLL) return fail(PISA_EUNSUPPORTED, "too many leaves");
    lv->n[l] = (int)n;
    lv->off[l] = off;
    off += n;
    ++l;
    if (n == 1) break;
    n = (n + 1) / 2;
  }
  lv->n_levels = l;
  lv->nodes = off;
  long long roff = 0;
  for (int j = 0; j < l; ++j) {
    lv->roff[j] = roff;
    roff += lv->n[j] >= 4 ? (lv->n[j] + 3) / 4 * 4 : lv->n[j];
  }
  lv->rnodes = (roff + 3) / 4 * 4;
  return PISA_OK;
}

pisa_status plan(const pisa_shape* s, Plan* pl) {
  if (!s) return fail(PISA_EINVAL, "shape: null pointer");
  if (s->batch < 1 || s->seq_len < 1 || s->n_q_heads < 1 || s->n_kv_heads < 1)
    return fail(PISA_EINVAL, "batch, seq_len and head counts must be >= 1");
  if (s->n_q_heads % s->n_kv_heads) return fail(PISA_EINVAL, "n_q_heads %% n_kv_heads != 0");
  const int G = s->n_q_heads / s->n_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8 && G != 16)
    return fail(PISA_EUNSUPPORTED, "query heads per KV head must be 1, 2, 4, 8 or 16 (got %d)", G);
  if (s->head_dim != 64 && s->head_dim != 128) return fail(PISA_EUNSUPPORTED, "head_dim must be 64 or 128");
  if (s->block != 32 && s->block != 64) return fail(PISA_EUNSUPPORTED, "block must be 32 or 64");
  if (s->top_k < 1) return fail(PISA_EINVAL, "top_k must be >= 1");
  if (s->top_k > 32) return fail(PISA_EUNSUPPORTED, "top_k must be <= 32");
  if (s->branch != 2) return fail(PISA_EUNSUPPORTED, "branch (merge factor) must be 2");
  if (s->causal != 1) return fail(PISA_EUNSUPPORTED, "causal must be 1 (the selection and attention are causal)");
  const int qt = s->q_tile;
  if (qt != 1 && qt != 2 && qt != 4 && qt != 8 && qt != 16) return fail(PISA_EINVAL, "q_tile must be 1, 2, 4, 8 or 16");
  if (qt * G > 16) return fail(PISA_EUNSUPPORTED, "q_tile * G must be <= 16");
  if (s->dtype != PISA_FP32 && s->dtype != PISA_BF16) return fail(PISA_EINVAL, "dtype must be PISA_FP32 or PISA_BF16");
  if (!(s->scale >= 0.f) || !std::isfinite(s->scale)) return fail(PISA_EINVAL, "scale must be finite and >= 0");
  const long long U = (long long)s->batch * s->n_kv_heads * s->seq_len;
  if (U >= (1LL << 27)) return fail(PISA_EUNSUPPORTED, "batch * n_kv_heads * seq_len must be < 2^27");
  if (U * s->top_k >= (1LL << 31)) return fail(PISA_EUNSUPPORTED, "units * top_k must be < 2^31");
  Plan p{};
  p.sd.B = s->batch;
  p.sd.Hq = s->n_q_heads;
  p.sd.Hkv = s->n_kv_heads;
  p.sd.G = G;
  p.sd.N = s->seq_len;
  p.sd.D = s->head_dim;
  p.sd.C = s->block;
  p.sd.K = s->top_k;
  p.sd.q_tile = qt;
  p.sd.scale = s->scale > 0.f ? s->scale : 1.f / std::sqrt((float)s->head_dim);
  p.sd.bf16 = s->dtype == PISA_BF16;
  pisa_status st = make_levels(s->seq_len, s->block, &p.sd.lv);
  if (st != PISA_OK) return st;
  p.U = U;
  p.BH = (long long)s->batch * s->n_kv_heads;
  p.n1_buckets = p.sd.lv.n_levels > 1 ? p.sd.lv.n[1] : 1;
  p.elem = p.sd.bf16 ? 2 : 4;
  // Pairs may be bucketed per position chunk (2^chunk_log2 positions) so that a run of buckets gathers
  // the queries of one chunk. The attention keeps one chunk per KV head (each chunk re-reads the K and V
  // of the leaves its queries select: 7% slower at 2^14 positions); the selection sets its own below.
  p.sd.chunk_log2 = 30;
  p.nch = 1;
  *pl = p;
  return PISA_OK;
}

// The selection's leaf stage buckets its pairs by position chunks as well: consecutive runs then gather
// the queries of one chunk, which stay in the caches (its leaf stage and regroup together 3% faster at 64K
// with 2^14-position chunks than with one chunk per KV head; the leaf tile is staged once per run either
// way). A sequence takes four chunks, of at least 2^14 positions: more chunks shorten the runs (more key
// tiles staged per pair) and lengthen the regroup's bucket scan (at 256K, 2^16 positions take the
// selection from 16.9 to 16.6 ms against 2^14).
constexpr int kSelectChunkLog2Min = 14;
static int select_chunk_log2(long long N) {
  int l = 0;
  while ((1LL << l) < N) ++l;  // ceil(log2 N)
  return l - 2 > kSelectChunkLog2Min ? l - 2 : kSelectChunkLog2Min;
}
static pisa_status select_plan(const pisa_shape* s, Plan* p) {
  const pisa_status st = plan(s, p);
  if (st != PISA_OK) return st;
  const int cl = select_chunk_log2(p->sd.N);
  p->sd.chunk_log2 = cl;
  p->nch = (int)(((long long)p->sd.N + (1LL << cl) - 1) >> cl);
  return PISA_OK;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Workspace carving: a list of (pointer, bytes) regions, each 256-byte aligned.
struct Carver {
  char* base;
  size_t off = 0;
  explicit Carver(void* b) : base((char*)b) {}
  void* take(size_t bytes) {
    void* p = base ? base + off : nullptr;
    off += align256(bytes);
    return p;
  }
};

struct SelectWs {
  uint16_t* hilo;
  float* norms;
  int* hexp;
  float* part_max;
  int* kept;
  int* counts;
  int* offsets;
  int* ranks;
  uint32_t* pairs;
  float* leaf_lse;
};

size_t carve_select(const Plan& p, void* ws, SelectWs* w) {
  Carver c(ws);
  SelectWs x{};
  if (p.sd.bf16) {
    x.hilo = (uint16_t*)c.take((size_t)p.BH * p.sd.lv.rnodes * 2 * p.sd.D * 2);
    x.norms = (float*)c.take((size_t)p.BH * p.sd.lv.rnodes * 4);
    x.hexp = (int*)c.take((size_t)p.BH * 4);
    x.part_max = (float*)c.take((size_t)p.BH * 64 * 4);
  }
  if (p.sd.q_tile > 1) {
    const size_t pairs = (size_t)p.U * p.sd.K;
    const size_t NB = (size_t)p.BH * p.nch * p.n1_buckets;
    x.kept = (int*)c.take(pairs * 4);
    x.counts = (int*)c.take(NB * 4);
    x.offsets = (int*)c.take((NB + 1) * 4);
    x.ranks = (int*)c.take(pairs * 4);
    x.pairs = (uint32_t*)c.take(pairs * 4);
    x.leaf_lse = (float*)c.take(pairs * 2 * p.sd.G * 4);
  }
  if (w) *w = x;
  return c.off;
}

struct AttnWs {
  int* counts;
  int* offsets;
  int* ranks;
  uint32_t* pairs;
  void* part;
  float* part_lse;
};

size_t carve_attn(const Plan& p, void* ws, AttnWs* w) {
  Carver c(ws);
  AttnWs x{};
  const size_t pairs = (size_t)p.U * p.sd.K;
  const size_t NB = (size_t)p.BH * p.nch * p.sd.lv.n[0];
  x.counts = (int*)c.take(NB * 4);
  x.offsets = (int*)c.take((NB + 1) * 4);
  x.ranks = (int*)c.take(pairs * 4);  // after the regroup: each pair's index in the sorted list
  x.pairs = (uint32_t*)c.take(pairs * 4);
  x.part = c.take(pairs * p.sd.G * p.sd.D * p.elem);  // rows in sorted-pair order
  x.part_lse = (float*)c.take(pairs * p.sd.G * 4);
  if (w) *w = x;
  return c.off;
}

struct AttnBwdWs {
  int* counts;
  int* offsets;
  int* ranks;
  uint32_t* pairs;
  float* dsum;
  float* acc;      // dk accumulators, then dv accumulators
  float* kv_part;  // per-task dK / dV sums of leaves shared between tasks
  void* part;
};

size_t carve_attn_bwd(const Plan& p, void* ws, AttnBwdWs* w) {
  Carver c(ws);
  AttnBwdWs x{};
  const size_t pairs = (size_t)p.U * p.sd.K;
  const size_t NB = (size_t)p.BH * p.nch * p.sd.lv.n[0];
  x.counts = (int*)c.take(NB * 4);
  x.offsets = (int*)c.take((NB + 1) * 4);
  x.ranks = (int*)c.take(pairs * 4);
  x.pairs = (uint32_t*)c.take(pairs * 4);
  x.dsum = (float*)c.take((size_t)p.sd.B * p.sd.Hq * p.sd.N * 4);
  x.acc = (float*)c.take((size_t)2 * p.U * p.sd.D * 4);
  x.kv_part = (float*)c.take(pisa::attn_backward_kv_part_bytes(p.sd));
  x.part = c.take(pairs * p.sd.G * p.sd.D * 2);
  if (w) *w = x;
  return c.off;
}

struct BsaWs {
  float* mean;
  uint16_t* hilo;
};

size_t carve_bsa(const Plan& p, void* ws, BsaWs* w) {
  Carver c(ws);
  BsaWs x{};
  const size_t rows = (size_t)p.BH * p.sd.lv.n[0];
  x.mean = (float*)c.take(rows * p.sd.D * 4);
  if (p.sd.bf16) x.hilo = (uint16_t*)c.take(rows * 2 * p.sd.D * 2);
  if (w) *w = x;
  return c.off;
}

// The attention and its backward run over chunks of consecutive (sequence, KV head) slices, so that
// their workspace (which holds a partial row per selected leaf, K times the slice's output) stays near
// kAttnChunkBytes whatever the batch and head count. Q, K, V, sel, O and the gradients are contiguous per
// slice ([B, H, N, ...] with the G query heads of KV head r at r G .. r G + G - 1), so a chunk of S
// slices starting at flat slice f is the shape (B = S, Hkv = 1, Hq = G) on pointers offset by f slices;
// every kernel computes a (unit, leaf) pair and a unit's merge independently of how units are grouped.
// The budget is a few percent of the device memory: a 64K-token prefill with 8 KV heads is one chunk,
// a batch of eight 256K-token sequences takes 22 chunks of 3 slices (13 GB instead of 280 GB).
constexpr size_t kAttnChunkBytes = size_t(16) << 30;

// The chunk budget: kAttnChunkBytes, or less when the environment variable PISA_ATTN_CHUNK_MIB holds a
// smaller positive number of MiB (read at every call, so the workspace query and the call agree as long
// as it does not change in between).
size_t attn_chunk_bytes() {
  const char* e = std::getenv("PISA_ATTN_CHUNK_MIB");
  if (!e || !*e) return kAttnChunkBytes;
  char* end = nullptr;
  const unsigned long long mib = std::strtoull(e, &end, 10);
  if (end == e || *end || mib == 0 || mib >= (kAttnChunkBytes >> 20)) return kAttnChunkBytes;
  return (size_t)mib << 20;
}

struct AttnChunks {
  long long slices;  // B * Hkv
  long long per;     // slices per chunk
  Plan cp;           // plan of a full chunk
};

// Chunking of shape s for a workspace carve function: the fewest chunks whose workspace fits
// kAttnChunkBytes (at least one slice per chunk), with the slices spread evenly over them.
template <class Carve>
pisa_status attn_chunks(const pisa_shape* s, Carve carve, AttnChunks* out) {
  pisa_shape one = *s;
  one.batch = 1;
  one.n_kv_heads = 1;
  one.n_q_heads = s->n_q_heads / s->n_kv_heads;
  Plan p1;
  pisa_status st = plan(&one, &p1);
  if (st != PISA_OK) return st;
  AttnChunks c;
  c.slices = (long long)s->batch * s->n_kv_heads;
  const size_t per_slice = carve(p1);
  long long fit = per_slice ? (long long)(attn_chunk_bytes() / per_slice) : c.slices;
  if (fit < 1) fit = 1;
  if (fit > c.slices) fit = c.slices;
  const long long chunks = (c.slices + fit - 1) / fit;
  c.per = (c.slices + chunks - 1) / chunks;
  pisa_shape full = one;
  full.batch = (int32_t)c.per;
  st = plan(&full, &c.cp);
  if (st != PISA_OK) return st;
  *out = c;
  return PISA_OK;
}

// Plan of the chunk of n slices (n <= per).
pisa_status chunk_plan(const AttnChunks& c, long long n, Plan* p) {
  if (n == c.per) {
    *p = c.cp;
    return PISA_OK;
  }
  pisa_shape sub{};
  sub.batch = (int32_t)n;
  sub.seq_len = c.cp.sd.N;
  sub.n_q_heads = c.cp.sd.G;
  sub.n_kv_heads = 1;
  sub.head_dim = c.cp.sd.D;
  sub.block = c.cp.sd.C;
  sub.top_k = c.cp.sd.K;
  sub.branch = 2;
  sub.causal = 1;
  sub.q_tile = c.cp.sd.q_tile;
  sub.scale = c.cp.sd.scale;
  sub.dtype = c.cp.sd.bf16 ? PISA_BF16 : PISA_FP32;
  return plan(&sub, p);
}

struct DecodeWs {
  int* ticket;
  float* part_lse;
  float* part_o;
};

// Decode workspace: the arrival counters first (the part that must be zero before the first step),
// then the per-candidate-leaf partial results.
size_t carve_decode(const Plan& p, void* ws, DecodeWs* w) {
  Carver c(ws);
  DecodeWs x{};
  const size_t cand = (size_t)p.BH * 2 * p.sd.K;
  x.ticket = (int*)c.take(p.BH * 4);
  x.part_lse = (float*)c.take(cand * p.sd.G * 4);
  x.part_o = (float*)c.take(cand * p.sd.G * p.sd.D * 4);
  if (w) *w = x;
  return c.off;
}

pisa_status check_ws(size_t need, const void* ws, size_t ws_bytes) {
  if (need == 0) return PISA_OK;
  if (!ws) return fail(PISA_EWORKSPACE, "workspace is null, %zu bytes needed", need);
  if (!aligned16(ws)) return fail(PISA_EINVAL, "workspace: not 16-byte aligned");
  if (ws_bytes < need) return fail(PISA_EWORKSPACE, "workspace has %zu bytes, %zu needed", ws_bytes, need);
  return PISA_OK;
}

pisa_status hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(PISA_EHIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

pisa_status lens_arg(const int32_t* host_lens, int B, int Hkv, int lo, int hi_incl, pisa::LensArg* la) {
  std::memset(la, 0, sizeof(*la));
  la->hkv = Hkv;
  if (!host_lens) return PISA_OK;
  if (B > pisa::kMaxLensBatch) return fail(PISA_EUNSUPPORTED, "host_lens supports batch <= %d", pisa::kMaxLensBatch);
  la->has = 1;
  for (int b = 0; b < B; ++b) {
    if (host_lens[b] < lo || host_lens[b] > hi_incl)
      return fail(PISA_EINVAL, "host_lens[%d] = %d outside [%d, %d]", b, host_lens[b], lo, hi_incl);
    la->len[b] = host_lens[b];
  }
  return PISA_OK;
}

// ---- scratch of pisa_select_noalloc
// One copy of the array per GPU, held until the process ends. Host code never passes the array's name
// to a kernel (on the host it only stands for the symbol); it passes the device address that
// hipGetSymbolAddress returns for the current device, resolved once per device.
constexpr size_t kNoAllocScratchBytes = size_t(64) << 20;
constexpr int kMaxDevices = 64;
__device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

pisa_status scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(PISA_EHIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(PISA_EUNSUPPORTED, "device %d: at most %d devices", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) return fail(PISA_EHIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return PISA_OK;
}

}  // namespace

extern "C" {

const char* pisa_status_string(int32_t s) {
  switch (s) {  // any int: callers may pass a value that is not a pisa_status
    case PISA_OK: return "PISA_OK";
    case PISA_EINVAL: return "PISA_EINVAL: invalid argument";
    case PISA_EUNSUPPORTED: return "PISA_EUNSUPPORTED: unsupported shape";
    case PISA_EWORKSPACE: return "PISA_EWORKSPACE: workspace missing or too small";
    case PISA_EHIP: return "PISA_EHIP: HIP launch failed";
  }
  return "unknown pisa_status";
}

const char* pisa_last_error(void) { return g_last_error.c_str(); }

pisa_status pisa_pyramid_layout(const pisa_shape* shape, int32_t* n_levels, int64_t* level_offset,
                                int64_t* nodes_per_head) {
  Plan p;
  pisa_status st = plan(shape, &p);
  if (st != PISA_OK) return st;
  if (n_levels) *n_levels = p.sd.lv.n_levels;
  if (level_offset)
    for (int l = 0; l < pisa::kMaxLevels; ++l) level_offset[l] = l < p.sd.lv.n_levels ? p.sd.lv.off[l] : -1;
  if (nodes_per_head) *nodes_per_head = p.sd.lv.nodes;
  return ok();
}

// The traced walk's plan: the shape at q_tile 1 (its workspace is the routing planes alone).
static pisa_status trace_plan(const pisa_shape* shape, Plan* p) {
  if (!shape) return fail(PISA_EINVAL, "shape: null pointer");
  pisa_shape s1 = *shape;
  s1.q_tile = 1;
  return plan(&s1, p);
}

pisa_status pisa_workspace_size(const pisa_shape* shape, int32_t op, size_t* bytes) {
  if (!bytes) return fail(PISA_EINVAL, "bytes: null pointer");
  Plan p;
  pisa_status st = op == PISA_OP_TRACE ? trace_plan(shape, &p) : op == PISA_OP_SELECT ? select_plan(shape, &p)
                                                                                   : plan(shape, &p);
  if (st != PISA_OK) return st;
  switch (op) {
    case PISA_OP_SELECT: *bytes = carve_select(p, nullptr, nullptr); break;
    case PISA_OP_ATTN: {
      AttnChunks c;
      st = attn_chunks(shape, [](const Plan& q) { return carve_attn(q, nullptr, nullptr); }, &c);
      if (st != PISA_OK) return st;
      *bytes = carve_attn(c.cp, nullptr, nullptr);
      break;
    }
    case PISA_OP_DECODE: *bytes = carve_decode(p, nullptr, nullptr); break;
    case PISA_OP_TRACE: *bytes = carve_select(p, nullptr, nullptr); break;
    case PISA_OP_BSA: *bytes = carve_bsa(p, nullptr, nullptr); break;
    case PISA_OP_ATTN_BWD: {
      AttnChunks c;
      st = attn_chunks(shape, [](const Plan& q) { return carve_attn_bwd(q, nullptr, nullptr); }, &c);
      if (st != PISA_OK) return st;
      *bytes = carve_attn_bwd(c.cp, nullptr, nullptr);
      break;
    }
    default: return fail(PISA_EINVAL, "unknown op %d", op);
  }
  return ok();
}

pisa_status pisa_build_pyramid(const pisa_shape* shape, const void* k, const int32_t* host_lens, float* pyr_mean,
                               float* pyr_sum, void* stream) {
  Plan p;
  pisa_status st = plan(shape, &p);
  if (st != PISA_OK) return st;
  PISA_CHECK_PTR(k, "k");
  PISA_CHECK_PTR(pyr_mean, "pyr_mean");
  PISA_CHECK_OPT_PTR(pyr_sum, "pyr_sum");
  pisa::LensArg la;
  st = lens_arg(host_lens, p.sd.B, p.sd.Hkv, 0, p.sd.N, &la);
  if (st != PISA_OK) return st;
  pisa::PyrDims pd{(int)p.BH, p.sd.N, p.sd.C, p.sd.D, p.sd.lv};
  hipError_t e;
  {
    Stage sc((hipStream_t)stream, "pyramid");
    e = pisa::launch_pool(k, p.sd.bf16, pd, la, p.sd.lv.n_levels - 1, pyr_mean, pyr_sum, (hipStream_t)stream);
  }
  return hip_status(e, "pisa_build_pyramid");
}

pisa_status pisa_select(const pisa_shape* shape, const void* q, const void* k, const float* pyr_mean, int32_t* sel,
                        float* sel_lse, void* ws, size_t ws_bytes, void* stream) {
  Plan p;
  pisa_status st = select_plan(shape, &p);
  if (st != PISA_OK) return st;
  PISA_CHECK_PTR(q, "q");
  PISA_CHECK_PTR(k, "k");
  PISA_CHECK_PTR(pyr_mean, "pyr_mean");
  PISA_CHECK_PTR(sel, "sel");
  PISA_CHECK_OPT_PTR(sel_lse, "sel_lse");
  const size_t need = carve_select(p, nullptr, nullptr);
  st = check_ws(need, ws, ws_bytes);
  if (st != PISA_OK) return st;
  SelectWs w;
  carve_select(p, ws, &w);
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = hipSuccess;
  const void* nodes = pyr_mean;
  if (p.sd.bf16) {
    {
      Stage sc(s, "route_planes");
      e = pisa::launch_route_planes(pyr_mean, p.BH, p.sd.lv, p.sd.D, w.part_max, w.hexp, w.hilo, w.norms, s);
    }
    if (e != hipSuccess) return hip_status(e, "route_planes");
    nodes = w.hilo;
  }
  if (p.sd.q_tile == 1) {
    {
      Stage sc(s, "route_fused_leaf");
      e = pisa::launch_route(p.sd, q, k, nodes, w.norms, w.hexp, true, nullptr, sel, sel_lse, s);
    }
    return hip_status(e, "route (fused leaf stage)");
  }
  {
    Stage sc(s, "route");
    if (pisa::route_group_supported(p.sd))
      e = pisa::launch_route_group(p.sd, q, nodes, w.norms, w.hexp, w.kept, s);
    else
      e = pisa::launch_route(p.sd, q, k, nodes, w.norms, w.hexp, false, w.kept, nullptr, nullptr, s);
  }
  if (e != hipSuccess) return hip_status(e, "route");
  {
    Stage sc(s, "regroup_select");
    e = pisa::launch_regroup(w.kept, p.U, p.sd.K, p.sd.N, p.n1_buckets, (int)p.BH, p.sd.chunk_log2, w.counts,
                             w.offsets, w.ranks, false, w.pairs, s);
  }
  if (e != hipSuccess) return hip_status(e, "regroup");
  const int* total = w.offsets + p.BH * p.nch * p.n1_buckets;
  {
    Stage sc(s, "leaf_lse");
    e = pisa::launch_leaf_lse(p.sd, q, k, w.kept, w.pairs, total, w.leaf_lse, s);
  }
  if (e != hipSuccess) return hip_status(e, "leaf_lse");
  {
    Stage sc(s, "finalize");
    e = pisa::launch_finalize(p.sd, w.kept, w.leaf_lse, sel, sel_lse, s);
  }
  return hip_status(e, "finalize");
}

pisa_status pisa_select_noalloc(const pisa_shape* shape, const void* q, const void* k, const float* pyr_mean,
                                int32_t* sel, float* sel_lse, void* stream) {
  Plan p;
  pisa_status st = select_plan(shape, &p);
  if (st != PISA_OK) return st;
  const size_t need = carve_select(p, nullptr, nullptr);
  if (need > kNoAllocScratchBytes)
    return fail(PISA_EUNSUPPORTED,
                "pisa_select_noalloc: this shape needs %zu bytes of scratch; the library's fixed scratch holds %zu "
                "(call pisa_select with a workspace instead)",
                need, kNoAllocScratchBytes);
  void* ws = nullptr;
  st = scratch_address(&ws);
  if (st != PISA_OK) return st;
  return pisa_select(shape, q, k, pyr_mean, sel, sel_lse, ws, kNoAllocScratchBytes, stream);
}

size_t pisa_select_noalloc_max_bytes(void) { return kNoAllocScratchBytes; }

pisa_status pisa_select_trace(const pisa_shape* shape, const void* q, const void* k, const float* pyr_mean,
                              const int64_t* units, int64_t n_units, int32_t* trace, void* ws, size_t ws_bytes,
                              void* stream) {
  Plan p;
  pisa_status st = trace_plan(shape, &p);
  if (st != PISA_OK) return st;
  if (n_units < 0) return fail(PISA_EINVAL, "n_units must be >= 0 (got %lld)", (long long)n_units);
  if (n_units > 4LL * 0x7fffffffLL) return fail(PISA_EINVAL, "n_units too large (%lld)", (long long)n_units);
  if (n_units == 0) return ok();
  PISA_CHECK_PTR(q, "q");
  PISA_CHECK_PTR(k, "k");
  PISA_CHECK_PTR(pyr_mean, "pyr_mean");
  PISA_CHECK_PTR(units, "units");
  PISA_CHECK_PTR(trace, "trace");
  st = check_ws(carve_select(p, nullptr, nullptr), ws, ws_bytes);
  if (st != PISA_OK) return st;
  SelectWs w;
  carve_select(p, ws, &w);
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = hipSuccess;
  const void* nodes = pyr_mean;
  if (p.sd.bf16) {
    e = pisa::launch_route_planes(pyr_mean, p.BH, p.sd.lv, p.sd.D, w.part_max, w.hexp, w.hilo, w.norms, s);
    if (e != hipSuccess) return hip_status(e, "route_planes");
    nodes = w.hilo;
  }
  e = pisa::launch_route_trace(p.sd, q, k, nodes, w.norms, w.hexp, (const long long*)units, (long long)n_units, trace,
                               s);
  return hip_status(e, "route (traced walk)");
}

pisa_status pisa_sparse_attn(const pisa_shape* shape, const void* q, const void* k, const void* v, const int32_t* sel,
                             void* o, float* o_lse, void* ws, size_t ws_bytes, void* stream) {
  Plan p;
  pisa_status st = plan(shape, &p);
  if (st != PISA_OK) return st;
  PISA_CHECK_PTR(q, "q");
  PISA_CHECK_PTR(k, "k");
  PISA_CHECK_PTR(v, "v");
  PISA_CHECK_PTR(sel, "sel");
  PISA_CHECK_PTR(o, "o");
  PISA_CHECK_OPT_PTR(o_lse, "o_lse");
  AttnChunks ch;
  st = attn_chunks(shape, [](const Plan& q) { return carve_attn(q, nullptr, nullptr); }, &ch);
  if (st != PISA_OK) return st;
  st = check_ws(carve_attn(ch.cp, nullptr, nullptr), ws, ws_bytes);
  if (st != PISA_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  const long long G = p.sd.G, N = p.sd.N, D = p.sd.D, K = p.sd.K;
  for (long long f = 0; f < ch.slices; f += ch.per) {
    const long long n = ch.slices - f < ch.per ? ch.slices - f : ch.per;
    Plan cp;
    st = chunk_plan(ch, n, &cp);
    if (st != PISA_OK) return st;
    const char* qc = (const char*)q + f * G * N * D * p.elem;
    const char* kc = (const char*)k + f * N * D * p.elem;
    const char* vc = (const char*)v + f * N * D * p.elem;
    const int32_t* selc = sel + f * N * K;
    char* oc = (char*)o + f * G * N * D * p.elem;
    float* lsec = o_lse ? o_lse + f * G * N : nullptr;
    AttnWs w;
    carve_attn(cp, ws, &w);
    hipError_t e;
    {
      Stage sc(s, "regroup_attn");
      e = pisa::launch_regroup(selc, cp.U, cp.sd.K, cp.sd.N, cp.sd.lv.n[0], (int)cp.BH, cp.sd.chunk_log2, w.counts,
                               w.offsets, w.ranks, true, w.pairs, s);
    }
    if (e != hipSuccess) return hip_status(e, "regroup");
    const int* total = w.offsets + cp.BH * cp.nch * cp.sd.lv.n[0];
    {
      Stage sc(s, "attn_leaf");
      e = pisa::launch_attn_leaf(cp.sd, qc, kc, vc, selc, w.pairs, total, w.part, w.part_lse, s);
    }
    if (e != hipSuccess) return hip_status(e, "attn_leaf");
    {
      Stage sc(s, "attn_merge");
      e = pisa::launch_attn_merge(cp.sd, selc, w.ranks, w.part, w.part_lse, oc, lsec, s);
    }
    if (e != hipSuccess) return hip_status(e, "attn_merge");
  }
  return ok();
}

pisa_status pisa_sparse_attn_backward(const pisa_shape* shape, const void* q, const void* k, const void* v,
                                      const int32_t* sel, const void* o, const float* o_lse, const void* d_o,
                                      void* d_q, void* d_k, void* d_v, void* ws, size_t ws_bytes, void* stream) {
  Plan p;
  pisa_status st = plan(shape, &p);
  if (st != PISA_OK) return st;
  if (!p.sd.bf16) return fail(PISA_EUNSUPPORTED, "pisa_sparse_attn_backward: bfloat16 inputs only");
  PISA_CHECK_PTR(q, "q");
  PISA_CHECK_PTR(k, "k");
  PISA_CHECK_PTR(v, "v");
  PISA_CHECK_PTR(sel, "sel");
  PISA_CHECK_PTR(o, "o");
  PISA_CHECK_PTR(o_lse, "o_lse");
  PISA_CHECK_PTR(d_o, "d_o");
  PISA_CHECK_PTR(d_q, "d_q");
  PISA_CHECK_PTR(d_k, "d_k");
  PISA_CHECK_PTR(d_v, "d_v");
  AttnChunks ch;
  st = attn_chunks(shape, [](const Plan& q) { return carve_attn_bwd(q, nullptr, nullptr); }, &ch);
  if (st != PISA_OK) return st;
  st = check_ws(carve_attn_bwd(ch.cp, nullptr, nullptr), ws, ws_bytes);
  if (st != PISA_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  const long long G = p.sd.G, N = p.sd.N, D = p.sd.D, K = p.sd.K;
  for (long long f = 0; f < ch.slices; f += ch.per) {
    const long long n = ch.slices - f < ch.per ? ch.slices - f : ch.per;
    Plan cp;
    st = chunk_plan(ch, n, &cp);
    if (st != PISA_OK) return st;
    const long long qo = f * G * N * D, ko = f * N * D;  // element offsets of the chunk's first slice
    const uint16_t* q16 = (const uint16_t*)q;
    const uint16_t* k16 = (const uint16_t*)k;
    const uint16_t* v16 = (const uint16_t*)v;
    const int32_t* selc = sel + f * N * K;
    AttnBwdWs w;
    carve_attn_bwd(cp, ws, &w);
    hipError_t e;
    {
      Stage sc(s, "regroup_attn_bwd");
      e = pisa::launch_regroup(selc, cp.U, cp.sd.K, cp.sd.N, cp.sd.lv.n[0], (int)cp.BH, cp.sd.chunk_log2, w.counts,
                               w.offsets, w.ranks, true, w.pairs, s);
    }
    if (e != hipSuccess) return hip_status(e, "regroup");
    const int* total = w.offsets + cp.BH * cp.nch * cp.sd.lv.n[0];
    {
      Stage sc(s, "attn_backward");
      e = pisa::launch_attn_backward(cp.sd, q16 + qo, k16 + ko, v16 + ko, selc, (const uint16_t*)o + qo,
                                     o_lse + f * G * N, (const uint16_t*)d_o + qo, w.pairs, total, w.ranks,
                                     w.offsets, w.dsum, w.acc, w.acc + (size_t)cp.U * cp.sd.D, w.kv_part, w.part,
                                     (uint16_t*)d_q + qo, (uint16_t*)d_k + ko, (uint16_t*)d_v + ko, s);
    }
    if (e != hipSuccess) return hip_status(e, "pisa_sparse_attn_backward");
  }
  return ok();
}

pisa_status pisa_decode_step(const pisa_shape* shape, const int32_t* host_lens, const void* q_new, const void* k_new,
                             const void* v_new, void* k_cache, void* v_cache, float* pyr_sum, float* pyr_mean, void* o,
                             int32_t* sel_out, void* ws, size_t ws_bytes, void* stream) {
  Plan p;
  pisa_status st = plan(shape, &p);
  if (st != PISA_OK) return st;
  if (!host_lens) return fail(PISA_EINVAL, "host_lens: null pointer");
  PISA_CHECK_PTR(q_new, "q_new");
  PISA_CHECK_PTR(k_new, "k_new");
  PISA_CHECK_PTR(v_new, "v_new");
  PISA_CHECK_PTR(k_cache, "k_cache");
  PISA_CHECK_PTR(v_cache, "v_cache");
  PISA_CHECK_PTR(pyr_sum, "pyr_sum");
  PISA_CHECK_PTR(pyr_mean, "pyr_mean");
  PISA_CHECK_PTR(o, "o");
  PISA_CHECK_OPT_PTR(sel_out, "sel_out");
  pisa::DecodeArgs da{};
  st = lens_arg(host_lens, p.sd.B, p.sd.Hkv, 0, p.sd.N - 1, &da.lens);
  if (st != PISA_OK) return st;
  da.B = p.sd.B;
  da.Hq = p.sd.Hq;
  da.Hkv = p.sd.Hkv;
  da.G = p.sd.G;
  da.Nmax = p.sd.N;
  da.D = p.sd.D;
  da.C = p.sd.C;
  da.K = p.sd.K;
  da.scale = p.sd.scale;
  da.bf16 = p.sd.bf16;
  da.lv = p.sd.lv;
  const size_t need = carve_decode(p, nullptr, nullptr);
  st = check_ws(need, ws, ws_bytes);
  if (st != PISA_OK) return st;
  DecodeWs w;
  carve_decode(p, ws, &w);
  da.ticket = w.ticket;
  da.part_o = w.part_o;
  da.part_lse = w.part_lse;
  hipError_t e;
  {
    Stage sc((hipStream_t)stream, "decode_step");
    e = pisa::launch_decode(da, q_new, k_new, v_new, k_cache, v_cache, pyr_sum, pyr_mean, o, sel_out,
                            (hipStream_t)stream);
  }
  return hip_status(e, "decode_step");
}

pisa_status bsa_select(const pisa_shape* shape, const void* q, const void* k, int32_t* sel, void* ws, size_t ws_bytes,
                       void* stream) {
  Plan p;
  pisa_status st = plan(shape, &p);
  if (st != PISA_OK) return st;
  PISA_CHECK_PTR(q, "q");
  PISA_CHECK_PTR(k, "k");
  PISA_CHECK_PTR(sel, "sel");
  const size_t need = carve_bsa(p, nullptr, nullptr);
  st = check_ws(need, ws, ws_bytes);
  if (st != PISA_OK) return st;
  BsaWs w;
  carve_bsa(p, ws, &w);
  hipStream_t s = (hipStream_t)stream;
  pisa::LensArg la;
  std::memset(&la, 0, sizeof la);
  la.hkv = p.sd.Hkv;
  // leaf means only: the leaf level is the whole pyramid the flat selection needs
  pisa::PyrDims pd{(int)p.BH, p.sd.N, p.sd.C, p.sd.D, p.sd.lv};
  pd.lv.n_levels = 1;
  pd.lv.nodes = p.sd.lv.n[0];
  hipError_t e;
  {
    Stage sc(s, "bsa_pool");
    e = pisa::launch_pool(k, p.sd.bf16, pd, la, 0, w.mean, nullptr, s);
    if (e == hipSuccess && p.sd.bf16) e = pisa::launch_split_hilo(w.mean, p.BH * p.sd.lv.n[0], p.sd.D, w.hilo, s);
  }
  if (e != hipSuccess) return hip_status(e, "bsa leaf pooling");
  {
    Stage sc(s, "bsa_select");
    e = pisa::launch_bsa(p.sd, q, w.mean, w.hilo, sel, s);
  }
  return hip_status(e, "bsa_select");
}

pisa_status pisa_flat_leaf_lse(const pisa_shape* shape, const void* q, const void* k, const int32_t* positions,
                               int32_t n_pos, float* leaf_lse, float* row_lse, void* stream) {
  Plan p;
  pisa_status st = plan(shape, &p);
  if (st != PISA_OK) return st;
  PISA_CHECK_PTR(q, "q");
  PISA_CHECK_PTR(k, "k");
  PISA_CHECK_PTR(positions, "positions");
  PISA_CHECK_PTR(leaf_lse, "leaf_lse");
  PISA_CHECK_PTR(row_lse, "row_lse");
  if (n_pos < 1) return fail(PISA_EINVAL, "n_pos must be >= 1");
  if ((long long)p.BH * n_pos * p.sd.lv.n[0] * p.sd.G >= (1LL << 40)) return fail(PISA_EUNSUPPORTED, "output too large");
  hipError_t e;
  {
    Stage sc((hipStream_t)stream, "flat_leaf_lse");
    e = pisa::launch_flat_leaf_lse(p.sd, q, k, positions, n_pos, leaf_lse, row_lse, (hipStream_t)stream);
  }
  return hip_status(e, "pisa_flat_leaf_lse");
}

pisa_status pisa_selection_quality(const pisa_shape* shape, const float* leaf_lse, const float* row_lse,
                                   const int32_t* positions, int32_t n_pos, const int32_t* sel, int32_t* flat_sel,
                                   float* recall, float* mass, void* stream) {
  Plan p;
  pisa_status st = plan(shape, &p);
  if (st != PISA_OK) return st;
  PISA_CHECK_PTR(leaf_lse, "leaf_lse");
  PISA_CHECK_PTR(row_lse, "row_lse");
  PISA_CHECK_PTR(positions, "positions");
  PISA_CHECK_PTR(sel, "sel");
  PISA_CHECK_PTR(flat_sel, "flat_sel");
  PISA_CHECK_PTR(recall, "recall");
  PISA_CHECK_PTR(mass, "mass");
  if (n_pos < 1) return fail(PISA_EINVAL, "n_pos must be >= 1");
  if (p.sd.lv.n[0] > 16384) return fail(PISA_EUNSUPPORTED, "at most 16384 leaves (the leaf scores of a unit are held in LDS)");
  hipError_t e;
  {
    Stage sc((hipStream_t)stream, "selection_quality");
    e = pisa::launch_quality(p.sd, leaf_lse, row_lse, positions, n_pos, sel, flat_sel, recall, mass,
                             (hipStream_t)stream);
  }
  return hip_status(e, "pisa_selection_quality");
}

pisa_status pisa_build_pyramid_pooled(const pisa_shape* shape, const void* k, int32_t pool, float* summary,
                                      float* variance, void* stream) {
  Plan p;
  pisa_status st = plan(shape, &p);
  if (st != PISA_OK) return st;
  PISA_CHECK_PTR(k, "k");
  PISA_CHECK_PTR(summary, "summary");
  PISA_CHECK_OPT_PTR(variance, "variance");
  if (pool != PISA_POOL_MEAN && pool != PISA_POOL_SUM && pool != PISA_POOL_MAX)
    return fail(PISA_EINVAL, "pool must be PISA_POOL_MEAN, PISA_POOL_SUM or PISA_POOL_MAX");
  if (variance && pool == PISA_POOL_MAX)
    return fail(PISA_EUNSUPPORTED, "variances are built with mean or sum pooling only");
  pisa::PyrDims pd{(int)p.BH, p.sd.N, p.sd.C, p.sd.D, p.sd.lv};
  hipError_t e;
  {
    Stage sc((hipStream_t)stream, "pyramid_pooled");
    e = pisa::launch_pool_pooled(k, p.sd.bf16, pd, pool, summary, variance, (hipStream_t)stream);
  }
  return hip_status(e, "pisa_build_pyramid_pooled");
}

pisa_status pisa_select_variant(const pisa_shape* shape, const pisa_variant* variant, const void* q, const void* k,
                                const float* summary, const float* variance, int32_t* sel, void* stream) {
  Plan p;
  pisa_status st = plan(shape, &p);
  if (st != PISA_OK) return st;
  if (!variant) return fail(PISA_EINVAL, "variant: null pointer");
  PISA_CHECK_PTR(q, "q");
  PISA_CHECK_PTR(k, "k");
  PISA_CHECK_PTR(summary, "summary");
  PISA_CHECK_OPT_PTR(variance, "variance");
  PISA_CHECK_PTR(sel, "sel");
  const int score = variant->score, budget = variant->budget;
  if (score != PISA_SCORE_LSE && score != PISA_SCORE_MEAN && score != PISA_SCORE_MEAN_VAR)
    return fail(PISA_EINVAL, "variant.score must be PISA_SCORE_LSE, PISA_SCORE_MEAN or PISA_SCORE_MEAN_VAR");
  if (budget != PISA_BUDGET_FIXED && budget != PISA_BUDGET_HALVING)
    return fail(PISA_EINVAL, "variant.budget must be PISA_BUDGET_FIXED or PISA_BUDGET_HALVING");
  if (score == PISA_SCORE_MEAN_VAR && !variance) return fail(PISA_EINVAL, "mean + variance scoring needs variance");
  if (variant->max_level < -1) return fail(PISA_EINVAL, "variant.max_level must be -1 (none) or >= 0");
  const pisa::Levels& lv = p.sd.lv;
  const int root = lv.n_levels - 1;
  const int start = variant->max_level < 0 || variant->max_level > root ? root : variant->max_level;
  // candidate lists held in LDS: every node of the starting level, then twice the kept nodes of the
  // level above
  auto kept_max = [&](int l) -> long long {
    const long long Kl = budget == PISA_BUDGET_FIXED ? p.sd.K : std::min((long long)lv.n[l], (long long)p.sd.K << l);
    return std::min((long long)lv.n[l], Kl);
  };
  if (lv.n[start] > pisa::kVariantLdsCand)
    return fail(PISA_EUNSUPPORTED, "the starting level has %d nodes; at most %d candidates per level", lv.n[start],
                pisa::kVariantLdsCand);
  for (int l = start; l >= 1; --l)
    if (2 * kept_max(l) > pisa::kVariantLdsCand)
      return fail(PISA_EUNSUPPORTED, "level %d would have %lld candidates; at most %d per level", l - 1,
                  2 * kept_max(l), pisa::kVariantLdsCand);
  hipError_t e;
  {
    Stage sc((hipStream_t)stream, "select_variant");
    e = pisa::launch_variant(p.sd, score, budget, start, q, k, summary, variance, sel, (hipStream_t)stream);
  }
  return hip_status(e, "pisa_select_variant");
}

pisa_status pisa_stage_timing(int32_t enable) {
  g_timer.on = enable != 0;
  if (!enable) {
    for (auto& e : g_timer.pending) {
      (void)hipEventSynchronize(e.b);  // only so that the events can be reused; their times are dropped
      g_timer.pool.push_back(e.a);
      g_timer.pool.push_back(e.b);
    }
    g_timer.pending.clear();
    g_timer.totals.clear();
  }
  return ok();
}

int32_t pisa_stage_times(char (*names)[32], double* total_ms, int32_t* count, int32_t cap) {
  if (cap < 0) return fail(PISA_EINVAL, "cap must be >= 0");
  for (auto& e : g_timer.pending) {
    if (hipEventSynchronize(e.b) != hipSuccess) return fail(PISA_EHIP, "hipEventSynchronize failed");
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, e.a, e.b) != hipSuccess) return fail(PISA_EHIP, "hipEventElapsedTime failed");
    auto& t = g_timer.totals[e.name];
    t.first += ms;
    t.second += 1;
    g_timer.pool.push_back(e.a);
    g_timer.pool.push_back(e.b);
  }
  g_timer.pending.clear();
  int32_t n = 0;
  for (auto& kv : g_timer.totals) {
    if (n < cap) {
      if (names) {
        std::strncpy(names[n], kv.first.c_str(), 31);
        names[n][31] = 0;
      }
      if (total_ms) total_ms[n] = kv.second.first;
      if (count) count[n] = kv.second.second;
    }
    ++n;
  }
  return n;
}

}  // extern "C"
